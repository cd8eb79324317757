"""Pins of the oracle's static per-head KLT key basis (CPU only).

* the key rotation's fixed order (a chain of fp32 fused multiply-adds) against an
  exact-rational emulation of the same sequence of roundings (tests/_brute.py), and the fused
  multiply-add itself against exact rationals;
* a closed form: calibration windows built from the columns of the Sylvester Hadamard matrix,
  scaled by distinct factors and shifted by a common mean, have the normalised Hadamard
  columns as eigenvectors (the mean drops out of the centred covariance), with eigenvalues
  the squared factors; order, signs and the excluded position 0 follow;
* a diagonal covariance gives a permutation basis, and the rotation is then an exact
  permutation of the key row;
* the rotated keys and queries keep every score up to fp32 rounding, with and without the
  smoothing, and g_K is taken over the rotated keys.

Source: [cache post] = rstation.ai post "NVFP4 attention cache on W4A4 Qwen3-8B: static key
smoothing is near-lossless, key rotations hurt", cache-config table rows "K: static per-head
KLT" and "K: static KLT + smoothing".
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import nvfp4_oracle as O
from tests import _brute


def _two_roundings(y, B):
    """The same sums with the product and the addition rounded separately (what a chain
    without fused multiply-adds gives), for the check that the pin tells the two apart."""
    acc = np.zeros(y.shape, dtype=np.float32)
    for j in range(128):
        acc = (acc + (B[:, j, :] * y[..., :, j:j + 1]).astype(np.float32)).astype(np.float32)
    return acc


def test_rotation_order_vs_exact_rationals():
    """Each output is the chain z <- fl32(B[j][i] * y_j + z) over j = 0..127 from z = 0: exact
    rational products and sums with one rounding per step."""
    rng = np.random.default_rng(71)
    y = (rng.standard_normal((2, 1, 128)) * np.exp(rng.uniform(-4, 4, (2, 1, 128)))).astype(np.float32)
    B = (rng.standard_normal((1, 128, 128)) / np.sqrt(128)).astype(np.float32)
    got = O.rotate_fp32(y, B)
    for n in range(2):
        for i in range(0, 128, 3):
            acc = Fraction(0)
            for j in range(128):
                acc = Fraction(float(_brute.fraction_to_f32(Fraction(float(B[0, j, i])) * Fraction(float(y[n, 0, j]))
                                                            + acc)))
            assert np.float32(float(acc)) == got[n, 0, i], (n, i)
    assert not np.array_equal(_two_roundings(y, B), got)           # the pin separates the orders


def test_fused_multiply_add_against_exact_rationals():
    """fma_f32 against exact rational arithmetic, over random magnitudes and near-cancelling
    sums (where the fp64 sum is inexact and its rounding direction matters)."""
    rng = np.random.default_rng(73)
    a = (rng.standard_normal(400) * np.exp(rng.uniform(-20, 20, 400))).astype(np.float32)
    b = (rng.standard_normal(400) * np.exp(rng.uniform(-20, 20, 400))).astype(np.float32)
    c = (rng.standard_normal(400) * np.exp(rng.uniform(-20, 20, 400))).astype(np.float32)
    c[:200] = (-(a[:200].astype(np.float64) * b[:200]) * (1 + rng.uniform(-1e-6, 1e-6, 200))).astype(np.float32)
    got = O.fma_f32(a, b, c)
    for k in range(400):
        want = _brute.fraction_to_f32(Fraction(float(a[k])) * Fraction(float(b[k])) + Fraction(float(c[k])))
        assert got[k] == want, (k, a[k], b[k], c[k], got[k], want)


def hadamard_windows(mu, scale):
    """Two windows of 129 positions: position 0 is junk (excluded), then x_k + mu in the
    first window and -x_k + mu in the second, x_k = scale * (1 + k/128) * H[:, k]."""
    H = O.sylvester_hadamard(128).astype(np.float64)
    f = scale * (1.0 + np.arange(128) / 128.0)
    X = (H * f[None, :]).T                          # row k = x_k
    win = np.zeros((2, 129, 128))
    win[:, 0] = 1000.0
    win[0, 1:] = X + mu
    win[1, 1:] = -X + mu
    return win, f


def test_klt_basis_closed_form_hadamard_columns():
    rng = np.random.default_rng(5)
    mu = np.round(rng.standard_normal(128) * 4) / 4                 # exact in bf16
    w0, f0 = hadamard_windows(mu, 1.0)
    w1, f1 = hadamard_windows(-mu, 0.5)
    kw = np.stack([w0, w1], axis=2)                                  # [2][129][Hkv=2][128]
    assert np.array_equal(kw.astype(np.float32).astype(np.float64), kw)
    B, lam = O.klt_basis(kw, None, O.FLAG_KLT, exclude_pos0=True)
    H = O.sylvester_hadamard(128).astype(np.float64) / np.sqrt(128.0)
    for h, f in ((0, f0), (1, f1)):
        # covariance = (1/128) sum_k f_k^2 H_k H_k^T: eigenvalue f_k^2 on H_k / sqrt(128)
        assert np.allclose(lam[h], (f ** 2)[::-1], rtol=1e-12, atol=0)
        want = H[:, ::-1]                     # decreasing eigenvalue: k = 127 first; H[0, k] = +1
        assert np.max(np.abs(B[h].astype(np.float64) - want)) <= 1e-7
        assert np.all(B[h][0] > 0)            # equal magnitudes: the first entry is positive
    # position 0 (junk) included: the basis changes
    B2, _ = O.klt_basis(kw, None, O.FLAG_KLT, exclude_pos0=False)
    assert np.max(np.abs(B2 - B)) > 1e-3


def test_diagonal_covariance_gives_an_exact_permutation():
    a = np.array([(1.0 + ((37 * j) % 128) / 128.0) for j in range(128)])   # distinct spreads
    rows = np.zeros((2, 129, 1, 128))
    for j in range(128):
        rows[0, 1 + j, 0, j] = a[j]
        rows[1, 1 + j, 0, j] = -a[j]
    B, lam = O.klt_basis(rows, None, O.FLAG_KLT)
    perm = np.argsort(-a, kind="stable")
    P = np.zeros((128, 128), np.float32)
    P[perm, np.arange(128)] = 1.0
    assert np.array_equal(B[0], P)
    rng = np.random.default_rng(3)
    y = rng.standard_normal((5, 1, 128)).astype(np.float32)
    assert np.array_equal(O.rotate_fp32(y, B), y[..., perm])


@pytest.mark.parametrize("flags", [O.FLAG_KLT, O.FLAG_KLT | O.FLAG_SMOOTH])
def test_klt_keeps_scores_and_g_is_over_rotated_keys(flags):
    rng = np.random.default_rng(9)
    scale = np.exp(rng.uniform(-1, 2, 128))
    kw = (rng.standard_normal((3, 40, 2, 128)) * scale).astype(np.float32)
    kw = kw.astype(np.float64)
    s, r, g = O.calibrate(kw, None, True, flags)
    B, _ = O.klt_basis(kw, r, flags)
    for h in range(2):
        assert np.max(np.abs(B[h].astype(np.float64).T @ B[h].astype(np.float64) - np.eye(128))) < 1e-6
    x = (rng.standard_normal((7, 2, 128)) * scale).astype(np.float32)
    q = rng.standard_normal((7, 2, 128))
    z = O.key_transform(x, r, flags, B).astype(np.float64)
    qp = O.query_transform(q, s if flags & O.FLAG_SMOOTH else None, flags, B)
    ref = np.einsum("nhd,nhd->nh", q, x.astype(np.float64))
    got = np.einsum("nhd,nhd->nh", qp, z)
    norm = np.linalg.norm(q, axis=-1) * np.linalg.norm(x.astype(np.float64), axis=-1)
    assert np.max(np.abs(got - ref) / norm) < 2e-6
    yall = O.key_transform(kw.astype(np.float32), r[None, None] if r is not None else None, flags, B)
    assert g[0] == np.float32(np.float64(np.float32(np.abs(yall.astype(np.float64)).max())) / 2688.0)


def test_hadamard_and_klt_exclude_each_other():
    with pytest.raises(ValueError):
        O.key_transform(np.zeros((1, 1, 128), np.float32), None, O.FLAG_KLT | O.FLAG_HADAMARD,
                        np.zeros((1, 128, 128), np.float32))
