"""Pins of the oracle's MSE-searched key block scale (CPU only).

The oracle ranks candidates with an algebraic rewrite of the squared error that it evaluates
exactly in fp64; the pins below recompute the squared error from its definition,
sum_j (y_j - y_hat_j)^2, in exact rational arithmetic with brute-force nearest-point
encoding (tests/_brute.py), and search the candidate set by enumeration:

* random blocks of several shapes (Gaussian, heavy-tailed, one outlier, clustered values,
  near-underflow and saturating blocks): the chosen code and the packed nibbles;
* a worked example derived by hand in the docstring, which includes an exact tie;
* special cases: an all-zero block, a block beyond the largest scale, a block whose
  absmax-to-6 scale underflows to zero while a searched scale keeps it;
* the searched error is never above the absmax-to-6 error (the absmax code is a candidate);
* the candidate codes form one run of consecutive codes between S0 - 2 and S0 + 15
  (S0 = the absmax-to-6 code) with at most 17 members, the window the kernel scans.

Sources: [OSFP4] = paperlayer.ai summary of arXiv 2610.08231v1 (section 1: absmax-to-6
flushes entries 24x below the block maximum; section 2.1 and appendix A: the smoothed FP4
error is flat between 7/4 and 7; section 3 and appendix C: a deterministic search over valid
E4M3 scales per block; appendix H: MSE-optimal E4M3 scales).
"""
from fractions import Fraction

import numpy as np

from oracle import nvfp4_oracle as O
from tests import _brute

E4M3 = _brute.e4m3_nonneg_table()


def _frac(x) -> Fraction:
    return Fraction(float(x))


def brute_sse(block, sigma: Fraction, g: Fraction) -> Fraction:
    """Exact squared error of a block quantised with scale sigma (zero scale: all codes 0)."""
    vals = dict(_brute.e2m1_codes_table())
    err = Fraction(0)
    for x in block:
        xf = _frac(x)
        yh = Fraction(0) if sigma == 0 else vals[_brute.e2m1_encode_brute(xf, sigma * g)] * sigma * g
        err += (xf - yh) ** 2
    return err


def brute_mse_code(block, g: float):
    """(chosen code, its exact error, absmax-to-6 code, its exact error) by enumeration."""
    gf = _frac(np.float32(g))
    A = max(abs(_frac(x)) for x in block)
    s0 = _brute.nearest_code(A / (6 * gf), E4M3)
    best, best_e = s0, brute_sse(block, E4M3[s0][1], gf)
    e0 = best_e
    for c, v in E4M3[1:]:
        if c == s0 or not (Fraction(7, 4) * v * gf <= A <= 7 * v * gf):
            continue
        e = brute_sse(block, v, gf)
        if e < best_e:
            best, best_e = c, e
    return best, best_e, s0, e0


def brute_nibbles(block, code: int, g: float):
    gf = _frac(np.float32(g))
    sigma = E4M3[code][1]
    if sigma == 0:
        return [0] * len(block)
    return [_brute.e2m1_encode_brute(_frac(x), sigma * gf) for x in block]


def _rows_from_blocks(blocks):
    """Pad a list of 16-element blocks to whole 128-element rows (zero blocks fill)."""
    flat = np.zeros((((len(blocks) + 7) // 8) * 8, 16), dtype=np.float32)
    for i, b in enumerate(blocks):
        flat[i] = b
    return flat.reshape(-1, 128)


def _block_zoo(rng, n_each=12):
    out = []
    for _ in range(n_each):
        out.append(rng.standard_normal(16))
        out.append(rng.standard_t(2, 16))
        b = rng.standard_normal(16) * 0.05
        b[rng.integers(16)] = 3.0 * rng.choice([-1, 1])
        out.append(b)                                              # one outlier
        out.append(rng.choice([-1, 1], 16) * (2.5 + 0.3 * rng.random(16)))   # clustered
        out.append(rng.standard_normal(16) * 10.0 ** rng.uniform(-5, -3.3))  # near underflow
        out.append(rng.standard_normal(16) * 10.0 ** rng.uniform(2.9, 3.6))  # near / past 448
    return [np.asarray(b, np.float32) for b in out]


def test_mse_scale_vs_fraction_brute_force_random_blocks():
    rng = np.random.default_rng(41)
    blocks = _block_zoo(rng)
    g = np.float32(1.0 / 6.0)
    y = _rows_from_blocks(blocks)
    codes, scales = O.quantize_rows_mse(y, g)
    nib = O.unpack_nibbles(codes).reshape(-1, 16)
    sc = scales.reshape(-1)
    n_changed = 0
    for i, b in enumerate(blocks):
        want, e, s0, e0 = brute_mse_code(b, g)
        assert int(sc[i]) == want, (i, int(sc[i]), want, s0)
        assert list(nib[i]) == brute_nibbles(b, want, g), i
        assert e <= e0
        n_changed += want != s0
    assert n_changed > len(blocks) // 4      # the search moves a good share of the blocks


def test_mse_scale_random_tensor_scales():
    """Several tensor scales g (not powers of two) on Gaussian rows."""
    rng = np.random.default_rng(42)
    for g in (np.float32(0.0123), np.float32(3.7e-4), np.float32(2.9)):
        blocks = [np.asarray(rng.standard_normal(16) * float(g) * 40 * rng.uniform(0.02, 1.2), np.float32)
                  for _ in range(24)]
        sc = O.mse_scale_codes(_rows_from_blocks(blocks), g).reshape(-1)
        for i, b in enumerate(blocks):
            assert int(sc[i]) == brute_mse_code(b, g)[0], (g, i)


def test_mse_worked_example_with_tie():
    """Block (6, 5, 5, ..., 5) with g = 1.

    absmax-to-6: sigma = 1; 5 is the midpoint of 4 and 6 and goes to the even code (4), so
    the error is 15 * 1^2 = 15.  sigma = 13/8 (code 0x3D, A/sigma = 48/13, inside [7/4, 7]):
    5 -> 40/13 ~ 3.08 -> 3 -> 39/8 (error 1/8), 6 -> 48/13 ~ 3.69 -> 4 -> 13/2 (error 1/2):
    15/64 + 16/64 = 31/64.  sigma = 13/4 (code 0x45) gives the same two codes' values, 5 ->
    20/13 -> 3/2 -> 39/8 and 6 -> 24/13 -> 2 -> 13/2, hence the same error 31/64: an exact
    tie, which goes to the smaller code.  No other candidate does better (checked by
    enumeration below)."""
    y = np.zeros((1, 128), np.float32)
    y[0, :16] = 5.0
    y[0, 0] = 6.0
    sc = O.mse_scale_codes(y, 1.0)[0]
    assert int(O.absmax_scale_codes(np.array([6.0]), 1.0)[0]) == 0x38
    assert int(sc[0]) == 0x3D and O.E4M3_GRID[0x3D] == 1.625 and O.E4M3_GRID[0x45] == 3.25
    assert np.all(sc[1:] == 0)
    blk = y[0, :16]
    assert brute_sse(blk, Fraction(13, 8), Fraction(1)) == Fraction(31, 64)
    assert brute_sse(blk, Fraction(13, 4), Fraction(1)) == Fraction(31, 64)
    assert brute_sse(blk, Fraction(1), Fraction(1)) == 15
    code, e, s0, e0 = brute_mse_code(blk, 1.0)
    assert (code, e, s0, e0) == (0x3D, Fraction(31, 64), 0x38, 15)
    codes, _ = O.quantize_rows_mse(y, 1.0)
    nib = O.unpack_nibbles(codes)[0, :16]
    assert list(nib) == [6] + [5] * 15          # magnitudes 4 and 3 (codes 6 and 5)


def test_mse_special_cases():
    g = np.float32(1.0)
    # all-zero block: code 0, zero nibbles
    y = np.zeros((1, 128), np.float32)
    codes, sc = O.quantize_rows_mse(y, g)
    assert np.all(codes == 0) and np.all(sc == 0)
    # beyond the largest scale: only the saturated absmax code qualifies
    y[0, :16] = 7.0 * 448.0 * 1.01
    assert int(O.mse_scale_codes(y, g)[0, 0]) == 126 == int(O.absmax_scale_codes(np.array([y[0, 0]]), 1.0)[0])
    # absmax-to-6 underflows (A/6 below half of 2^-9) but 2^-9 puts A at 2.5 units
    y[0, :16] = 2.5 * 2.0 ** -9
    assert int(O.absmax_scale_codes(np.array([float(y[0, 0])]), 1.0)[0]) == 0
    codes, sc = O.quantize_rows_mse(y, g)
    assert int(sc[0, 0]) == 1
    assert list(O.unpack_nibbles(codes)[0, :16]) == [4] * 16      # 2.5 -> 2 (tie to even)
    # the absmax-to-6 code is outside the interval (A = 7.5 sigma_1) and still the best:
    # (7.5, 0.5 x 15) * 2^-9 costs 1.5^2 with sigma = 2^-9 (7.5 clips to 6, 0.5 is exact)
    # against 0.5^2 + 15 * 0.5^2 with the first in-interval code 2 (0.25 ties down to 0)
    y[0, :16] = 0.5 * 2.0 ** -9
    y[0, 0] = 7.5 * 2.0 ** -9
    assert int(O.absmax_scale_codes(np.array([float(y[0, 0])]), 1.0)[0]) == 1
    assert not O.mse_candidate_mask(np.array([float(y[0, 0])]), 1.0, 1)[0]
    assert brute_mse_code(y[0, :16], 1.0)[:2] == (1, Fraction(9, 4) * Fraction(1, 2 ** 18))
    assert int(O.mse_scale_codes(y, g)[0, 0]) == 1


def test_mse_candidates_are_one_run_near_the_absmax_code():
    xs = np.concatenate([np.exp(np.linspace(np.log(2.0 ** -12), np.log(600.0), 400_000)),
                         O.E4M3_GRID[1:] * 6 / 1.75, O.E4M3_GRID[1:] * 6 / 7, O.E4M3_GRID[1:]])
    A = (6 * xs).astype(np.float32).astype(np.float64)
    s0 = O.absmax_scale_codes(A, 1.0)
    mask = np.stack([O.mse_candidate_mask(A, 1.0, c) for c in range(1, 127)], axis=1)
    cnt = mask.sum(axis=1)
    has = cnt > 0
    first = np.argmax(mask, axis=1) + 1
    last = 126 - np.argmax(mask[:, ::-1], axis=1)
    assert np.all((last - first + 1)[has] == cnt[has])            # one run of codes
    assert cnt.max() <= 17
    assert (first - s0)[has].min() >= -2 and (last - s0)[has].max() <= 15
    # every block of nonzero maximum up to 7 * 448 g has a candidate
    assert np.all(has[(A > 2.0 ** -9 * 1.75) & (A <= 7 * 448)])
