"""Pins of the oracle's transforms, calibration, attention and sizes (CPU only).

* Hadamard-128: integer identities (H H^T = 128 I, symmetry), the fp32 butterfly on unit
  vectors equals the dense matrix columns exactly, and it stays within the fp32 error bound
  of the dense fp64 product ([cache post] Hadamard-128 rows; an orthogonal basis change).
* SmoothAttention invariance: with the oracle's key and query transforms, q'.y equals q.k
  up to the rounding of r = fl32(1/s) and of the fp32 key multiply ([cache post] smoothing
  row, [QServe rec] SmoothAttention field).
* calibration: position 0 is excluded from the absmax, s is the correctly rounded fp32
  square root (checked with exact rationals), g = amax/2688 over transformed keys.
* attention: torch's scaled_dot_product_attention in fp64 as a library reference, and the
  special cases n = 1, zero query, identical keys, empty sequence.
* causal attention: torch's scaled_dot_product_attention in fp64 with an explicit
  position-offset causal mask, and closed forms: position 0 returns v_0; identical keys give
  the running mean of V; rows before the sequence start are zero.
* sizes printed on the pages (tests/golden/page_facts.json).
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import nvfp4_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_hadamard_integer_identities():
    H = O.sylvester_hadamard(128)
    assert H.shape == (128, 128)
    assert np.array_equal(H, H.T)
    assert np.array_equal(H @ H.T, 128 * np.eye(128, dtype=np.int64))
    x = np.random.default_rng(0).integers(-50, 50, 128)
    assert np.array_equal(H @ (H @ x), 128 * x)
    # entry formula: (-1)^popcount(i & j)
    i, j = np.meshgrid(np.arange(128), np.arange(128), indexing="ij")
    pc = np.vectorize(lambda v: bin(v).count("1"))(i & j)
    assert np.array_equal(H, np.where(pc % 2 == 0, 1, -1))


def test_butterfly_unit_vectors_equal_dense_columns():
    E = np.eye(128, dtype=np.float32)
    Y = O.hadamard_butterfly_fp32(E)          # row j = H e_j = column j of H
    assert np.array_equal(Y, O.sylvester_hadamard(128).T.astype(np.float32))


def test_butterfly_within_fp32_bound_of_dense_fp64():
    rng = np.random.default_rng(1)
    X = (rng.standard_normal((64, 128)) * np.exp(rng.uniform(-2, 2, (64, 128)))).astype(np.float32)
    Y = O.hadamard_butterfly_fp32(X).astype(np.float64)
    ref = X.astype(np.float64) @ O.sylvester_hadamard(128).T.astype(np.float64)
    # 7 stages of fp32 additions: |err| <= 7 * 2^-24 * (|H| |x|) per entry (first order)
    bound = 7 * 2.0 ** -24 * (np.abs(X.astype(np.float64)) @ np.ones((128, 128))) * 1.01
    assert np.all(np.abs(Y - ref) <= bound)
    # the butterfly must not be a no-op or a transposed variant on non-trivial data
    assert np.max(np.abs(Y - X)) > 1.0


def test_smoothing_preserves_scores_up_to_rounding():
    rng = np.random.default_rng(2)
    hkv = 2
    k = (rng.standard_normal((10, hkv, 128)) * np.exp(rng.uniform(-2, 4, (1, hkv, 128)))).astype(np.float32)
    q = rng.standard_normal((hkv, 128)).astype(np.float32)
    a = np.abs(k).max(axis=0)
    s = np.sqrt(a.astype(np.float64)).astype(np.float32)
    r = (np.float32(1) / s).astype(np.float32)
    for flags in (O.FLAG_SMOOTH, O.FLAG_SMOOTH | O.FLAG_HADAMARD, O.FLAG_HADAMARD):
        y = O.key_transform(k, r[None], flags).astype(np.float64)
        qp = O.query_transform(q, s, flags)
        got = np.einsum("thd,hd->th", y, qp)
        ref = np.einsum("thd,hd->th", k.astype(np.float64), q.astype(np.float64))
        mag = np.einsum("thd,hd->th", np.abs(k.astype(np.float64)), np.abs(q.astype(np.float64)))
        rel = 2.0 ** -22 if flags & O.FLAG_SMOOTH else 0
        rel += 8 * 2.0 ** -24 * np.sqrt(128) if flags & O.FLAG_HADAMARD else 0
        assert np.all(np.abs(got - ref) <= rel * mag * 4 + 1e-12), flags
    # exact-arithmetic identity of the transform pair: (q*s).(k/s) == q.k
    qs = [Fraction(float(v)) for v in q[0, :8]]
    ks = [Fraction(float(v)) for v in k[0, 0, :8]]
    ss = [Fraction(float(v)) for v in s[0, :8]]
    assert sum(a_ * b_ for a_, b_ in zip(qs, ks)) == sum((a_ * c_) * (b_ / c_) for a_, b_, c_ in zip(qs, ks, ss))


def _sqrt_correctly_rounded_f32(a: float, s: np.float32) -> bool:
    """s is the fp32 nearest to sqrt(a): (s - ulp/2)^2 <= a <= (s + ulp/2)^2, exactly."""
    lo = Fraction(float(s)) + (Fraction(float(np.nextafter(s, np.float32(0)))) - Fraction(float(s))) / 2
    hi = Fraction(float(s)) + (Fraction(float(np.nextafter(s, np.float32(np.inf)))) - Fraction(float(s))) / 2
    A = Fraction(float(a))
    return lo * lo <= A <= hi * hi


def test_calibrate_excludes_position0_and_rounds_exactly():
    rng = np.random.default_rng(3)
    W, T, hkv = 4, 9, 2
    k = rng.standard_normal((W, T, hkv, 128)).astype(np.float32)
    v = rng.standard_normal((W, T, hkv, 128)).astype(np.float32)
    k[:, 0] *= 40                                    # sinks at position 0 of every window
    k[2, 5, 1, 7] = 123.0                            # a genuine outlier after position 0
    s, r, g = O.calibrate(k, v, exclude_pos0=True, k_flags=O.FLAG_SMOOTH)
    a_ref = np.abs(k[:, 1:]).max(axis=(0, 1))
    assert s[1, 7] == np.float32(np.sqrt(123.0))
    for h in range(hkv):
        for j in range(0, 128, 9):
            assert _sqrt_correctly_rounded_f32(a_ref[h, j], s[h, j])
            # r is the fp32 nearest to 1/s
            rr = Fraction(float(r[h, j]))
            exact = 1 / Fraction(float(s[h, j]))
            for nb in (np.nextafter(r[h, j], np.float32(0)), np.nextafter(r[h, j], np.float32(9))):
                assert abs(rr - exact) <= abs(Fraction(float(nb)) - exact)
    s2, _, _ = O.calibrate(k, v, exclude_pos0=False, k_flags=O.FLAG_SMOOTH)
    assert np.all(s2 >= s) and np.any(s2 > s)       # including the sink raises the absmax
    # g_K is amax of the transformed keys INCLUDING position 0, over 2688
    y = O.key_transform(k, r[None, None], O.FLAG_SMOOTH)
    assert Fraction(float(g[0])) == Fraction(float(np.float32(np.abs(y).max() / np.float64(2688))))
    assert g[1] == np.float32(np.abs(v.astype(np.float64)).max() / 2688.0)
    # a zero channel gives s = 1; all-zero values give g = 1
    k0 = k.copy()
    k0[:, :, 0, 3] = 0
    s0, r0, g0 = O.calibrate(k0, np.zeros_like(v))
    assert s0[0, 3] == 1.0 and r0[0, 3] == 1.0 and g0[1] == 1.0


def test_attention_matches_torch_sdpa_fp64():
    rng = np.random.default_rng(4)
    B, Hq, Hkv, n = 3, 8, 2, 37
    qp = rng.standard_normal((B, Hq, 128))
    K = [rng.standard_normal((n + 5, Hkv, 128)) for _ in range(B)]
    V = [rng.standard_normal((n + 5, Hkv, 128)) for _ in range(B)]
    seq = [n, 1, 17]
    out = O.attention(qp, K, V, seq, 0.125)
    for b in range(B):
        kk = torch.from_numpy(K[b][:seq[b]]).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
        vv = torch.from_numpy(V[b][:seq[b]]).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
        qq = torch.from_numpy(qp[b])[:, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, scale=0.125)[:, 0]
        assert np.allclose(out[b], ref.numpy(), rtol=1e-12, atol=1e-12)


def test_attention_special_cases():
    rng = np.random.default_rng(5)
    V = [rng.standard_normal((6, 1, 128))]
    K = [rng.standard_normal((6, 1, 128))]
    q = rng.standard_normal((1, 4, 128))
    assert np.allclose(O.attention(q, K, V, [1], 0.1)[0], V[0][0, 0])            # n = 1
    assert np.allclose(O.attention(np.zeros_like(q), K, V, [6], 0.1)[0],
                       V[0][:, 0].mean(0))                                          # q = 0
    Ksame = [np.repeat(K[0][:1], 6, axis=0)]
    assert np.allclose(O.attention(q, Ksame, V, [6], 0.1)[0], V[0][:, 0].mean(0))  # same keys
    assert np.all(O.attention(q, K, V, [0], 0.1) == 0)                               # empty


def _sdpa_causal_ref(qp, K, V, n, Hq):
    """Library reference: torch SDPA in fp64, GQA by repeating KV heads, boolean mask with
    query i at position n - Tq + i seeing keys 0..n-Tq+i."""
    Tq = qp.shape[0]
    Hkv = K.shape[1]
    kk = torch.from_numpy(K[:n]).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)     # [Hq][n][D]
    vv = torch.from_numpy(V[:n]).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
    qq = torch.from_numpy(qp).permute(1, 0, 2)                                           # [Hq][Tq][D]
    pos = n - Tq + np.arange(Tq)
    mask = torch.from_numpy(np.arange(n)[None, :] <= pos[:, None])                       # [Tq][n]
    return qq, kk, vv, mask, pos


def test_causal_attention_matches_torch_sdpa_fp64():
    rng = np.random.default_rng(14)
    B, Tq, Hq, Hkv = 3, 9, 8, 2
    seq = [23, 9, 40]
    qp = rng.standard_normal((B, Tq, Hq, 128))
    K = [rng.standard_normal((n + 3, Hkv, 128)) for n in seq]
    V = [rng.standard_normal((n + 3, Hkv, 128)) for n in seq]
    out = O.causal_attention(qp, K, V, seq, 0.11)
    for b, n in enumerate(seq):
        qq, kk, vv, mask, pos = _sdpa_causal_ref(qp[b], K[b], V[b], n, Hq)
        ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask, scale=0.11)
        assert np.allclose(out[b], ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


def test_causal_attention_special_cases():
    rng = np.random.default_rng(15)
    n, Tq = 12, 12
    K = [rng.standard_normal((n, 1, 128))]
    V = [rng.standard_normal((n, 1, 128))]
    q = rng.standard_normal((1, Tq, 4, 128))
    out = O.causal_attention(q, K, V, [n], 0.2)
    # full window: position 0 sees only itself
    assert np.allclose(out[0, 0], np.broadcast_to(V[0][0, 0], (4, 128)), rtol=0, atol=1e-15)
    # identical keys: uniform weights, so row i is the running mean of v_0..v_i
    Ksame = [np.repeat(K[0][:1], n, axis=0)]
    run_mean = np.cumsum(V[0][:, 0], axis=0) / np.arange(1, n + 1)[:, None]
    out_same = O.causal_attention(q, Ksame, V, [n], 0.2)
    for hq in range(4):
        assert np.allclose(out_same[0, :, hq], run_mean, rtol=1e-12, atol=1e-12)
    # more queries than cached tokens: the first Tq - n rows come before the sequence start
    q2 = rng.standard_normal((1, 5, 4, 128))
    out2 = O.causal_attention(q2, K, V, [3], 0.2)
    assert np.all(out2[0, :2] == 0)
    assert np.allclose(out2[0, 2], np.broadcast_to(V[0][0, 0], (4, 128)), rtol=0, atol=1e-15)
    # two keys: the weight of key 1 is the logistic function of the score difference
    e0, e1 = 0.2 * (K[0][0, 0] @ q[0, 1, 0]), 0.2 * (K[0][1, 0] @ q[0, 1, 0])
    w1 = 1.0 / (1.0 + np.exp(e0 - e1))
    assert np.allclose(out[0, 1, 0], (1 - w1) * V[0][0, 0] + w1 * V[0][1, 0], rtol=1e-12, atol=1e-12)


def test_sizes_printed_on_the_pages():
    with open(os.path.join(GOLDEN, "page_facts.json")) as f:
        facts = json.load(f)
    sh = facts["bf16_cache_bytes_per_token"]["shape"]
    per_tok = O.cache_bytes_per_token("bf16", "bf16", sh["kv_heads"], sh["layers"], sh["head_dim"])
    assert per_tok == facts["bf16_cache_bytes_per_token"]["value"] == 144 * 1024
    e = facts["bf16_cache_bytes_batch4_ctx2300"]
    total = per_tok * e["batch"] * e["context_tokens"]
    assert total == 1358954496 and abs(total / e["value_approx"] - 1) < 0.05
    assert O.bits_per_value("nvfp4") == facts["nvfp4_bits_per_value"]["value"]
    assert O.cache_bytes_per_token("nvfp4", "nvfp4", 8, 36) == 41472
    assert O.row_bytes("nvfp4") == 72 and O.row_bytes("bf16") == 256
    assert O.BLOCK == facts["block_size"]["value"]
    assert O.E2M1_MAX == facts["fp4_max_value"]["value"]
