"""GPU parity of the causal multi-query attention (prefill_attention_nvfp4) against the
oracle's causal_attention over the same quantised cache.

Bar (as for decode): max |err| <= 1e-3 * max|V_hat| over the layer and per-row (sequence,
query position, query head) relative L2 <= 1e-4 against the fp64 oracle; rows whose position
falls before the sequence start are exactly zero.

Cases: the tiny reference as a full teacher-forced window (Tq = T = 256) and a Qwen3-8B layer
(B = 4, T = 2304) with a 40-position block; every key-transform combination and MSE-searched
key scales, contiguous and paged caches; ragged lengths (0, shorter than the block, page and tile boundaries, a block
size that is not a multiple of the 8-position tile); BF16 keys; a full 2304-position window
checked on sampled rows; agreement of the last row with the decode kernel.
"""
import numpy as np
import pytest
import torch

from oracle import nvfp4_oracle as O
from synth import kv_inputs as S
from tests import _pipeline as P
from tests.test_gpu_parity import FLAG_SETS, MSE, gpu_calibrate, gpu_decode, gpu_fill_cache, oracle_layer

pytestmark = pytest.mark.gpu

ATOL_FRAC = 1e-3
REL_L2 = 1e-4


def oracle_inputs(qb, so, flags, kc, ks, vc, vs, go, hkv, k_bf16=None):
    """Transformed queries and dequantised caches for the oracle."""
    B, Tq, Hq = qb.shape[:3]
    qf = S.bf16_to_f32(qb).astype(np.float64)
    if k_bf16 is None:
        s_per_q = np.repeat(so, Hq // hkv, axis=0)[None, None]          # [1][1][Hq][128]
        qp = O.query_transform(qf, s_per_q, flags)
        khat = [O.dequantize(kc[b], ks[b], go[0]) for b in range(B)]
    else:
        qp = qf
        khat = [S.bf16_to_f32(k_bf16[b]).astype(np.float64) for b in range(B)]
    vhat = [O.dequantize(vc[b], vs[b], go[1]) for b in range(B)]
    vmax = max(float(np.abs(vh).max()) for vh in vhat)
    return qp, khat, vhat, vmax


def oracle_prefill(qb, so, flags, kc, ks, vc, vs, go, seq_lens, hkv, k_bf16=None):
    qp, khat, vhat, vmax = oracle_inputs(qb, so, flags, kc, ks, vc, vs, go, hkv, k_bf16)
    return O.causal_attention(qp, khat, vhat, seq_lens, P.sm_scale()), vmax


def gpu_prefill(nk, cache, qb, pages, seq_lens, max_seq_len, table=None):
    B, Tq, Hq = qb.shape[:3]
    out = torch.full((B, Tq, Hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    tab = pages.table if table is None else table
    nk.prefill_attention_nvfp4(cache.struct(), P.to_dev_u16(qb), B, Tq, Hq, P.to_dev_i32(tab), tab.shape[1],
                               P.to_dev_i32(np.asarray(seq_lens)), max_seq_len, P.sm_scale(), out)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def assert_rows_close(got, ref, vmax, seq_lens, rows=None):
    """rows: optional list of (b, i) to check (all rows otherwise)."""
    B, Tq = ref.shape[:2]
    rows = rows if rows is not None else [(b, i) for b in range(B) for i in range(Tq)]
    for b, i in rows:
        g, r = got[b, i], ref[b, i]
        assert np.all(np.isfinite(g)), (b, i)
        if seq_lens[b] - Tq + i < 0:
            assert np.all(g == 0), (b, i)
            continue
        err = np.abs(g - r).max()
        assert err <= ATOL_FRAC * vmax, f"row {(b, i)}: max abs err {err:.3e} > {ATOL_FRAC * vmax:.3e}"
        rel = np.linalg.norm(g - r, axis=-1) / np.maximum(np.linalg.norm(r, axis=-1), 1e-30)
        assert rel.max() <= REL_L2, f"row {(b, i)}: rel L2 {rel.max():.3e} > {REL_L2}"


def build_layer(lib, name, flags, paged, T=None, B=None, k_fmt=1):
    c, k, v, kw, vw, q = P.workload(name, T=T, B=B)
    hkv = c["hkv"]
    s, r, g = gpu_calibrate(lib, kw, vw, hkv, flags)
    so, ro, go, kc, ks, vc, vs = oracle_layer(k, v, kw, vw, flags)
    pages = P.Pages(c["B"], c["T"], paged)
    cache = gpu_fill_cache(lib, k, v, hkv, flags, pages, s, r, g, k_fmt=k_fmt)
    return c, k, so, go, kc, ks, vc, vs, pages, cache


@pytest.mark.parametrize("name,Tq,flags", [(n, t, f) for n, t in (("tiny", 256), ("layer", 40)) for f in FLAG_SETS]
                         + [("tiny", 256, MSE | 3), ("layer", 40, MSE | 1)])
@pytest.mark.parametrize("paged", [False, True])
def test_prefill_parity(lib, name, Tq, flags, paged):
    c, k, so, go, kc, ks, vc, vs, pages, cache = build_layer(lib, name, flags, paged)
    T, B, hkv = c["T"], c["B"], c["hkv"]
    qb = S.make_query_block(c["cfg"], 0, B, Tq, c["hq"])
    seq = [T] * B
    ref, vmax = oracle_prefill(qb, so, flags, kc, ks, vc, vs, go, seq, hkv)
    got = gpu_prefill(lib, cache, qb, pages, seq, T)
    assert_rows_close(got, ref, vmax, seq)


@pytest.mark.parametrize("paged", [False, True])
def test_prefill_ragged_lengths(lib, paged):
    c, k, so, go, kc, ks, vc, vs, pages, cache = build_layer(lib, "layer", 3, paged, T=300)
    hkv = c["hkv"]
    for seq, Tq in (([0, 1, 16, 17], 21), ([33, 32, 300, 2], 13), ([65, 64, 97, 129], 64), ([299, 0, 256, 7], 9)):
        qb = S.make_query_block(c["cfg"], 0, 4, Tq, c["hq"])
        ref, vmax = oracle_prefill(qb, so, 3, kc, ks, vc, vs, go, seq, hkv)
        got = gpu_prefill(lib, cache, qb, pages, seq, 300)
        assert_rows_close(got, ref, vmax, seq)


@pytest.mark.parametrize("paged", [False, True])
def test_prefill_bf16_keys(lib, paged):
    c, k, so, go, kc, ks, vc, vs, pages, cache = build_layer(lib, "layer", 0, paged, T=700, k_fmt=0)
    hkv = c["hkv"]
    for seq, Tq in (([700, 700, 700, 700], 24), ([1, 0, 333, 97], 31)):
        qb = S.make_query_block(c["cfg"], 0, 4, Tq, c["hq"])
        ref, vmax = oracle_prefill(qb, so, 0, kc, ks, vc, vs, go, seq, hkv, k_bf16=k)
        got = gpu_prefill(lib, cache, qb, pages, seq, 700)
        assert_rows_close(got, ref, vmax, seq)


def test_prefill_full_window_sampled_rows(lib):
    """A full teacher-forced window of one Qwen3-8B layer (4 x 2304 positions); the oracle
    computes sampled rows one by one (row i alone is the last position of a block of one)."""
    c, k, so, go, kc, ks, vc, vs, pages, cache = build_layer(lib, "layer", 1, True)
    T, B, hkv = c["T"], c["B"], c["hkv"]
    qb = S.make_query_block(c["cfg"], 0, B, T, c["hq"])
    got = gpu_prefill(lib, cache, qb, pages, [T] * B, T)
    qp, khat, vhat, vmax = oracle_inputs(qb, so, 1, kc, ks, vc, vs, go, hkv)
    rng = np.random.default_rng(21)
    rows = [(b, i) for b in range(B) for i in sorted(set([0, 1, 7, 8, 31, 32, T - 1] +
                                                         list(rng.integers(0, T, 6))))]
    ref = np.zeros_like(got)
    for b, i in rows:
        ref[b, i] = O.causal_attention(qp[b:b + 1, i:i + 1], [khat[b]], [vhat[b]], [i + 1], P.sm_scale())[0, 0]
    assert_rows_close(got, ref, vmax, [T] * B, rows)


def test_prefill_last_row_matches_decode(lib):
    """The last position of a block attends to exactly what a decode query at that position
    does; the two kernels agree to within summation order."""
    c, k, so, go, kc, ks, vc, vs, pages, cache = build_layer(lib, "layer", 3, True, T=500)
    B = c["B"]
    qb = S.make_query_block(c["cfg"], 0, B, 16, c["hq"])
    seq = [500, 431, 77, 16]
    got = gpu_prefill(lib, cache, qb, pages, seq, 500)
    dec = gpu_decode(lib, cache, np.ascontiguousarray(qb[:, -1]), pages, seq, 500)
    assert np.max(np.abs(got[:, -1] - dec)) <= 1e-5 * np.max(np.abs(dec))


def test_prefill_is_deterministic(lib):
    c, k, so, go, kc, ks, vc, vs, pages, cache = build_layer(lib, "layer", 1, True, T=600)
    qb = S.make_query_block(c["cfg"], 0, c["B"], 48, c["hq"])
    a = gpu_prefill(lib, cache, qb, pages, [600, 599, 37, 48], 600)
    b = gpu_prefill(lib, cache, qb, pages, [600, 599, 37, 48], 600)
    assert np.array_equal(a, b)
