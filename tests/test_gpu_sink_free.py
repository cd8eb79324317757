"""GPU parity on sink-free workloads.

The other parity cases build every sequence and calibration window with a x40 key at
position 0 (the attention sink the u/krylov_schur thread on rstation.ai reports at 30-50x
RMS norm for Qwen3-8B).  With isotropic queries that sink takes more than 0.99 of the softmax
weight of many rows, whose outputs then reduce to the first value row on both sides.  Here
the same workloads are drawn without the sink, so the weight spreads over the context and
every row's output depends on the whole cache (checked: on the Qwen3-8B layer the median
row's largest softmax weight stays below 0.5, and no row puts more than 0.99 on position 0).

Bar as everywhere: max |err| <= 1e-3 * max|V_hat| over the layer and per-row relative L2
<= 1e-4 against the fp64 oracle; codes and scales bit-exact.  Covered: decode (every key
transform, MSE-searched key scales, bf16 keys), the fused decode step, causal prefill
attention, the static per-head KLT basis (with the oracle's basis installed, and end to end
with the library's own calibration).
"""
import numpy as np
import pytest

from oracle import nvfp4_oracle as O
from synth import kv_inputs as S
from tests import _pipeline as P
from tests.test_gpu_fused import check_cache_rows, gpu_decode_append, new_rows, spoil_slots
from tests.test_gpu_klt import KLT, gpu_calibrate_basis, install, oracle_klt_decode, oracle_klt_layer
from tests.test_gpu_parity import (FLAG_SETS, MSE, assert_close, gpu_calibrate, gpu_decode, gpu_fill_cache,
                                   oracle_decode, oracle_layer)
from tests.test_gpu_prefill import assert_rows_close, gpu_prefill, oracle_prefill

pytestmark = pytest.mark.gpu


def sink_free_layer(lib, name, flags, paged, k_fmt=1):
    c, k, v, kw, vw, q = P.workload(name, sink=False)
    s, r, g = gpu_calibrate(lib, kw, vw, c["hkv"], flags)
    so, ro, go, kc, ks, vc, vs = oracle_layer(k, v, kw, vw, flags)
    assert np.array_equal(g.cpu().numpy(), go) and np.array_equal(r.cpu().numpy(), ro)
    pages = P.Pages(c["B"], c["T"], paged)
    cache = gpu_fill_cache(lib, k, v, c["hkv"], flags, pages, s, r, g, k_fmt=k_fmt,
                           chunk=1000 if name == "layer" else None)
    return c, k, v, q, so, go, kc, ks, vc, vs, pages, cache


@pytest.mark.parametrize("name,flags", [(n, f) for n in ("tiny", "layer") for f in FLAG_SETS]
                         + [("tiny", MSE | 3), ("layer", MSE | 1)])
def test_decode_sink_free(lib, name, flags):
    c, k, v, q, so, go, kc, ks, vc, vs, pages, cache = sink_free_layer(lib, name, flags, paged=True)
    for b in range(c["B"]):
        gc, gs = P.rows_from_cache_vec(cache.k_data.cpu().numpy(), cache.k_scales.cpu().numpy(), pages, c["hkv"],
                                       b, c["T"])
        assert np.array_equal(gs, ks[b]) and np.array_equal(gc, kc[b]), f"K rows differ, seq {b}"
    seq = [c["T"]] * c["B"]
    ref, vmax = oracle_decode(q, so, flags, kc, ks, vc, vs, go, seq, c["hkv"])
    for split in (0, 32, 96, P.ceil_to(c["T"], 32)):
        assert_close(gpu_decode(lib, cache, q, pages, seq, c["T"], split), ref, vmax, seq)
    ragged = [c["T"], c["T"] - 17, 33, 1][:c["B"]] if c["B"] > 1 else [c["T"] - 17]
    ref, vmax = oracle_decode(q, so, flags, kc, ks, vc, vs, go, ragged, c["hkv"])
    assert_close(gpu_decode(lib, cache, q, pages, ragged, c["T"], 0), ref, vmax, ragged)


@pytest.mark.parametrize("paged", [False, True])
def test_decode_sink_free_bf16_keys(lib, paged):
    c, k, v, q, so, go, kc, ks, vc, vs, pages, cache = sink_free_layer(lib, "layer", 0, paged, k_fmt=0)
    seq = [c["T"], 1000, 17, 2048]
    ref, vmax = oracle_decode(q, so, 0, kc, ks, vc, vs, go, seq, c["hkv"], k_bf16=k)
    for split in (0, 64):
        assert_close(gpu_decode(lib, cache, q, pages, seq, c["T"], split), ref, vmax, seq)


@pytest.mark.parametrize("name,flags", [(n, f) for n in ("tiny", "layer") for f in (1, 3)] + [("layer", MSE | 1)])
@pytest.mark.parametrize("paged", [False, True])
def test_fused_step_sink_free(lib, name, flags, paged):
    c, k, v, q, so, go, kc, ks, vc, vs, pages, cache = sink_free_layer(lib, name, flags, paged)
    hkv, T, B = c["hkv"], c["T"], c["B"]
    seq = [T] * B
    kn, vn = new_rows(k, v, seq)
    ref, vmax = oracle_decode(q, so, flags, kc, ks, vc, vs, go, seq, hkv)
    for split in (0, 32, 96):
        spoil_slots(lib, cache, pages, seq, hkv, seed=split + 1)
        got = gpu_decode_append(lib, cache, q, kn, vn, pages, seq, T, split)
        assert_close(got, ref, vmax, seq)
        check_cache_rows(cache, pages, hkv, kc, ks, vc, vs, seq)


@pytest.mark.parametrize("name,Tq,flags", [("tiny", 256, 1), ("tiny", 256, 3), ("layer", 40, 1), ("layer", 40, 3)])
def test_prefill_sink_free(lib, name, Tq, flags):
    c, k, v, q, so, go, kc, ks, vc, vs, pages, cache = sink_free_layer(lib, name, flags, paged=True)
    B, T, hkv = c["B"], c["T"], c["hkv"]
    qb = S.make_query_block(c["cfg"], 0, B, Tq, c["hq"])
    for seq in ([T] * B, [T, T - 5, Tq + 3, 7][:B]):
        ref, vmax = oracle_prefill(qb, so, flags, kc, ks, vc, vs, go, seq, hkv)
        assert_rows_close(gpu_prefill(lib, cache, qb, pages, seq, T), ref, vmax, seq)


@pytest.mark.parametrize("name", ["tiny", "layer"])
def test_klt_sink_free(lib, name):
    """The oracle's KLT basis installed: decode, fused step and prefill over sink-free
    workloads."""
    flags = KLT | 1
    c, k, v, kw, vw, q, s, r, g, basis, lam, kc, ks, vc, vs = oracle_klt_layer(name, flags, sink=False)
    T, B, hkv, hq = c["T"], c["B"], c["hkv"], c["hq"]
    pages = P.Pages(B, T, True)
    cache = install(lib, c, k, v, flags, pages, s, r, g, basis)
    seq = [T] * B
    ref, vmax = oracle_klt_decode(q, s, flags, basis, kc, ks, vc, vs, g, seq, hkv)
    for split in (0, 64):
        assert_close(gpu_decode(lib, cache, q, pages, seq, T, split), ref, vmax, seq)
    kn, vn = new_rows(k, v, seq)
    spoil_slots(lib, cache, pages, seq, hkv, seed=5)
    assert_close(gpu_decode_append(lib, cache, q, kn, vn, pages, seq, T, 0), ref, vmax, seq)
    check_cache_rows(cache, pages, hkv, kc, ks, vc, vs, seq)
    Tq = 40
    qb = S.make_query_block(c["cfg"], 0, B, Tq, hq)
    grp = hq // hkv
    qp = O.query_transform(S.bf16_to_f32(qb).astype(np.float64), np.repeat(s, grp, axis=0)[None, None], flags,
                           np.repeat(basis, grp, axis=0)[None, None])
    khat = [O.dequantize(kc[b], ks[b], g[0]) for b in range(B)]
    vhat = [O.dequantize(vc[b], vs[b], g[1]) for b in range(B)]
    pref = O.causal_attention(qp, khat, vhat, seq, P.sm_scale())
    assert_rows_close(gpu_prefill(lib, cache, qb, pages, seq, T), pref, vmax, seq)


@pytest.mark.parametrize("sink", [True, False])
def test_klt_end_to_end_layer(lib, sink):
    """The library's own KLT calibration (s, r, fp64 Jacobi basis, g) -> append -> decode and
    fused step on a Qwen3-8B layer, against the oracle's own calibration (LAPACK basis) and
    encoding, held to the decode bar.  Separately bounded: the two bases differ by at most
    1e-5 per entry on every column the eigenvalue gaps determine (columns of near-equal
    eigenvalues may rotate within their span), and at most 1e-4 of the key code bytes differ
    (a rotated key lands on the other side of an E2M1 midpoint only when it lies within the
    basis difference of that midpoint)."""
    flags = KLT | 1
    c, k, v, kw, vw, q, s, r, g, basis, lam, kc, ks, vc, vs = oracle_klt_layer("layer", flags, sink=sink)
    T, B, hkv = c["T"], c["B"], c["hkv"]
    sg, rg, gg = gpu_calibrate(lib, kw, vw, hkv, flags)
    assert np.array_equal(rg.cpu().numpy(), r)
    Bg, g2 = gpu_calibrate_basis(lib, kw, hkv, flags, rg)
    for h in range(hkv):
        l = lam[h]
        gap = np.minimum(np.abs(np.diff(l, prepend=np.inf)), np.abs(np.diff(l, append=-np.inf)))
        sep = gap > 1e-6 * np.abs(l).max()
        assert np.max(np.abs(Bg[h][:, sep].astype(np.float64) - basis[h][:, sep])) <= 1e-5
    assert abs(float(g2[0]) - float(g[0])) <= 1e-5 * float(g[0])
    gg[0] = float(g2[0])
    pages = P.Pages(B, T, True)
    cache = gpu_fill_cache(lib, k, v, hkv, flags, pages, sg, rg, gg, basis=Bg, chunk=1000)
    kd, ksd = cache.k_data.cpu().numpy(), cache.k_scales.cpu().numpy()
    diff = total = 0
    for b in range(B):
        gc, gs = P.rows_from_cache_vec(kd, ksd, pages, hkv, b, T)
        diff += int(np.count_nonzero(gc != kc[b])) + int(np.count_nonzero(gs != ks[b]))
        total += gc.size + gs.size
    assert diff <= 1e-4 * total, (diff, total)
    seq = [T] * B
    ref, vmax = oracle_klt_decode(q, s, flags, basis, kc, ks, vc, vs, g, seq, hkv)
    for split in (0, 96):
        assert_close(gpu_decode(lib, cache, q, pages, seq, T, split), ref, vmax, seq)
    kn, vn = new_rows(k, v, seq)
    assert_close(gpu_decode_append(lib, cache, q, kn, vn, pages, seq, T, 0), ref, vmax, seq)
