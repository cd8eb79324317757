"""GPU parity: the native library against the CPU oracle on the same seeded inputs.

* calibration outputs s, r, g and packed codes / scales: bit-exact;
* decode attention: max |err| <= 1e-3 * max|V_hat| over the layer's cache and per-(b, q-head)
  relative L2 <= 1e-4 against the fp64 oracle.
Workloads: the tiny reference (1 KV head, 4 query heads, context 256) and one Qwen3-8B-shaped
layer (8 KV heads, 32 query heads, batch 4, context 2304); contiguous and 16-token paged
caches with a shuffled page table; every key-transform combination; BF16 keys; the
MSE-searched key block scale (NVKV_K_MSE_SCALE) with each key transform.
"""
import hashlib

import numpy as np
import pytest
import torch

from oracle import nvfp4_oracle as O
from synth import kv_inputs as S
from tests import _pipeline as P
from tests.conftest import gpu_available

pytestmark = pytest.mark.gpu

FLAG_SETS = [0, 1, 2, 3]
MSE = O.FLAG_MSE_SCALE
MSE_FLAG_SETS = [MSE, MSE | 1, MSE | 3]
# (workload, key flags): every flag set on the tiny reference, the MSE search on the
# Qwen3-8B layer with smoothing (the oracle's search takes ~15 s per layer)
QUANT_CASES = ([(n, f) for n in ("tiny", "layer") for f in FLAG_SETS] + [("tiny", f) for f in MSE_FLAG_SETS]
               + [("layer", MSE | 1)])
ATOL_FRAC = 1e-3
REL_L2 = 1e-4


def gpu_calibrate(nk, kw, vw, hkv, flags, exclude_pos0=True):
    W, Tw = kw.shape[0], kw.shape[1]
    s = torch.empty((hkv, 128), dtype=torch.float32, device="cuda")
    r = torch.empty_like(s)
    g = torch.empty(2, dtype=torch.float32, device="cuda")
    nk.calibrate_key_smoothing(P.to_dev_u16(kw), P.to_dev_u16(vw), W, Tw, hkv, exclude_pos0, flags, s, r, g)
    torch.cuda.synchronize()
    return s, r, g


def gpu_fill_cache(nk, k, v, hkv, flags, pages, s, r, g, k_fmt=1, chunk=None, basis=None):
    """Append every token of every sequence; returns the CacheLayer.  basis: the KLT key
    basis to install (flags with NVKV_K_KLT)."""
    B, T = k.shape[0], k.shape[1]
    cache = nk.CacheLayer(pages.num_pages, pages.page_size, hkv, k_fmt=k_fmt, k_flags=flags if k_fmt == 1 else 0)
    cache.smooth.copy_(s)
    cache.inv_smooth.copy_(r)
    cache.gscale.copy_(torch.as_tensor(g))
    if basis is not None:
        cache.basis.copy_(torch.as_tensor(basis))
    L = cache.struct()
    slots = np.concatenate([pages.slots(b, 0, T) for b in range(B)])
    kk = k.reshape(B * T, hkv, 128)
    vv = v.reshape(B * T, hkv, 128)
    step = chunk or B * T
    for i in range(0, B * T, step):
        nk.quantize_append_kv(L, P.to_dev_u16(kk[i:i + step]), P.to_dev_u16(vv[i:i + step]),
                              P.to_dev_i32(slots[i:i + step]), min(step, B * T - i))
    torch.cuda.synchronize()
    return cache


_ORACLE_LAYERS = {}


def _digest(*arrays) -> str:
    h = hashlib.sha1()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def oracle_layer(k, v, kw, vw, flags, exclude_pos0=True):
    """Oracle calibration and encoding of one layer (memoised per input and flags; callers
    treat the returned arrays as read-only)."""
    key = (_digest(k, v, kw, vw), flags, exclude_pos0)
    if key not in _ORACLE_LAYERS:
        kwf, vwf = S.bf16_to_f32(kw), S.bf16_to_f32(vw)
        s, r, g = O.calibrate(kwf, vwf, exclude_pos0=exclude_pos0, k_flags=flags)
        y = O.key_transform(S.bf16_to_f32(k), r[None, None], flags)
        kc, ks = O.quantize_keys(y, g[0], flags)
        vc, vs = O.quantize_rows(S.bf16_to_f32(v), g[1])
        _ORACLE_LAYERS[key] = (s, r, g, kc, ks, vc, vs)
    return _ORACLE_LAYERS[key]


@pytest.mark.parametrize("name", ["tiny", "layer"])
@pytest.mark.parametrize("flags", FLAG_SETS)
def test_calibrate_bit_exact(lib, name, flags):
    c, k, v, kw, vw, q = P.workload(name)
    for excl in (True, False):
        s, r, g = gpu_calibrate(lib, kw, vw, c["hkv"], flags, excl)
        so, ro, go = O.calibrate(S.bf16_to_f32(kw), S.bf16_to_f32(vw), exclude_pos0=excl, k_flags=flags)
        assert np.array_equal(s.cpu().numpy().view(np.uint32), so.view(np.uint32))
        assert np.array_equal(r.cpu().numpy().view(np.uint32), ro.view(np.uint32))
        assert np.array_equal(g.cpu().numpy().view(np.uint32), go.view(np.uint32)), (g, go)


@pytest.mark.parametrize("name,flags", QUANT_CASES)
@pytest.mark.parametrize("paged", [False, True])
def test_quantize_bit_exact(lib, name, flags, paged):
    c, k, v, kw, vw, q = P.workload(name)
    s, r, g = gpu_calibrate(lib, kw, vw, c["hkv"], flags)
    so, ro, go, kc, ks, vc, vs = oracle_layer(k, v, kw, vw, flags)
    assert np.array_equal(g.cpu().numpy(), go)
    pages = P.Pages(c["B"], c["T"], paged)
    cache = gpu_fill_cache(lib, k, v, c["hkv"], flags, pages, s, r, g, chunk=1000 if name == "layer" else None)
    kd, ksd = cache.k_data.cpu().numpy(), cache.k_scales.cpu().numpy()
    vd, vsd = cache.v_data.cpu().numpy(), cache.v_scales.cpu().numpy()
    for b in range(c["B"]):
        gc, gs = P.rows_from_cache_vec(kd, ksd, pages, c["hkv"], b, c["T"])
        assert np.array_equal(gs, ks[b]), f"K scales differ, seq {b}"
        assert np.array_equal(gc, kc[b]), f"K codes differ, seq {b}"
        gc, gs = P.rows_from_cache_vec(vd, vsd, pages, c["hkv"], b, c["T"], values=True)
        assert np.array_equal(gs, vs[b]), f"V scales differ, seq {b}"
        assert np.array_equal(gc, vc[b]), f"V codes differ, seq {b}"


def oracle_decode(q, so, flags, kc, ks, vc, vs, go, seq_lens, hkv, k_bf16=None):
    B, Hq = q.shape[0], q.shape[1]
    grp = Hq // hkv
    qf = S.bf16_to_f32(q).astype(np.float64)
    if k_bf16 is None:
        s_per_q = np.repeat(so, grp, axis=0)[None]               # [1][Hq][128]
        qp = O.query_transform(qf, s_per_q, flags)
        khat = [O.dequantize(kc[b], ks[b], go[0]) for b in range(B)]
    else:
        qp = qf
        khat = [S.bf16_to_f32(k_bf16[b]).astype(np.float64) for b in range(B)]
    vhat = [O.dequantize(vc[b], vs[b], go[1]) for b in range(B)]
    out = O.attention(qp, khat, vhat, seq_lens, P.sm_scale())
    vmax = max(float(np.abs(vh).max()) for vh in vhat)
    return out, vmax


def gpu_decode(nk, cache, q, pages, seq_lens, max_seq_len, split_tokens=0):
    B, Hq = q.shape[0], q.shape[1]
    out = torch.full((B, Hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    wsb = nk.decode_workspace_bytes(B, Hq, cache.hkv, max_seq_len, split_tokens)
    ws = torch.zeros(max(wsb, 256), dtype=torch.uint8, device="cuda")
    nk.decode_attention_nvfp4(cache.struct(), P.to_dev_u16(q), B, Hq, P.to_dev_i32(pages.table),
                              pages.table.shape[1], P.to_dev_i32(np.asarray(seq_lens)), max_seq_len, P.sm_scale(),
                              out, ws, wsb, split_tokens)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def assert_close(got, ref, vmax, seq_lens):
    assert np.all(np.isfinite(got))
    err = np.abs(got - ref)
    assert err.max() <= ATOL_FRAC * vmax, f"max abs err {err.max():.3e} > {ATOL_FRAC * vmax:.3e}"
    for b in range(ref.shape[0]):
        if seq_lens[b] == 0:
            assert np.all(got[b] == 0)
            continue
        num = np.linalg.norm(got[b] - ref[b], axis=-1)
        den = np.linalg.norm(ref[b], axis=-1)
        rel = num / np.maximum(den, 1e-30)
        assert rel.max() <= REL_L2, f"seq {b}: rel L2 {rel.max():.3e} > {REL_L2}"


@pytest.mark.parametrize("name,flags", [(n, f) for n in ("tiny", "layer") for f in FLAG_SETS]
                         + [("tiny", MSE | 3), ("layer", MSE | 1)])
@pytest.mark.parametrize("paged", [False, True])
def test_decode_parity(lib, name, flags, paged):
    c, k, v, kw, vw, q = P.workload(name)
    s, r, g = gpu_calibrate(lib, kw, vw, c["hkv"], flags)
    so, ro, go, kc, ks, vc, vs = oracle_layer(k, v, kw, vw, flags)
    pages = P.Pages(c["B"], c["T"], paged)
    cache = gpu_fill_cache(lib, k, v, c["hkv"], flags, pages, s, r, g)
    seq = [c["T"]] * c["B"]
    ref, vmax = oracle_decode(q, so, flags, kc, ks, vc, vs, go, seq, c["hkv"])
    for split in (0, 32, 96, P.ceil_to(c["T"], 32)):
        got = gpu_decode(lib, cache, q, pages, seq, c["T"], split)
        assert_close(got, ref, vmax, seq)


@pytest.mark.parametrize("paged", [False, True])
def test_decode_ragged_and_empty_sequences(lib, paged):
    c, k, v, kw, vw, q = P.workload("layer", T=300)
    flags = 1
    s, r, g = gpu_calibrate(lib, kw, vw, c["hkv"], flags)
    so, ro, go, kc, ks, vc, vs = oracle_layer(k, v, kw, vw, flags)
    pages = P.Pages(c["B"], c["T"], paged)
    cache = gpu_fill_cache(lib, k, v, c["hkv"], flags, pages, s, r, g)
    for seq in ([0, 1, 15, 16], [17, 31, 33, 300], [299, 0, 64, 65], [128, 129, 255, 257]):
        ref, vmax = oracle_decode(q, so, flags, kc, ks, vc, vs, go, seq, c["hkv"])
        for split in (0, 32, 64, 320):
            got = gpu_decode(lib, cache, q, pages, seq, 300, split)
            assert_close(got, ref, vmax, seq)


def test_decode_split_invariance_and_determinism(lib):
    c, k, v, kw, vw, q = P.workload("layer")
    flags = 1
    s, r, g = gpu_calibrate(lib, kw, vw, c["hkv"], flags)
    pages = P.Pages(c["B"], c["T"], True)
    cache = gpu_fill_cache(lib, k, v, c["hkv"], flags, pages, s, r, g)
    seq = [c["T"]] * c["B"]
    outs = [gpu_decode(lib, cache, q, pages, seq, c["T"], sp) for sp in (0, 32, 128, 288, 512, 1024, 2304)]
    for o in outs[1:]:
        assert np.max(np.abs(o - outs[0])) <= 1e-5 * np.max(np.abs(outs[0]))
    a = gpu_decode(lib, cache, q, pages, seq, c["T"], 128)
    b = gpu_decode(lib, cache, q, pages, seq, c["T"], 128)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("paged", [False, True])
def test_bf16_keys_nvfp4_values(lib, paged):
    """The 'NVFP4 V only' cache configuration: keys stay bf16, values NVFP4."""
    c, k, v, kw, vw, q = P.workload("layer")
    s, r, g = gpu_calibrate(lib, kw, vw, c["hkv"], 0)
    so, ro, go, kc, ks, vc, vs = oracle_layer(k, v, kw, vw, 0)
    pages = P.Pages(c["B"], c["T"], paged)
    cache = gpu_fill_cache(lib, k, v, c["hkv"], 0, pages, s, r, g, k_fmt=0)
    kd = cache.k_data.cpu().numpy()
    for b in range(c["B"]):
        assert np.array_equal(P.bf16_rows_from_cache(kd, pages, c["hkv"], b, c["T"]), k[b])
        gc, gs = P.rows_from_cache_vec(cache.v_data.cpu().numpy(), cache.v_scales.cpu().numpy(), pages,
                                       c["hkv"], b, c["T"], values=True)
        assert np.array_equal(gc, vc[b]) and np.array_equal(gs, vs[b])
    seq = [c["T"], 1000, 17, 2048]
    ref, vmax = oracle_decode(q, so, 0, kc, ks, vc, vs, go, seq, c["hkv"], k_bf16=k)
    for split in (0, 64):
        got = gpu_decode(lib, cache, q, pages, seq, c["T"], split)
        assert_close(got, ref, vmax, seq)


def test_special_rows_bit_exact(lib):
    """Rows built to hit the codec's corner cases: zero and underflowing blocks (scale 0),
    E4M3 subnormal scales, saturated scales, exact E2M1 midpoints, signed zeros."""
    rng = np.random.default_rng(11)
    hkv, N = 2, 96
    g_val = np.float32(2.0 ** -7)
    rows = (rng.standard_normal((N, hkv, 128)) * np.exp(rng.uniform(-6, 1, (N, hkv, 128)))).astype(np.float32)
    rows[0, 0] = 0.0
    rows[1, 0, :16] = 1e-20                                  # scale underflows to 0
    rows[2, 0, :16] = 3e-4                                   # A/(6g) in the E4M3 subnormal range
    rows[3, 0, :16] = 4e4                                    # saturates the scale (0x7E)
    rows[4, 0, ::2] = -0.0
    # exact E2M1 midpoints with a representable block scale: A = 6 * sigma * g, sigma = 3
    unit = np.float32(3.0) * g_val
    rows[5, 1, 0] = np.float32(18.0) * g_val
    for i, m in enumerate([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]):
        rows[5, 1, 1 + i] = np.float32(m) * unit
    kbits = S.bf16_round(rows)
    vbits = S.bf16_round(rows[::-1].copy())
    k32, v32 = S.bf16_to_f32(kbits), S.bf16_to_f32(vbits)
    assert np.array_equal(k32[5, 1, :8], rows[5, 1, :8])     # midpoints survive bf16 rounding
    g = np.array([g_val, g_val], np.float32)
    kc, ks = O.quantize_rows(k32, g[0])
    vc, vs = O.quantize_rows(v32, g[1])
    pages = P.Pages(1, N, True)
    cache = lib.CacheLayer(pages.num_pages, pages.page_size, hkv, k_flags=0)
    cache.gscale.copy_(torch.from_numpy(g))
    lib.quantize_append_kv(cache.struct(), P.to_dev_u16(kbits), P.to_dev_u16(vbits),
                           P.to_dev_i32(pages.slots(0, 0, N)), N)
    torch.cuda.synchronize()
    gc, gs = P.rows_from_cache_vec(cache.k_data.cpu().numpy(), cache.k_scales.cpu().numpy(), pages, hkv, 0, N)
    assert np.array_equal(gs, ks) and np.array_equal(gc, kc)
    gc, gs = P.rows_from_cache_vec(cache.v_data.cpu().numpy(), cache.v_scales.cpu().numpy(), pages, hkv, 0, N,
                                   values=True)
    assert np.array_equal(gs, vs) and np.array_equal(gc, vc)
    assert 0 in ks[:, 0, 0] and 0x7E in ks[:, 0, 0] and np.any((ks > 0) & (ks < 8))


@pytest.mark.parametrize("flags", [1, 1 | 4])
def test_near_midpoint_keys_bit_exact(lib, flags):
    """Smoothed keys placed within a few ulp of every E2M1 midpoint of their block (the
    encoder's converter brackets disagree there and the exact bound-based path decides), at
    the midpoints themselves, and 64 ulp away (the brackets agree); also with the MSE-searched
    scales.  The smoothing factors r are chosen per channel so that y = fl32(x * r) lands on
    the target; the block maximum fixes sigma = 3."""
    rng = np.random.default_rng(29)
    hkv, N = 8, 16
    g = np.float32(2.0 ** -7)
    u = np.float32(3.0) * g                                     # sigma * g, exact
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    offs = [-64, -3, -2, -1, 0, 1, 2, 3, 64]
    r = np.ones((hkv, 128), np.float32)
    x = np.zeros((hkv, 128), np.float32)
    k_idx = 0
    for h in range(hkv):
        for blk in range(8):
            j0 = 16 * blk
            x[h, j0] = np.float32(18.0) * g                       # block maximum 6 * sigma * g
            for t in range(1, 16):
                T = np.float32(mids[k_idx % 7]) * u               # exact midpoint threshold
                target = (T.view(np.uint32) + np.int64(offs[k_idx % 9])).astype(np.uint32).view(np.float32)
                X = S.bf16_to_f32(S.bf16_round(np.float32(rng.uniform(0.5, 4.0)) * np.ones(1, np.float32)))[0]
                X = X if k_idx % 5 else -X
                r[h, j0 + t] = np.float32(target / np.float64(abs(X)))
                x[h, j0 + t] = X
                k_idx += 1
    kbits = np.broadcast_to(S.bf16_round(x)[None, None], (1, N, hkv, 128)).copy()
    vbits = S.bf16_round(rng.standard_normal((1, N, hkv, 128)).astype(np.float32))
    k32 = S.bf16_to_f32(kbits)
    assert np.array_equal(k32[0, 0], x)
    y = O.key_transform(k32, r[None, None], flags)
    near = np.abs(np.abs(y[0, 0]) / np.float64(u) - np.array(mids)[:, None, None]).min(axis=0)
    assert np.count_nonzero(near < 2.0 ** -21) > 200                   # many within the bracket margin
    gg = np.array([g, g], np.float32)
    kc, ks = O.quantize_keys(y, gg[0], flags)
    vc, vs = O.quantize_rows(S.bf16_to_f32(vbits), gg[1])
    pages = P.Pages(1, N, True)
    s = (np.float32(1.0) / r).astype(np.float32)
    cache = gpu_fill_cache(lib, kbits, vbits, hkv, flags, pages, torch.from_numpy(s).cuda(),
                           torch.from_numpy(r).cuda(), gg)
    gc, gs = P.rows_from_cache_vec(cache.k_data.cpu().numpy(), cache.k_scales.cpu().numpy(), pages, hkv, 0, N)
    assert np.array_equal(gs, ks[0]) and np.array_equal(gc, kc[0])
    gc, gs = P.rows_from_cache_vec(cache.v_data.cpu().numpy(), cache.v_scales.cpu().numpy(), pages, hkv, 0, N,
                                   values=True)
    assert np.array_equal(gs, vs[0]) and np.array_equal(gc, vc[0])


@pytest.mark.parametrize("flags", [1, 1 | 4])
def test_absmax_near_e4m3_midpoints_bit_exact(lib, flags):
    """Smoothed keys whose block absmax lies 0, 1, 3 or 64 fp32 ulp from 6 g times an E4M3
    midpoint (subnormal, normal and near-saturation codes): the append's E4M3 converter
    brackets disagree within about 2^-20 of a midpoint and the exact tests decide there; also
    with the MSE-searched scales, whose search starts from that code.  The smoothing factor of
    each block's first channel puts y there exactly (x = 1 in bf16)."""
    rng = np.random.default_rng(31)
    hkv, N = 8, 16
    g = np.float32(2.0 ** -7)
    grid = O.E4M3_GRID
    codes = [1, 3, 6, 7, 8, 21, 50, 77, 100, 118, 124, 125]
    offs = [-64, -3, -1, 0, 1, 3, 64]
    r = np.ones((hkv, 128), np.float32)
    x = S.bf16_to_f32(S.bf16_round(rng.uniform(-1, 1, (hkv, 128)).astype(np.float32)))
    targets = []
    for h in range(hkv):
        for blk in range(8):
            i = 8 * h + blk
            k, off = codes[i % len(codes)], offs[(i // len(codes) + i) % len(offs)]
            m6 = np.float32(3.0 * (grid[k] + grid[k + 1]) * np.float64(g))     # 6 g midpoint, exact
            t = (m6.view(np.uint32) + np.int64(off)).astype(np.uint32).view(np.float32)
            j0 = 16 * blk
            x[h, j0] = 1.0
            r[h, j0] = t
            x[h, j0 + 1:j0 + 16] *= np.float32(0.9) * t          # r = 1 there: |y| < t
            targets.append(t)
    x = S.bf16_to_f32(S.bf16_round(x))
    kbits = np.broadcast_to(S.bf16_round(x)[None, None], (1, N, hkv, 128)).copy()
    kbits[0, 1::2] ^= np.uint16(0x8000)                          # odd tokens negated
    vbits = S.bf16_round(rng.standard_normal((1, N, hkv, 128)).astype(np.float32))
    y = O.key_transform(S.bf16_to_f32(kbits), r[None, None], flags)
    amax = np.abs(y[0, 0]).reshape(hkv, 8, 16).max(-1)
    assert np.array_equal(amax.ravel(), np.array(targets, np.float32))
    gg = np.array([g, g], np.float32)
    kc, ks = O.quantize_keys(y, gg[0], flags)
    if flags == 1:      # exact ties went to the even code, and the neighbours to their side
        assert len(set(ks[0, 0].ravel().tolist())) > 12
    vc, vs = O.quantize_rows(S.bf16_to_f32(vbits), gg[1])
    pages = P.Pages(1, N, True)
    s = (np.float32(1.0) / r).astype(np.float32)
    cache = gpu_fill_cache(lib, kbits, vbits, hkv, flags, pages, torch.from_numpy(s).cuda(),
                           torch.from_numpy(r).cuda(), gg)
    gc, gs = P.rows_from_cache_vec(cache.k_data.cpu().numpy(), cache.k_scales.cpu().numpy(), pages, hkv, 0, N)
    assert np.array_equal(gs, ks[0]) and np.array_equal(gc, kc[0])
    gc, gs = P.rows_from_cache_vec(cache.v_data.cpu().numpy(), cache.v_scales.cpu().numpy(), pages, hkv, 0, N,
                                   values=True)
    assert np.array_equal(gs, vs[0]) and np.array_equal(gc, vc[0])


def test_scale_code_at_every_e4m3_midpoint(lib):
    """Block absmax exactly at 6*g times each of the 126 E4M3 midpoints (ties: the even code
    wins), and one bf16 step above and below each, for two tensor scales; codes and scales
    bit-exact against the oracle."""
    grid = O.E4M3_GRID
    mids6 = 3.0 * (grid[:-1] + grid[1:])                      # 6 * midpoint, exact
    hkv = 1
    for g_val in (np.float32(2.0 ** -9), np.float32(0.0390625)):   # power of two, and 5 * 2^-7
        amax = []
        for m6 in mids6:
            t = np.float32(m6 * np.float64(g_val))
            b = S.bf16_round(np.array([t], np.float32))[0]
            for d in (-1, 0, 1):
                amax.append(S.bf16_to_f32(np.array([int(b) + d], np.uint16))[0])
        amax = np.array(amax, np.float32)
        N = len(amax)
        rows = np.zeros((N, hkv, 128), np.float32)
        rng = np.random.default_rng(5)
        for blk in range(8):
            rows[:, 0, 16 * blk] = amax * (1 if blk % 2 == 0 else -1)
            rows[:, 0, 16 * blk + 1: 16 * blk + 16] = amax[:, None] * rng.uniform(-1, 1, (N, 15))
        bits = S.bf16_round(rows)
        r32 = S.bf16_to_f32(bits)
        g = np.array([g_val, g_val], np.float32)
        kc, ks = O.quantize_rows(r32, g[0])
        pages = P.Pages(1, N, True)
        cache = lib.CacheLayer(pages.num_pages, pages.page_size, hkv, k_flags=0)
        cache.gscale.copy_(torch.from_numpy(g))
        lib.quantize_append_kv(cache.struct(), P.to_dev_u16(bits), P.to_dev_u16(bits),
                               P.to_dev_i32(pages.slots(0, 0, N)), N)
        torch.cuda.synchronize()
        gc, gs = P.rows_from_cache_vec(cache.k_data.cpu().numpy(), cache.k_scales.cpu().numpy(), pages, hkv, 0, N)
        assert np.array_equal(gs, ks), np.argwhere(gs != ks)[:5]
        assert np.array_equal(gc, kc)
        gc, gs = P.rows_from_cache_vec(cache.v_data.cpu().numpy(), cache.v_scales.cpu().numpy(), pages, hkv, 0, N,
                                       values=True)
        assert np.array_equal(gs, ks) and np.array_equal(gc, kc)
        # the ties really are ties for the power-of-two scale: every code 1..126 is hit
        if g_val == np.float32(2.0 ** -9):
            assert set(np.unique(ks[:, 0, 0])) >= set(range(1, 127))


def test_append_canaries_and_skipped_slots(lib):
    """Only the addressed slots change; negative and out-of-range slots write nothing."""
    rng = np.random.default_rng(12)
    hkv, N = 3, 40
    pages = P.Pages(2, 64, True, spare=2)
    cache = lib.CacheLayer(pages.num_pages, pages.page_size, hkv, k_flags=3, fill=0xA5)
    cache.smooth.fill_(1.5)
    cache.inv_smooth.copy_(torch.full_like(cache.smooth, 1 / 1.5))
    cache.gscale.fill_(0.01)
    before = [t.cpu().numpy().copy() for t in (cache.k_data, cache.k_scales, cache.v_data, cache.v_scales)]
    k = S.bf16_round(rng.standard_normal((N, hkv, 128)).astype(np.float32))
    v = S.bf16_round(rng.standard_normal((N, hkv, 128)).astype(np.float32))
    slots = pages.slots(1, 5, 5 + N).copy()
    slots[3] = -1
    slots[7] = pages.num_pages * pages.page_size          # one past the end
    slots[8] = 2 ** 31 - 1
    lib.quantize_append_kv(cache.struct(), P.to_dev_u16(k), P.to_dev_u16(v), P.to_dev_i32(slots), N)
    torch.cuda.synchronize()
    after = [t.cpu().numpy() for t in (cache.k_data, cache.k_scales, cache.v_data, cache.v_scales)]
    written = set(int(x) for i, x in enumerate(slots) if i not in (3, 7, 8))
    ps = pages.page_size
    for idx, (arr_b, arr_a) in enumerate(zip(before, after)):
        if idx in (0, 2):                                   # K codes, V codes (their layouts)
            b3 = P.codes_view(arr_b, pages, hkv, values=idx == 2)
            a3 = P.codes_view(arr_a, pages, hkv, values=idx == 2)
            for pg in range(pages.num_pages):
                for off in range(ps):
                    same = np.array_equal(b3[pg, :, off], a3[pg, :, off])
                    assert same == ((pg * ps + off) not in written)
        else:
            b5 = arr_b.reshape(pages.num_pages, hkv, ps // 4, 8, 4)
            a5 = arr_a.reshape(pages.num_pages, hkv, ps // 4, 8, 4)
            for pg in range(pages.num_pages):
                for off in range(ps):
                    same = np.array_equal(b5[pg, :, off // 4, :, off % 4], a5[pg, :, off // 4, :, off % 4])
                    if (pg * ps + off) not in written:
                        assert same


def test_append_unaligned_arrays(lib):
    """Scale arrays at odd byte addresses and code arrays off 16-byte alignment (allowed by
    the layout) take the per-token stores: bytes identical to the oracle's, with page-ordered
    slots that would otherwise use the word-wide quad stores, and a ragged token count."""
    rng = np.random.default_rng(41)
    hkv, N = 2, 77
    pages = P.Pages(2, 48, True, spare=1)
    flags = 1
    cache = lib.CacheLayer(pages.num_pages, pages.page_size, hkv, k_flags=flags, fill=0)
    sm = (1.0 + rng.random((hkv, 128))).astype(np.float32)
    cache.smooth.copy_(torch.from_numpy(sm))
    r = (np.float32(1.0) / sm).astype(np.float32)
    cache.inv_smooth.copy_(torch.from_numpy(r))
    cache.gscale.copy_(torch.tensor([0.004, 0.003], dtype=torch.float32))
    L = cache.struct()
    nbytes = {name: getattr(cache, name).numel() for name in ("k_data", "k_scales", "v_data", "v_scales")}
    offs = {"k_data": 8, "k_scales": 1, "v_data": 4, "v_scales": 3}
    bufs = {name: torch.zeros(nbytes[name] + 64, dtype=torch.uint8, device="cuda") for name in offs}
    for name, off in offs.items():
        setattr(L, name, bufs[name].data_ptr() + off)
    k = S.bf16_round(rng.standard_normal((N, hkv, 128)).astype(np.float32))
    v = S.bf16_round(rng.standard_normal((N, hkv, 128)).astype(np.float32))
    slots = np.concatenate([pages.slots(0, 0, 40), pages.slots(1, 0, N - 40)])
    lib.quantize_append_kv(L, P.to_dev_u16(k), P.to_dev_u16(v), P.to_dev_i32(slots), N)
    torch.cuda.synchronize()
    got = {name: bufs[name].cpu().numpy()[off:off + nbytes[name]] for name, off in offs.items()}
    for name, off in offs.items():      # nothing outside the arrays
        full = bufs[name].cpu().numpy()
        assert not full[:off].any() and not full[off + nbytes[name]:].any(), name
    y = O.key_transform(S.bf16_to_f32(k)[None], r[None, None], flags)[0]
    kc, ks = O.quantize_rows(y, np.float32(0.004))
    vc, vs = O.quantize_rows(S.bf16_to_f32(v), np.float32(0.003))
    ps = pages.page_size
    for n, slot in enumerate(slots):
        pg, t = int(slot) // ps, int(slot) % ps
        for h in range(hkv):
            blk = (pg * hkv + h) * ps
            for w in range(16):
                for by in range(4):
                    assert got["k_data"][blk * 64 + 64 * t + 4 * w + by] == kc[n, h, 4 * w + by]
                    assert got["v_data"][blk * 64 + ((t // 4) * 16 + w) * 16 + (t % 4) * 4 + by] == vc[n, h, 4 * w + by]
            for b8 in range(8):
                assert got["k_scales"][blk * 8 + ((t // 4) * 8 + b8) * 4 + t % 4] == ks[n, h, b8]
                assert got["v_scales"][blk * 8 + ((t // 4) * 8 + b8) * 4 + t % 4] == vs[n, h, b8]


def test_cache_byte_positions(lib):
    """Codes and scales sit where the header's layout formulas put them, checked byte by byte
    with the formulas written out (keys row-major, values quad-interleaved, scales
    [quad][block][token in quad]) for tokens at every position in a quad and page."""
    rng = np.random.default_rng(31)
    hkv, N = 2, 37
    pages = P.Pages(3, 32, True, spare=1)
    cache = lib.CacheLayer(pages.num_pages, pages.page_size, hkv, k_flags=0, fill=0)
    cache.gscale.fill_(0.02)
    k = S.bf16_round(rng.standard_normal((N, hkv, 128)).astype(np.float32))
    v = S.bf16_round(rng.standard_normal((N, hkv, 128)).astype(np.float32))
    slots = np.concatenate([pages.slots(0, 0, 20), pages.slots(2, 3, 20)])
    lib.quantize_append_kv(cache.struct(), P.to_dev_u16(k), P.to_dev_u16(v), P.to_dev_i32(slots), N)
    torch.cuda.synchronize()
    kc, ks = O.quantize_rows(S.bf16_to_f32(k), np.float32(0.02))
    vc, vs = O.quantize_rows(S.bf16_to_f32(v), np.float32(0.02))
    kd, vd = cache.k_data.cpu().numpy(), cache.v_data.cpu().numpy()
    ksd, vsd = cache.k_scales.cpu().numpy(), cache.v_scales.cpu().numpy()
    ps = pages.page_size
    for n, slot in enumerate(slots):
        pg, t = int(slot) // ps, int(slot) % ps
        for h in range(hkv):
            blk = (pg * hkv + h) * ps                     # tokens before this (page, head) block
            for w in range(16):
                for by in range(4):
                    assert kd[blk * 64 + 64 * t + 4 * w + by] == kc[n, h, 4 * w + by]
                    assert vd[blk * 64 + ((t // 4) * 16 + w) * 16 + (t % 4) * 4 + by] == vc[n, h, 4 * w + by]
            for b8 in range(8):
                assert ksd[blk * 8 + ((t // 4) * 8 + b8) * 4 + t % 4] == ks[n, h, b8]
                assert vsd[blk * 8 + ((t // 4) * 8 + b8) * 4 + t % 4] == vs[n, h, b8]


def test_error_paths_on_gpu_host(lib):
    """Argument errors still come back as status codes with a GPU present."""
    L = lib.Layer()
    with pytest.raises(lib.NvkvError) as e:
        lib.quantize_append_kv(L, None, None, None, 1)
    assert e.value.status == 2


def test_calibrate_rounding_wide_range(lib):
    """s = fl32(sqrt(a)), r = fl32(1/s), g = fl32(A/2688) correctly rounded over absmax values
    spanning many binades (one window, position 1 carries every channel's absmax)."""
    rng = np.random.default_rng(21)
    hkv = 64
    kw = np.zeros((1, 2, hkv, 128), np.float32)
    kw[0, 0] = 1e8                                           # position 0 is excluded
    kw[0, 1] = rng.choice([-1, 1], (hkv, 128)) * np.exp(rng.uniform(-60, 60, (hkv, 128)))
    kbits = S.bf16_round(kw)
    vbits = S.bf16_round(rng.standard_normal((1, 2, hkv, 128)).astype(np.float32) * 3e-30)
    for flags in (0, 1):
        s, r, g = gpu_calibrate(lib, kbits, vbits, hkv, flags)
        so, ro, go = O.calibrate(S.bf16_to_f32(kbits), S.bf16_to_f32(vbits), exclude_pos0=True, k_flags=flags)
        assert np.array_equal(s.cpu().numpy(), so)
        assert np.array_equal(r.cpu().numpy(), ro)
        assert np.array_equal(g.cpu().numpy().view(np.uint32), go.view(np.uint32))


def test_decode_cross_workgroup_merge_stress(lib):
    """The last-arriving workgroup merges the splits through device-coherent stores/loads and a
    self-resetting counter: many calls that interleave split counts on one workspace must give
    bitwise-repeatable outputs (the merge order is fixed) that match the oracle."""
    c, k, v, kw, vw, q = P.workload("layer")
    flags = 1
    s, r, g = gpu_calibrate(lib, kw, vw, c["hkv"], flags)
    so, ro, go, kc, ks, vc, vs = oracle_layer(k, v, kw, vw, flags)
    pages = P.Pages(c["B"], c["T"], True)
    cache = gpu_fill_cache(lib, k, v, c["hkv"], flags, pages, s, r, g)
    seq = [c["T"], 2000, 1500, 77]
    ref, vmax = oracle_decode(q, so, flags, kc, ks, vc, vs, go, seq, c["hkv"])
    B, Hq = q.shape[0], q.shape[1]
    wsb = max(lib.decode_workspace_bytes(B, Hq, c["hkv"], c["T"], sp) for sp in (32, 64, 128, 256))
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    qd, tab, lens = P.to_dev_u16(q), P.to_dev_i32(pages.table), P.to_dev_i32(np.asarray(seq))
    first = {}
    for it in range(25):
        for sp in (32, 256, 64, 128):
            out = torch.empty((B, Hq, 128), dtype=torch.float32, device="cuda")
            lib.decode_attention_nvfp4(cache.struct(), qd, B, Hq, tab, pages.table.shape[1], lens, c["T"],
                                       P.sm_scale(), out, ws, wsb, sp)
            got = out.cpu().numpy()
            if sp not in first:
                first[sp] = got
                assert_close(got.astype(np.float64), ref, vmax, seq)
            else:
                assert np.array_equal(got, first[sp]), f"split {sp}, call {it}: output changed"
