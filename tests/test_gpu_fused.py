"""GPU parity of the fused decode step (decode_append_attention_nvfp4): the new token of each
sequence is quantised into the cache and attended in the same launch.

* cache bytes after the call: bit-exact against the oracle's codes and scales for every row,
  and byte-identical to what quantize_append_kv writes for the same token;
* output: the oracle's attention over [0, n) including the new token, to the decode
  tolerance (max |err| <= 1e-3 max|V_hat|, per-row relative L2 <= 1e-4);
* the stale content of the new token's slot is never read (the slot is pre-filled with a
  different token before the call);
* every split size, ragged lengths (n = 0, 1, page and split boundaries), bf16 keys, an
  out-of-range page for the new token, MSE-searched key scales (the new token's search runs
  on four lanes per block inside the decode launch).
"""
import numpy as np
import pytest
import torch

from oracle import nvfp4_oracle as O
from synth import kv_inputs as S
from tests import _pipeline as P
from tests.test_gpu_parity import (FLAG_SETS, MSE, MSE_FLAG_SETS, assert_close, gpu_calibrate, gpu_fill_cache, oracle_decode,
                                   oracle_layer)

pytestmark = pytest.mark.gpu


def gpu_decode_append(nk, cache, q, k_new, v_new, pages, seq_lens, max_seq_len, split_tokens=0, table=None):
    B, Hq = q.shape[0], q.shape[1]
    out = torch.full((B, Hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    wsb = nk.decode_workspace_bytes(B, Hq, cache.hkv, max_seq_len, split_tokens)
    ws = torch.zeros(max(wsb, 256), dtype=torch.uint8, device="cuda")
    tab = pages.table if table is None else table
    nk.decode_append_attention_nvfp4(cache.struct(), P.to_dev_u16(q), P.to_dev_u16(k_new), P.to_dev_u16(v_new), B,
                                     Hq, P.to_dev_i32(tab), tab.shape[1], P.to_dev_i32(np.asarray(seq_lens)),
                                     max_seq_len, P.sm_scale(), out, ws, wsb, split_tokens)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def spoil_slots(nk, cache, pages, seq_lens, hkv, seed):
    """Overwrite the slot of position n-1 of every sequence with an unrelated token."""
    rng = np.random.default_rng(seed)
    slots = np.array([pages.slots(b, n - 1, n)[0] for b, n in enumerate(seq_lens) if n > 0], np.int32)
    if len(slots) == 0:
        return
    junk = S.bf16_round((rng.standard_normal((len(slots), hkv, 128)) * 7).astype(np.float32))
    nk.quantize_append_kv(cache.struct(), P.to_dev_u16(junk), P.to_dev_u16(junk[:, ::-1].copy()),
                          P.to_dev_i32(slots), len(slots))
    torch.cuda.synchronize()


def new_rows(k, v, seq_lens):
    """The new token's bf16 rows of each sequence ([B][Hkv][128]; zeros where n = 0)."""
    B, hkv = k.shape[0], k.shape[2]
    kn = np.zeros((B, hkv, 128), np.uint16)
    vn = np.zeros((B, hkv, 128), np.uint16)
    for b, n in enumerate(seq_lens):
        if n > 0:
            kn[b], vn[b] = k[b, n - 1], v[b, n - 1]
    return kn, vn


def check_cache_rows(cache, pages, hkv, kc, ks, vc, vs, seq_lens, k_bf16=None):
    kd = cache.k_data.cpu().numpy()
    ksd = cache.k_scales.cpu().numpy() if k_bf16 is None else None
    vd, vsd = cache.v_data.cpu().numpy(), cache.v_scales.cpu().numpy()
    for b, n in enumerate(seq_lens):
        if n == 0:
            continue
        if k_bf16 is None:
            gc, gs = P.rows_from_cache_vec(kd, ksd, pages, hkv, b, n)
            assert np.array_equal(gc, kc[b, :n]) and np.array_equal(gs, ks[b, :n]), f"K rows differ, seq {b}"
        else:
            assert np.array_equal(P.bf16_rows_from_cache(kd, pages, hkv, b, n), k_bf16[b, :n])
        gc, gs = P.rows_from_cache_vec(vd, vsd, pages, hkv, b, n, values=True)
        assert np.array_equal(gc, vc[b, :n]) and np.array_equal(gs, vs[b, :n]), f"V rows differ, seq {b}"


@pytest.mark.parametrize("name,flags", [(n, f) for n in ("tiny", "layer") for f in FLAG_SETS]
                         + [("tiny", f) for f in MSE_FLAG_SETS] + [("layer", MSE | 1)])
@pytest.mark.parametrize("paged", [False, True])
def test_decode_append_parity(lib, name, flags, paged):
    c, k, v, kw, vw, q = P.workload(name)
    hkv, T, B = c["hkv"], c["T"], c["B"]
    s, r, g = gpu_calibrate(lib, kw, vw, hkv, flags)
    so, ro, go, kc, ks, vc, vs = oracle_layer(k, v, kw, vw, flags)
    pages = P.Pages(B, T, paged)
    cache = gpu_fill_cache(lib, k, v, hkv, flags, pages, s, r, g)
    seq = [T] * B
    kn, vn = new_rows(k, v, seq)
    ref, vmax = oracle_decode(q, so, flags, kc, ks, vc, vs, go, seq, hkv)
    for split in (0, 32, 96, P.ceil_to(T, 32)):
        spoil_slots(lib, cache, pages, seq, hkv, seed=split)
        got = gpu_decode_append(lib, cache, q, kn, vn, pages, seq, T, split)
        assert_close(got, ref, vmax, seq)
        check_cache_rows(cache, pages, hkv, kc, ks, vc, vs, seq)


@pytest.mark.parametrize("paged", [False, True])
def test_decode_append_ragged_lengths(lib, paged):
    c, k, v, kw, vw, q = P.workload("layer", T=300)
    hkv = c["hkv"]
    flags = 3
    s, r, g = gpu_calibrate(lib, kw, vw, hkv, flags)
    so, ro, go, kc, ks, vc, vs = oracle_layer(k, v, kw, vw, flags)
    pages = P.Pages(c["B"], c["T"], paged)
    cache = gpu_fill_cache(lib, k, v, hkv, flags, pages, s, r, g)
    for seq in ([0, 1, 16, 17], [33, 32, 300, 2], [65, 64, 97, 129], [299, 0, 256, 257]):
        kn, vn = new_rows(k, v, seq)
        ref, vmax = oracle_decode(q, so, flags, kc, ks, vc, vs, go, seq, hkv)
        for split in (0, 32, 64, 320):
            spoil_slots(lib, cache, pages, seq, hkv, seed=split + sum(seq))
            got = gpu_decode_append(lib, cache, q, kn, vn, pages, seq, 300, split)
            assert_close(got, ref, vmax, seq)
            check_cache_rows(cache, pages, hkv, kc, ks, vc, vs, seq)


def test_decode_append_matches_separate_calls(lib):
    """Cache bytes after the fused call equal those after quantize_append_kv of the same
    token; the outputs agree with the separate decode to within summation order."""
    c, k, v, kw, vw, q = P.workload("layer")
    hkv, T, B = c["hkv"], c["T"], c["B"]
    flags = 1
    s, r, g = gpu_calibrate(lib, kw, vw, hkv, flags)
    pages = P.Pages(B, T, True)
    k_prev, v_prev = k[:, :T - 1], v[:, :T - 1]
    fused = gpu_fill_cache(lib, k_prev, v_prev, hkv, flags, pages, s, r, g)
    sep = gpu_fill_cache(lib, k_prev, v_prev, hkv, flags, pages, s, r, g)
    seq = [T] * B
    kn, vn = new_rows(k, v, seq)
    out_f = gpu_decode_append(lib, fused, q, kn, vn, pages, seq, T)
    slots = np.array([pages.slots(b, T - 1, T)[0] for b in range(B)], np.int32)
    lib.quantize_append_kv(sep.struct(), P.to_dev_u16(kn), P.to_dev_u16(vn), P.to_dev_i32(slots), B)
    from tests.test_gpu_parity import gpu_decode
    out_s = gpu_decode(lib, sep, q, pages, seq, T)
    for a_, b_ in ((fused.k_data, sep.k_data), (fused.k_scales, sep.k_scales), (fused.v_data, sep.v_data),
                   (fused.v_scales, sep.v_scales)):
        assert torch.equal(a_, b_)
    assert np.max(np.abs(out_f - out_s)) <= 1e-5 * np.max(np.abs(out_s))


@pytest.mark.parametrize("paged", [False, True])
def test_decode_append_bf16_keys(lib, paged):
    c, k, v, kw, vw, q = P.workload("layer", T=700)
    hkv = c["hkv"]
    s, r, g = gpu_calibrate(lib, kw, vw, hkv, 0)
    so, ro, go, kc, ks, vc, vs = oracle_layer(k, v, kw, vw, 0)
    pages = P.Pages(c["B"], c["T"], paged)
    cache = gpu_fill_cache(lib, k, v, hkv, 0, pages, s, r, g, k_fmt=0)
    for seq in ([700, 700, 700, 700], [1, 0, 333, 97]):
        kn, vn = new_rows(k, v, seq)
        ref, vmax = oracle_decode(q, so, 0, kc, ks, vc, vs, go, seq, hkv, k_bf16=k)
        for split in (0, 64, 704):
            spoil_slots(lib, cache, pages, seq, hkv, seed=split)
            got = gpu_decode_append(lib, cache, q, kn, vn, pages, seq, 700, split)
            assert_close(got, ref, vmax, seq)
            check_cache_rows(cache, pages, hkv, kc, ks, vc, vs, seq, k_bf16=k)


def test_decode_append_out_of_range_page(lib):
    """A new token whose page index is out of range writes nothing and is left out of the
    attention (as the separate append, which skips the slot, and decode, which masks the
    page, would do)."""
    c, k, v, kw, vw, q = P.workload("layer", T=161)
    hkv, B = c["hkv"], c["B"]
    flags = 1
    s, r, g = gpu_calibrate(lib, kw, vw, hkv, flags)
    so, ro, go, kc, ks, vc, vs = oracle_layer(k, v, kw, vw, flags)
    pages = P.Pages(B, 161, True)
    cache = gpu_fill_cache(lib, k[:, :160], v[:, :160], hkv, flags, pages, s, r, g)
    before = [t.clone() for t in (cache.k_data, cache.k_scales, cache.v_data, cache.v_scales)]
    table = pages.table.copy()
    table[:, 10] = pages.num_pages + 5                 # page of position 160 (page 10) is invalid
    seq = [161] * B
    kn, vn = new_rows(k, v, seq)
    got = gpu_decode_append(lib, cache, q, kn, vn, pages, seq, 161, 0, table=table)
    for t0, t1 in zip(before, (cache.k_data, cache.k_scales, cache.v_data, cache.v_scales)):
        assert torch.equal(t0, t1)
    ref, vmax = oracle_decode(q, so, flags, kc, ks, vc, vs, go, [160] * B, hkv)
    assert_close(got, ref, vmax, [160] * B)
