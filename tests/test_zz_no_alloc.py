"""GPU check of the allocation-free fused decode step
(nvkv_decode_append_attention_nvfp4_noalloc) against the workspace form
(nvkv_decode_append_attention_nvfp4), through the C ABI.

Both run the same kernels with the same split plan and a fixed merge order, so the outputs
and the cache bytes they write must be identical.  Two calls in a row share the static
scratch, the second with a smaller input (fewer sequences, a shorter context), then one with
a single split per sequence (no scratch use), then one with many splits.
"""
import numpy as np
import pytest
import torch

from tests import _pipeline as P
from tests.test_gpu_fused import new_rows, spoil_slots
from tests.test_gpu_parity import gpu_calibrate, gpu_fill_cache

pytestmark = pytest.mark.gpu


def both_forms(lib, name, T, B, flags, split_tokens):
    c, k, v, kw, vw, q = P.workload(name, T=T, B=B, sink=False)
    hkv, Hq = c["hkv"], c["hq"]
    s, r, g = gpu_calibrate(lib, kw, vw, hkv, flags)
    pages = P.Pages(B, T, True)
    seq = [T] * B
    kn, vn = new_rows(k, v, seq)
    ca = gpu_fill_cache(lib, k, v, hkv, flags, pages, s, r, g)
    cb = gpu_fill_cache(lib, k, v, hkv, flags, pages, s, r, g)
    spoil_slots(lib, ca, pages, seq, hkv, seed=3)
    spoil_slots(lib, cb, pages, seq, hkv, seed=3)
    qd, knd, vnd = P.to_dev_u16(q), P.to_dev_u16(kn), P.to_dev_u16(vn)
    tab, lens = P.to_dev_i32(pages.table), P.to_dev_i32(np.asarray(seq))
    wsb = lib.decode_workspace_bytes(B, Hq, hkv, T, split_tokens)
    ws = torch.zeros(max(wsb, 256), dtype=torch.uint8, device="cuda")
    out_ws = torch.full((B, Hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    out_na = torch.full((B, Hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    lib.decode_append_attention_nvfp4(ca.struct(), qd, knd, vnd, B, Hq, tab, pages.table.shape[1], lens, T,
                                      P.sm_scale(), out_ws, ws, wsb, split_tokens)
    lib.decode_append_attention_nvfp4_noalloc(cb.struct(), qd, knd, vnd, B, Hq, tab, pages.table.shape[1], lens, T,
                                              P.sm_scale(), out_na, split_tokens)
    torch.cuda.synchronize()
    assert torch.all(torch.isfinite(out_na))
    assert torch.equal(out_na, out_ws), float((out_na - out_ws).abs().max())
    for x, y in ((ca.k_data, cb.k_data), (ca.k_scales, cb.k_scales), (ca.v_data, cb.v_data),
                 (ca.v_scales, cb.v_scales)):
        assert torch.equal(x, y)
    return out_na


def test_noalloc_matches_workspace_form_two_calls(lib):
    # a Qwen3-8B layer (4 x 2304, several splits per sequence), then a smaller call on the same
    # scratch (2 x 700), then one split per sequence, then many splits
    both_forms(lib, "layer", 2304, 4, 1, 0)
    both_forms(lib, "layer", 700, 2, 3, 0)
    both_forms(lib, "layer", 700, 2, 1, 704)
    both_forms(lib, "layer", 2304, 4, 1, 32)
    both_forms(lib, "tiny", 256, 1, 3, 32)
