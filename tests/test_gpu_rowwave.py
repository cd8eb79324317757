"""GPU parity of the comparison append layout (one wavefront per (token, KV head) row,
libnvkv_bench.so's nvkvb_quantize_append_rowwave): its cache bytes equal the library's
quantize_append_kv (one lane per 16-element block) and the oracle's, with plain, smoothed and
smoothed + Hadamard keys, a ragged token count, shuffled pages, skipped and out-of-range slots."""
import ctypes
import os

import numpy as np
import pytest
import torch

from oracle import nvfp4_oracle as O
from synth import kv_inputs as S
from tests import _pipeline as P

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def blib(lib):
    path = os.path.join(ROOT, "nvfp4_bit_kv_amd", "libnvkv_bench.so")
    b = ctypes.CDLL(path)
    vp = ctypes.c_void_p
    b.nvkvb_quantize_append_rowwave.argtypes = [ctypes.POINTER(lib.Layer), vp, vp, vp, ctypes.c_int32, vp]
    b.nvkvb_quantize_append_rowwave.restype = ctypes.c_int
    return b


def calibrated_cache(lib, pages, hkv, flags, rng):
    cache = lib.CacheLayer(pages.num_pages, pages.page_size, hkv, k_flags=flags, fill=0xA5)
    sm = (0.5 + rng.random((hkv, 128))).astype(np.float32)
    cache.smooth.copy_(torch.from_numpy(sm))
    cache.inv_smooth.copy_(torch.from_numpy((np.float32(1.0) / sm).astype(np.float32)))
    cache.gscale.copy_(torch.tensor([0.0021, 0.0017], dtype=torch.float32))
    return cache


@pytest.mark.parametrize("flags,hkv", [(0, 2), (1, 8), (3, 8), (3, 1)])
def test_rowwave_bytes_equal_library_and_oracle(lib, blib, flags, hkv):
    rng = np.random.default_rng(100 + flags + hkv)
    N = 77
    pages = P.Pages(3, 40, True, spare=2)
    slots = np.concatenate([pages.slots(0, 0, 30), pages.slots(1, 3, 40), pages.slots(2, 0, N - 67)])
    slots[5] = -1                                            # skipped
    slots[11] = pages.num_pages * pages.page_size            # out of range: skipped
    k = S.bf16_round((rng.standard_normal((N, hkv, 128)) * np.exp(rng.uniform(-3, 2, (N, hkv, 1))))
                     .astype(np.float32))
    v = S.bf16_round(rng.standard_normal((N, hkv, 128)).astype(np.float32))
    a = calibrated_cache(lib, pages, hkv, flags, rng)
    b = lib.CacheLayer(pages.num_pages, pages.page_size, hkv, k_flags=flags, fill=0xA5)
    for name in ("smooth", "inv_smooth", "gscale"):
        getattr(b, name).copy_(getattr(a, name))
    kd, vd, sd = P.to_dev_u16(k), P.to_dev_u16(v), P.to_dev_i32(slots)
    lib.quantize_append_kv(a.struct(), kd, vd, sd, N)
    Lb = b.struct()
    st = blib.nvkvb_quantize_append_rowwave(ctypes.byref(Lb), kd.data_ptr(), vd.data_ptr(), sd.data_ptr(), N,
                                            torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    for name in ("k_data", "k_scales", "v_data", "v_scales"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name
    # and the oracle's bytes, token by token through the slots
    r = a.inv_smooth.cpu().numpy()
    g = a.gscale.cpu().numpy()
    y = O.key_transform(S.bf16_to_f32(k)[None], r[None, None] if flags & 1 else None, flags)[0]
    kc, ks = O.quantize_rows(y, g[0])
    vc, vs = O.quantize_rows(S.bf16_to_f32(v), g[1])
    got = {name: getattr(b, name).cpu().numpy() for name in ("k_data", "k_scales", "v_data", "v_scales")}
    ps = pages.page_size
    for n, slot in enumerate(slots):
        if slot < 0 or slot >= pages.num_pages * ps:
            continue
        pg, t = int(slot) // ps, int(slot) % ps
        for h in range(hkv):
            blk = (pg * hkv + h) * ps
            assert np.array_equal(got["k_data"][(blk + t) * 64:(blk + t + 1) * 64], kc[n, h]), (n, h)
            vw = [got["v_data"][blk * 64 + ((t // 4) * 16 + w) * 16 + (t % 4) * 4 + by]
                  for w in range(16) for by in range(4)]
            assert np.array_equal(np.array(vw, dtype=np.uint8), vc[n, h]), (n, h)
            for bl in range(8):
                at = blk * 8 + ((t // 4) * 8 + bl) * 4 + t % 4
                assert got["k_scales"][at] == ks[n, h, bl] and got["v_scales"][at] == vs[n, h, bl], (n, h, bl)
    # the slots that were skipped left their fill untouched
    used = np.zeros(pages.num_pages * ps, dtype=bool)
    used[slots[(slots >= 0) & (slots < pages.num_pages * ps)]] = True
    for sl in np.nonzero(~used)[0][:8]:
        pg, t = int(sl) // ps, int(sl) % ps
        blk = (pg * hkv) * ps
        assert np.all(got["k_data"][(blk + t) * 64:(blk + t + 1) * 64] == 0xA5)
