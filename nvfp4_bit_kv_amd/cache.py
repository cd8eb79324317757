"""Device buffers of one cache layer (torch allocations) and the matching nvkv_layer struct.

PyTorch only provides memory here; every computation happens in the native library.
"""
from __future__ import annotations

import torch

from . import _native as N


class CacheLayer:
    """Pages of NVFP4 (or BF16-key) cache for one layer plus its calibration state.

    Layout (include/nvfp4kv.h): codes u8 [pages][Hkv][page_size][64]; scales u8
    [pages][Hkv][page_size/4][8][4]; BF16 keys u16 [pages][Hkv][page_size][128]."""

    def __init__(self, num_pages: int, page_size: int, num_kv_heads: int, k_fmt: int = N.FMT_NVFP4,
                 v_fmt: int = N.FMT_NVFP4, k_flags: int = 0, device: str = "cuda", fill: int = 0):
        self.num_pages, self.page_size, self.hkv = num_pages, page_size, num_kv_heads
        self.k_fmt, self.v_fmt, self.k_flags = k_fmt, v_fmt, k_flags
        rows = num_pages * num_kv_heads * page_size
        u8 = dict(dtype=torch.uint8, device=device)
        if k_fmt == N.FMT_NVFP4:
            self.k_data = torch.full((rows * 64,), fill, **u8)
            self.k_scales = torch.full((rows * 8,), fill, **u8)
        else:
            self.k_data = torch.full((rows * 256,), fill, **u8)
            self.k_scales = None
        self.v_data = torch.full((rows * 64,), fill, **u8)
        self.v_scales = torch.full((rows * 8,), fill, **u8)
        f32 = dict(dtype=torch.float32, device=device)
        self.smooth = torch.ones((num_kv_heads, N.HEAD_DIM), **f32)
        self.inv_smooth = torch.ones((num_kv_heads, N.HEAD_DIM), **f32)
        self.gscale = torch.ones((2,), **f32)
        # KLT key basis [Hkv][128][128] (identity until calibrated); only with N.K_KLT
        self.basis = None
        if k_flags & N.K_KLT:
            self.basis = torch.eye(N.HEAD_DIM, **f32).repeat(num_kv_heads, 1, 1).contiguous()

    def struct(self) -> N.Layer:
        L = N.Layer()
        L.num_kv_heads, L.head_dim = self.hkv, N.HEAD_DIM
        L.page_size, L.num_pages = self.page_size, self.num_pages
        L.k_fmt, L.v_fmt, L.k_flags, L.reserved = self.k_fmt, self.v_fmt, self.k_flags, 0
        L.k_data, L.v_data = self.k_data.data_ptr(), self.v_data.data_ptr()
        L.k_scales = self.k_scales.data_ptr() if self.k_scales is not None else None
        L.v_scales = self.v_scales.data_ptr()
        L.k_smooth, L.k_inv_smooth = self.smooth.data_ptr(), self.inv_smooth.data_ptr()
        L.global_scale = self.gscale.data_ptr()
        L.k_basis = self.basis.data_ptr() if self.basis is not None else None
        return L
