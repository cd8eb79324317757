"""Shared GPU-test plumbing: seeded inputs -> native library calls, and the documented cache
layout (include/nvfp4kv.h) mapped back to logical per-token rows for comparison with the
oracle.  Nothing here computes any part of the method."""
from __future__ import annotations

import math

import numpy as np
import torch

from synth import kv_inputs as S

HD = 128


def ceil_to(x: int, m: int) -> int:
    return (x + m - 1) // m * m


class Pages:
    """Page table for B sequences of capacity `cap` tokens: contiguous (one page per sequence)
    or paged with 16-token pages in a seeded shuffled order."""

    def __init__(self, B: int, cap: int, paged: bool, seed: int = 7, spare: int = 3):
        self.B = B
        if paged:
            self.page_size = 16
            self.pages_per_seq = ceil_to(max(cap, 1), 16) // 16
            self.num_pages = B * self.pages_per_seq + spare
            perm = np.random.default_rng(seed).permutation(self.num_pages)[: B * self.pages_per_seq]
            self.table = perm.reshape(B, self.pages_per_seq).astype(np.int32)
        else:
            self.page_size = ceil_to(max(cap, 1), 16)
            self.pages_per_seq = 1
            self.num_pages = B
            self.table = np.arange(B, dtype=np.int32).reshape(B, 1)

    def slots(self, b: int, t0: int, t1: int) -> np.ndarray:
        t = np.arange(t0, t1)
        return (self.table[b, t // self.page_size] * self.page_size + t % self.page_size).astype(np.int32)

    def locate(self, b: int, t: int):
        return int(self.table[b, t // self.page_size]), t % self.page_size


def codes_view(codes_u8: np.ndarray, pages: Pages, hkv: int, values: bool) -> np.ndarray:
    """Codes of one layer as [page][head][token in page][64] (header layout: keys row-major,
    values quad-interleaved: word w of token t at ((t/4)*16 + w)*16 + (t%4)*4)."""
    ps = pages.page_size
    if not values:
        return codes_u8.reshape(pages.num_pages, hkv, ps, 64)
    q = codes_u8.reshape(pages.num_pages, hkv, ps // 4, 16, 4, 4)        # [pg][h][quad][w][j][byte]
    return q.transpose(0, 1, 2, 4, 3, 5).reshape(pages.num_pages, hkv, ps, 64)


def rows_from_cache(codes_u8: np.ndarray, scales_u8: np.ndarray, pages: Pages, hkv: int, b: int, T: int,
                    values: bool = False):
    """Logical rows of sequence b, tokens [0, T): codes [T][Hkv][64], scales [T][Hkv][8]."""
    ps = pages.page_size
    codes = codes_view(codes_u8, pages, hkv, values)
    sc = scales_u8.reshape(pages.num_pages, hkv, ps // 4, 8, 4)
    out_c = np.empty((T, hkv, 64), np.uint8)
    out_s = np.empty((T, hkv, 8), np.uint8)
    for t in range(T):
        pg, off = pages.locate(b, t)
        out_c[t] = codes[pg, :, off]
        out_s[t] = sc[pg, :, off // 4, :, off % 4]
    return out_c, out_s


def rows_from_cache_vec(codes_u8: np.ndarray, scales_u8: np.ndarray, pages: Pages, hkv: int, b: int, T: int,
                        values: bool = False):
    """Vectorised rows_from_cache for long sequences."""
    ps = pages.page_size
    codes = codes_view(codes_u8, pages, hkv, values)
    sc = scales_u8.reshape(pages.num_pages, hkv, ps // 4, 8, 4)
    t = np.arange(T)
    pg = pages.table[b, t // ps]
    off = t % ps
    c = codes[pg, :, off]                         # [T][Hkv][64]
    s = sc[pg, :, off // 4, :, off % 4]          # [T][Hkv][8]
    return c, s


def bf16_rows_from_cache(data_u8: np.ndarray, pages: Pages, hkv: int, b: int, T: int) -> np.ndarray:
    ps = pages.page_size
    rows = data_u8.view(np.uint16).reshape(pages.num_pages, hkv, ps, HD)
    t = np.arange(T)
    return rows[pages.table[b, t // ps], :, t % ps]


def to_dev_u16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def to_dev_i32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def workload(name: str, layer: int = 0, T: int | None = None, B: int | None = None, sink: bool = True):
    """bf16 K, V [B][T][Hkv][128], calibration windows, and queries for a named workload."""
    c = dict(S.CONFIGS[name])
    if T is not None:
        c["T"] = T
    if B is not None:
        c["B"] = B
    k = np.stack([S.make_keys(c["kind"], c["cfg"], layer, b, c["T"], c["hkv"], sink=sink) for b in range(c["B"])])
    v = np.stack([S.make_values(c["cfg"], layer, b, c["T"], c["hkv"]) for b in range(c["B"])])
    kw, vw = S.make_calib_windows(c["kind"], c["cfg"], layer, 4, c["Tw"], c["hkv"], sink=sink)
    q = S.make_queries(c["cfg"], layer, c["B"], c["hq"])
    return c, k, v, kw, vw, q


def sm_scale() -> float:
    return 1.0 / math.sqrt(HD)
