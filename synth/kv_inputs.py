"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no arithmetic of the method itself (no transform, no quantisation, no
attention): it only draws K/V/query tensors with the shapes and value structure of the
workloads and rounds them to bf16.  The CPU oracle and the GPU path both consume what it
returns; neither is imported here.

Value structure (stand-ins for the post-RoPE cache of W4A4 Qwen3-8B evaluated on WikiText
and C4 windows in the rstation.ai post "NVFP4 attention cache on W4A4 Qwen3-8B ...", whose
weights and datasets are not available):
  * "outlier"   K ~ N(0,1) with 4 seeded channels per KV head scaled x20.
  * "lognormal" K ~ sigma_{h,j} N(0,1), sigma_{h,j} ~ LogNormal(0, 1) per (head, channel),
                then a NeoX rotary embedding (base 1e6, position = token index) so that the
                rows look post-RoPE.
  * position 0 of every sequence / window is a sink: its key row is scaled x40 (the
    u/krylov_schur thread on rstation.ai reports 30-50x RMS norms for Qwen3-8B sink tokens).
  * V ~ N(0,1); queries ~ N(0,1).
Seeds: seed = ((cfg*16 + role)*64 + layer)*64 + index, roles 0 K, 1 V, 2 query,
3 channel structure, 4 query blocks (causal prefill attention), 10..13 calibration windows
0..3.
"""
from __future__ import annotations

import numpy as np

HEAD_DIM = 128
ROLE_K, ROLE_V, ROLE_Q, ROLE_CHAN = 0, 1, 2, 3
ROLE_QBLK = 4
ROLE_WIN0 = 10


def seed_of(cfg: int, role: int, layer: int = 0, index: int = 0) -> int:
    return ((cfg * 16 + role) * 64 + layer) * 64 + index


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returns uint16 bit patterns."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    return r


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32)


def channel_scales(kind: str, cfg: int, layer: int, hkv: int, d: int = HEAD_DIM) -> np.ndarray:
    """Per (KV head, channel) key scale, fixed per layer (shared by cache and calibration)."""
    rng = np.random.Generator(np.random.PCG64(seed_of(cfg, ROLE_CHAN, layer)))
    if kind == "outlier":
        sc = np.ones((hkv, d), dtype=np.float64)
        for h in range(hkv):
            idx = rng.choice(d, size=4, replace=False)
            sc[h, idx] = 20.0
        return sc
    if kind == "lognormal":
        return rng.lognormal(mean=0.0, sigma=1.0, size=(hkv, d))
    if kind == "none":
        return np.ones((hkv, d), dtype=np.float64)
    raise ValueError(kind)


def neox_rope(x: np.ndarray, positions: np.ndarray, base: float = 1e6) -> np.ndarray:
    """Rotate channel pairs (j, j+64) by angle pos * base^(-2j/128) (input generation)."""
    d = x.shape[-1]
    half = d // 2
    inv = base ** (-np.arange(half, dtype=np.float64) * 2.0 / d)
    ang = positions[:, None].astype(np.float64) * inv[None, :]          # [T][64]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1 = x[..., :half]
    x2 = x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def make_keys(kind: str, cfg: int, layer: int, index: int, T: int, hkv: int,
              sink: bool = True, role: int = ROLE_K, d: int = HEAD_DIM) -> np.ndarray:
    """One sequence (or window) of keys, bf16 bits [T][Hkv][D]."""
    rng = np.random.Generator(np.random.PCG64(seed_of(cfg, role, layer, index)))
    x = rng.standard_normal((T, hkv, d)) * channel_scales(kind, cfg, layer, hkv, d)[None]
    if kind == "lognormal":
        x = neox_rope(x, np.arange(T))
    if sink and T > 0:
        x[0] *= 40.0
    return bf16_round(x.astype(np.float32))


def make_values(cfg: int, layer: int, index: int, T: int, hkv: int, role: int = ROLE_V,
                d: int = HEAD_DIM) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed_of(cfg, role, layer, index)))
    return bf16_round(rng.standard_normal((T, hkv, d)).astype(np.float32))


def make_queries(cfg: int, layer: int, B: int, hq: int, d: int = HEAD_DIM) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed_of(cfg, ROLE_Q, layer)))
    return bf16_round(rng.standard_normal((B, hq, d)).astype(np.float32))


def make_query_block(cfg: int, layer: int, B: int, Tq: int, hq: int, d: int = HEAD_DIM) -> np.ndarray:
    """Queries of Tq consecutive positions per sequence, bf16 bits [B][Tq][Hq][D], N(0,1)."""
    rng = np.random.Generator(np.random.PCG64(seed_of(cfg, ROLE_QBLK, layer)))
    return bf16_round(rng.standard_normal((B, Tq, hq, d)).astype(np.float32))


def make_calib_windows(kind: str, cfg: int, layer: int, W: int, Tw: int, hkv: int,
                       sink: bool = True):
    """W calibration windows of keys and values, bf16 bits [W][Tw][Hkv][D] each."""
    k = np.stack([make_keys(kind, cfg, layer, w, Tw, hkv, sink=sink, role=ROLE_WIN0 + w)
                  for w in range(W)])
    v = np.stack([make_values(cfg, layer, w, Tw, hkv, role=ROLE_WIN0 + 4 + w)
                  for w in range(W)])
    return k, v


# Workload table: shapes of the five configurations (tiny reference, one Qwen3-8B layer,
# the 36-layer cache decode step, prefill append, long-context decode).
CONFIGS = {
    "tiny":    dict(cfg=0, layers=1, B=1, T=256, hkv=1, hq=4, kind="outlier", Tw=256),
    "layer":   dict(cfg=1, layers=1, B=4, T=2304, hkv=8, hq=32, kind="lognormal", Tw=2048),
    "step36":  dict(cfg=2, layers=36, B=4, T=2304, hkv=8, hq=32, kind="lognormal", Tw=2048),
    "prefill": dict(cfg=3, layers=36, B=16, T=8192, hkv=8, hq=32, kind="lognormal", Tw=2048),
    "long":    dict(cfg=4, layers=36, B=64, T=32768, hkv=8, hq=32, kind="outlier", Tw=2048),
}


# ----------------------------------------------------------------------------------------
# Device-side generation of the same distributions for workloads too large to build on the
# host (seeded torch generator per layer; values differ from the NumPy stream, the
# distribution and structure are the same).
# ----------------------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def make_keys_device(kind: str, cfg: int, layer: int, B: int, T: int, hkv: int, sink: bool = True,
                     role: int = ROLE_K, t_offset: int = 0, seed_index: int = 0, d: int = HEAD_DIM):
    """Keys bf16 [B][T][Hkv][D] on the current GPU; positions t_offset .. t_offset+T-1."""
    torch = _torch()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed_of(cfg, role, layer, seed_index))
    sc = torch.from_numpy(channel_scales(kind, cfg, layer, hkv, d).astype(np.float32)).cuda()
    x = torch.randn((B, T, hkv, d), generator=gen, device="cuda", dtype=torch.float32) * sc
    if kind == "lognormal":
        half = d // 2
        inv = torch.pow(torch.tensor(1e6, dtype=torch.float64),
                        -torch.arange(half, dtype=torch.float64) * 2.0 / d).cuda()
        pos = torch.arange(t_offset, t_offset + T, dtype=torch.float64, device="cuda")
        ang = (pos[:, None] * inv[None, :])
        c = torch.cos(ang).float()[None, :, None, :]
        s = torch.sin(ang).float()[None, :, None, :]
        x1, x2 = x[..., :half], x[..., half:]
        x = torch.cat([x1 * c - x2 * s, x2 * c + x1 * s], dim=-1)
    if sink and t_offset == 0 and T > 0:
        x[:, 0] *= 40.0
    return x.to(torch.bfloat16)


def make_values_device(cfg: int, layer: int, B: int, T: int, hkv: int, role: int = ROLE_V,
                       seed_index: int = 0, d: int = HEAD_DIM):
    torch = _torch()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed_of(cfg, role, layer, seed_index))
    return torch.randn((B, T, hkv, d), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)


def make_queries_device(cfg: int, layer: int, B: int, hq: int, d: int = HEAD_DIM):
    torch = _torch()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed_of(cfg, ROLE_Q, layer))
    return torch.randn((B, hq, d), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)


def make_query_block_device(cfg: int, layer: int, B: int, Tq: int, hq: int, d: int = HEAD_DIM):
    torch = _torch()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed_of(cfg, ROLE_QBLK, layer))
    return torch.randn((B, Tq, hq, d), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
