"""GPU parity of the MSE-searched key block scale (NVKV_K_MSE_SCALE) on constructed corner
blocks, through both key encoders: quantize_append_kv (one lane per block) and the fused
decode step's new-token path (four lanes per block).  Codes and scales bit-exact against
the oracle's quantize_rows_mse; values keep absmax-to-6.

Corner blocks (tensor scale g = 2^-7, so every constructed value is exact in bf16):
* the worked example (6, 5, ..., 5) * g, whose best two scales tie exactly;
* an all-zero block; a block past 7 * 448 * g (only the saturated absmax code qualifies);
* a block whose absmax-to-6 scale underflows to 0 while the smallest E4M3 scale keeps it;
* a block whose absmax code lies outside the search interval and still wins;
* blocks whose absmax is exactly 7 g times an E4M3 value, so that the run holds 17 codes;
* random blocks spanning the E4M3 subnormal scales, clustered blocks and one-outlier blocks;
* tie-heavy blocks: every element a signed E2M1 midpoint times the scale of a code c of the
  search run (times 2^-1, 1 or 2, so that the quotients of the codes c - 8, c and c + 8 land
  on midpoints as well), some of them one bf16 ulp off.

Near-midpoint blocks at a generic tensor scale (smoothed keys ±2^m times per-channel factors
placed 2 to 64 units of 2^-24 off an E2M1 midpoint of an E4M3 scale): the blocks that pass the
append kernel's midpoint screen take one converter pass per candidate scale, the others the
bracketed pass, and both must match the oracle.
"""
import numpy as np
import pytest
import torch

from oracle import nvfp4_oracle as O
from synth import kv_inputs as S
from tests import _pipeline as P

pytestmark = pytest.mark.gpu

G = np.float32(2.0 ** -7)


def corner_rows(hkv: int, n: int, seed: int = 3) -> np.ndarray:
    rng = np.random.default_rng(seed)
    rows = (rng.standard_normal((n, hkv, 128)) * np.exp(rng.uniform(-9, 1, (n, hkv, 8, 1)))
            .repeat(16, axis=-1).reshape(n, hkv, 128) * 0.05).astype(np.float32)
    blocks = rows.reshape(n, hkv, 8, 16)
    blocks[0, 0, 0] = 5.0 * G
    blocks[0, 0, 0, 0] = 6.0 * G                            # worked example with a tie
    blocks[0, 0, 1] = 0.0
    blocks[0, 0, 2] = 7.0 * 448.0 * 1.01 * G                # beyond the largest scale
    blocks[0, 0, 3] = 2.5 * 2.0 ** -9 * G                   # absmax scale underflows
    blocks[0, 0, 4] = 0.5 * 2.0 ** -9 * G
    blocks[0, 0, 4, 0] = 7.5 * 2.0 ** -9 * G                # absmax code outside the interval
    for b, code in ((0, 60), (1, 21)):                     # A = 7 g sigma_c: a run of 17 codes
        sig = float(O.e4m3_decode(code))
        blocks[0, 1, b] = rng.uniform(-6.5, 6.5, 16) * sig * G
        blocks[0, 1, b, 3] = -7.0 * sig * G
    for i in range(1, n):                                   # clustered and one-outlier blocks
        blocks[i, 0, 5] = rng.choice([-1, 1], 16) * (2.5 + 0.3 * rng.random(16)) * G * 40
        blocks[i, 0, 6] = rng.standard_normal(16) * 0.05 * G * 40
        blocks[i, 0, 6, rng.integers(16)] = 3.0 * G * 40
        sig = float(O.e4m3_decode(int(rng.integers(40, 88))))    # normal scale, 4 significant bits
        mids = rng.choice([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], 16) * rng.choice([0.5, 1.0, 2.0], 16)
        ulp = rng.choice([-1, 0, 0, 1], 16) * 2.0 ** -7              # one bf16 ulp at [1, 2), or none
        blocks[i, 0, 7] = rng.choice([-1, 1], 16) * mids * sig * G * (1.0 + ulp)
    return S.bf16_round(rows)


def check_rows(cache, pages, hkv, n_tok, kc, ks, vc, vs, b=0):
    gc, gs = P.rows_from_cache_vec(cache.k_data.cpu().numpy(), cache.k_scales.cpu().numpy(), pages, hkv, b, n_tok)
    assert np.array_equal(gs, ks), np.argwhere(gs != ks)[:5]
    assert np.array_equal(gc, kc)
    gc, gs = P.rows_from_cache_vec(cache.v_data.cpu().numpy(), cache.v_scales.cpu().numpy(), pages, hkv, b, n_tok,
                                   values=True)
    assert np.array_equal(gs, vs) and np.array_equal(gc, vc)


def test_mse_corner_blocks_append_kernel(lib):
    hkv, N = 2, 200
    kbits = corner_rows(hkv, N)
    vbits = kbits[::-1].copy()
    k32, v32 = S.bf16_to_f32(kbits), S.bf16_to_f32(vbits)
    kc, ks = O.quantize_rows_mse(k32, G)
    vc, vs = O.quantize_rows(v32, G)
    # the constructed blocks decide as derived by hand
    assert list(ks[0, 0, :5]) == [0x3D, 0, 126, 1, 1]
    grid = np.array([float(O.e4m3_decode(c)) for c in range(1, 127)])
    for b in (0, 1):
        A = float(np.max(np.abs(k32[0, 1, 16 * b:16 * b + 16])))
        assert np.count_nonzero((A >= 1.75 * G * grid) & (A <= 7.0 * G * grid)) == 17
    assert np.any(ks != O.quantize_rows(k32, G)[1])
    pages = P.Pages(1, N, True)
    cache = lib.CacheLayer(pages.num_pages, pages.page_size, hkv, k_flags=lib.K_MSE_SCALE)
    cache.gscale.copy_(torch.tensor([G, G]))
    lib.quantize_append_kv(cache.struct(), P.to_dev_u16(kbits), P.to_dev_u16(vbits),
                           P.to_dev_i32(pages.slots(0, 0, N)), N)
    torch.cuda.synchronize()
    check_rows(cache, pages, hkv, N, kc, ks, vc, vs)


def screen_distance(y: np.ndarray, g: np.float32) -> np.ndarray:
    """Distance, in units of the last place, of fl(|y| / g) from the nearest number with 7
    significant bits (the quantity the append kernel's midpoint screen bounds from below)."""
    w = (np.abs(y).astype(np.float64) / np.float64(g)).astype(np.float32)
    low = w.view(np.uint32) & np.uint32(0x1FFFF)
    return np.minimum(low, np.uint32(0x20000) - low)


def test_mse_near_midpoints_append_kernel(lib):
    hkv, N = 8, 128
    g = np.float32(0.0021)
    rng = np.random.default_rng(21)
    sig = np.vectorize(lambda c: float(O.e4m3_decode(int(c))))(rng.integers(40, 80, (hkv, 8)))
    mids = rng.choice([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], (hkv, 8, 16))
    # half the blocks 36 to 64 units off (fl(|y|/g) 18 to 64 ulps from a 7-bit number), half 2 to 24
    far = rng.random((hkv, 8, 1)) < 0.5
    off = rng.choice([-1, 1], (hkv, 8, 16)) * np.where(far, rng.integers(36, 65, (hkv, 8, 16)),
                                                      rng.integers(2, 25, (hkv, 8, 16)))
    r = (np.float64(g) * sig[..., None] * mids * (1.0 + off * 2.0 ** -24)).astype(np.float32).reshape(hkv, 128)
    # keys +-2^m, m in {-1, 0, 1}: y = k r is exact, so every element keeps its offset
    kf = (rng.choice([-1.0, 1.0], (N, hkv, 128)) * 2.0 ** rng.integers(-1, 2, (N, hkv, 128))).astype(np.float32)
    kbits = S.bf16_round(kf)
    vbits = S.bf16_round(rng.standard_normal((N, hkv, 128)).astype(np.float32))
    flags = lib.K_SMOOTH | lib.K_MSE_SCALE
    y = O.key_transform(S.bf16_to_f32(kbits)[None], r[None, None], flags)[0]
    assert np.array_equal(y, kf * r[None])
    kc, ks = O.quantize_rows_mse(y, g)
    vc, vs = O.quantize_rows(S.bf16_to_f32(vbits), g)
    # the construction reaches both sides of the screen, and blocks that pass it by a few units
    dist = screen_distance(y, g).reshape(N, hkv, 8, 16).min(-1)
    assert np.count_nonzero(dist < 16) > 100 and np.count_nonzero((dist >= 16) & (dist < 32)) > 100
    assert np.any(ks != O.quantize_rows(y, g)[1])
    pages = P.Pages(1, N, True)
    cache = lib.CacheLayer(pages.num_pages, pages.page_size, hkv, k_flags=flags)
    cache.smooth.copy_(torch.from_numpy((np.float32(1.0) / r).astype(np.float32)))
    cache.inv_smooth.copy_(torch.from_numpy(r))
    cache.gscale.copy_(torch.tensor([g, g]))
    lib.quantize_append_kv(cache.struct(), P.to_dev_u16(kbits), P.to_dev_u16(vbits),
                           P.to_dev_i32(pages.slots(0, 0, N)), N)
    torch.cuda.synchronize()
    check_rows(cache, pages, hkv, N, kc, ks, vc, vs)


def test_mse_corner_blocks_fused_new_token(lib):
    """Each sequence's new token is one corner row; the fused step writes it into its slot."""
    hkv, B = 2, 24
    rows = corner_rows(hkv, B, seed=4)
    k32 = S.bf16_to_f32(rows)
    vbits = rows[:, ::-1].copy()
    kc, ks = O.quantize_rows_mse(k32, G)
    vc, vs = O.quantize_rows(S.bf16_to_f32(vbits), G)
    T = 1                                                   # the new token is the whole sequence
    pages = P.Pages(B, 16, True)
    cache = lib.CacheLayer(pages.num_pages, pages.page_size, hkv, k_flags=lib.K_MSE_SCALE)
    cache.gscale.copy_(torch.tensor([G, G]))
    q = S.bf16_round(np.random.default_rng(9).standard_normal((B, 4 * hkv, 128)).astype(np.float32))
    out = torch.empty((B, 4 * hkv, 128), dtype=torch.float32, device="cuda")
    wsb = lib.decode_workspace_bytes(B, 4 * hkv, hkv, T, 0)
    ws = torch.zeros(max(wsb, 256), dtype=torch.uint8, device="cuda")
    lib.decode_append_attention_nvfp4(cache.struct(), P.to_dev_u16(q), P.to_dev_u16(rows), P.to_dev_u16(vbits), B,
                                      4 * hkv, P.to_dev_i32(pages.table), pages.table.shape[1],
                                      P.to_dev_i32(np.full(B, T)), T, P.sm_scale(), out, ws, wsb, 0)
    torch.cuda.synchronize()
    for b in range(B):
        check_rows(cache, pages, hkv, T, kc[b:b + 1], ks[b:b + 1], vc[b:b + 1], vs[b:b + 1], b=b)
    # one token: the output is its dequantised value row, whatever the scores
    vhat = O.dequantize(vc, vs, G)                                     # [B][Hkv][128]
    want = np.repeat(vhat, 4, axis=1)
    got = out.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(got - want)) <= 1e-6 * max(np.max(np.abs(want)), 1e-30)
