"""Plain CPU oracle for the NVFP4 KV-cache path.  TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import this module.  The product package never imports it, and this module imports
nothing from the product package: the two share no code, tables or constants.

Sources, by page title (section / table named at each function):
  [cache post]  rstation.ai post "NVFP4 attention cache on W4A4 Qwen3-8B: static key
                smoothing is near-lossless, key rotations hurt"
  [OSFP4]       paperlayer.ai summary of arXiv 2610.08231v1, "OSFP4: Joint Optimization of
                Diagonal Smoothing and Block Scales for NVFP4 Quantization"
  [QServe rec]  inference-research record "QServe SmoothAttention (4-bit KV cache with an
                accuracy-preserving correction)"
  [GPTQ thread] rstation.ai comment thread of u/krylov_schur

What the oracle computes (plain, slow, obviously correct; NumPy, fp64 unless noted):
  * calibrate           -- static per-channel key smoothing s = sqrt(absmax) with window
                           position 0 excluded, r = 1/s, and per-tensor fp32 scales g.
  * key_transform       -- fp32 smoothing multiply, optional unnormalised Hadamard-128
                           butterfly in a fixed stage order (this *is* the encoding input,
                           so it is computed in fp32 exactly as specified).
  * quantize_rows       -- NVFP4 encoding: per 16-element block an E4M3 scale chosen so the
                           block absmax maps to 6, then E2M1 codes; both roundings are
                           round-to-nearest-even on the EXACT real quotient.
  * quantize_rows_mse   -- the same encoding with each key block's E4M3 scale searched for
                           the smallest exact squared error (optional key flag).
  * dequantize          -- code value * block scale * tensor scale, in fp64 (exact).
  * klt_basis           -- the static per-head KLT key basis (fp64 eigendecomposition of the
                           calibration keys' covariance, fp32 result); rotate_fp32 applies
                           it to key rows in a fixed fp32 order.
  * query_transform     -- q*s, optionally H(q*s)/128 or B^T(q*s), in fp64.
  * attention           -- textbook softmax attention over the dequantised cache, fp64.
  * causal_attention    -- the same for a block of query positions with the causal mask
                           (teacher-forced evaluation over the cache), fp64.

Readings taken where the pages leave a step open (each is repeated in the design notes):
  - tensor scale g = amax / (6*448), from calibration windows, over ALL positions of the
    transformed keys (the sink is not clipped); g = 1 when amax = 0.
  - E4M3 is the OCP E4M3FN variant (bias 7, subnormals, max 448, no infinities).
  - block scale = E4M3 round-to-nearest-even of A_b/(6 g), saturating to 448; quotients at
    or below 2^-10 give scale 0, and a zero scale gives an all-zero block.
  - E2M1 rounding is to nearest with ties to the even code; magnitudes >= 6 give 6; a zero
    magnitude is stored as the +0 code.
  - smoothing multiplies keys by r = fl32(1/s) and queries by s; V is never transformed.
  - Hadamard is the Sylvester +-1 matrix applied to keys unnormalised (stages h=1..64,
    (a,b) -> (a+b, a-b), each rounded to fp32); the query side carries the exact 1/128.
  - smoothing is applied before the Hadamard basis when both are selected.
  - a block of Tq queries of a sequence holding n cached tokens sits at positions
    n-Tq .. n-1 (the block's own keys are in the cache); position p sees keys 0..p.
  - KLT basis: eigenvectors of the centred covariance of the (smoothed) calibration keys over
    the smoothing's positions, decreasing eigenvalues, largest entry of each positive (ties
    within a relative 1e-6: the first), fp32;
    keys rotated as z = B^T y with each output a chain of fp32 fused multiply-adds over the
    input index, z <- fl32(B[j][i] * y_j + z) for j = 0..127 from z = 0, one rounding per
    step; not combined with the Hadamard basis.
  - MSE-searched key scales: candidates are the absmax-to-6 code and every E4M3 code that
    puts the block maximum between 7/4 and 7 times the scale; the exact squared error
    decides, ties to the absmax-to-6 code, then to the smallest code.

Every function here is pinned by a CPU test against something other than itself
(brute-force nearest search with exact rationals, closed forms printed on the pages,
algebraic invariants, and a library attention routine); no function is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

HEAD_DIM = 128
BLOCK = 16
N_BLOCKS = HEAD_DIM // BLOCK

FLAG_SMOOTH = 1
FLAG_HADAMARD = 2
FLAG_MSE_SCALE = 4
FLAG_KLT = 8

# Largest E2M1 magnitude ([OSFP4] section 1: the FP4 constellation tops out at 6) and
# largest finite E4M3FN value (bias 7, mantissa 0b110 at exponent 15).
E2M1_MAX = 6.0
E4M3_MAX = 448.0
TENSOR_SCALE_DIVISOR = E2M1_MAX * E4M3_MAX  # 2688: amax maps to 6 * 448


# ----------------------------------------------------------------------------------------
# Number formats ([OSFP4] appendix D.1: E2M1 values, E4M3 scales per 16 channels and an
# FP32 tensor scale; appendix I: the scale constellation is the positive E4M3 points).
# ----------------------------------------------------------------------------------------
def e2m1_decode(code: int) -> float:
    """Value of a 4-bit E2M1 code: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0."""
    sign = -1.0 if (code >> 3) & 1 else 1.0
    e = (code >> 1) & 3
    m = code & 1
    if e == 0:
        mag = 0.5 * m                      # subnormal: m * 2^(1-1) * 1/2
    else:
        mag = 2.0 ** (e - 1) * (1.0 + m / 2.0)
    return sign * mag


def e4m3_decode(code: int) -> float:
    """Value of an 8-bit E4M3FN code: sign bit 7, exponent bits 6..3 (bias 7), mantissa 2..0.
    Exponent 15 with mantissa 7 is NaN; there is no infinity."""
    sign = -1.0 if (code >> 7) & 1 else 1.0
    e = (code >> 3) & 15
    m = code & 7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:
        mag = (m / 8.0) * 2.0 ** (1 - 7)
    else:
        mag = 2.0 ** (e - 7) * (1.0 + m / 8.0)
    return sign * mag


E2M1_MAG_GRID = np.array([e2m1_decode(c) for c in range(8)], dtype=np.float64)   # codes 0..7
E4M3_GRID = np.array([e4m3_decode(c) for c in range(127)], dtype=np.float64)     # 0 .. 448


def rne_grid_index(a: np.ndarray, unit: np.ndarray, grid: np.ndarray) -> np.ndarray:
    """Index of the point of ``grid`` nearest to the exact quotient a/unit, ties to the even
    index; quotients beyond the last point give the last index (saturation).

    ``grid`` is increasing and starts at 0.  The midpoint between grid[k] and grid[k+1] is
    passed when a > mid_k*unit, or when a == mid_k*unit and k+1 is even.  Callers guarantee
    that a and every mid_k*unit are exact in fp64 (a is an fp32 value, unit is a product of
    at most 26 significant bits, each midpoint has at most 5), so each comparison is exact.
    """
    a = np.asarray(a, dtype=np.float64)
    unit = np.broadcast_to(np.asarray(unit, dtype=np.float64), a.shape)
    mids = (grid[:-1] + grid[1:]) / 2.0
    idx = np.zeros(a.shape, dtype=np.int64)
    for k, mk in enumerate(mids):
        thr = mk * unit
        idx += (a > thr) | ((a == thr) & ((k + 1) % 2 == 0))
    return idx


# ----------------------------------------------------------------------------------------
# Key transform ([cache post] cache-config table rows "static per-channel smoothing" and
# "Hadamard-128 on head_dim"; [QServe rec] SmoothAttention).  fp32, fixed op order.
# ----------------------------------------------------------------------------------------
def hadamard_butterfly_fp32(y: np.ndarray) -> np.ndarray:
    """Unnormalised Sylvester Hadamard along the last axis (length 128) in fp32: stages
    h = 1, 2, 4, ..., 64; in each stage every pair (i, i+h) with (i & h) == 0 becomes
    (fl32(y_i + y_{i+h}), fl32(y_i - y_{i+h}))."""
    y = np.array(y, dtype=np.float32, copy=True)
    n = y.shape[-1]
    lead = y.shape[:-1]
    h = 1
    while h < n:
        v = y.reshape(lead + (n // (2 * h), 2, h))
        a = v[..., 0, :]
        b = v[..., 1, :]
        s = (a + b).astype(np.float32)
        d = (a - b).astype(np.float32)
        y = np.stack([s, d], axis=-2).reshape(lead + (n,))
        h *= 2
    return y


def sylvester_hadamard(n: int = HEAD_DIM) -> np.ndarray:
    """Dense Sylvester matrix H_n, H_1 = [1], H_2k = [[H_k, H_k], [H_k, -H_k]] (int64)."""
    H = np.ones((1, 1), dtype=np.int64)
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H


def key_transform(x: np.ndarray, r: np.ndarray | None, flags: int, basis: np.ndarray | None = None) -> np.ndarray:
    """Post-RoPE key rows x (any float dtype holding bf16 values, last axes [Hkv][128]) -> fp32
    rows that get quantised.  Smoothing: y_j = fl32(x_j * r_j); then the Hadamard butterfly or
    the KLT basis rotation (basis [Hkv][128][128], see rotate_fp32)."""
    if (flags & FLAG_HADAMARD) and (flags & FLAG_KLT):
        raise ValueError("the Hadamard and KLT key bases exclude each other")
    y = np.asarray(x, dtype=np.float32)
    if flags & FLAG_SMOOTH:
        y = (y * np.asarray(r, dtype=np.float32)).astype(np.float32)
    if flags & FLAG_HADAMARD:
        y = hadamard_butterfly_fp32(y)
    if flags & FLAG_KLT:
        y = rotate_fp32(y, basis)
    return y


# ----------------------------------------------------------------------------------------
# Static per-head KLT key basis ([cache post] cache-config table rows "K: static per-head
# KLT" and "K: static KLT + smoothing": the keys of each KV head are expressed in a fixed
# basis computed once from calibration data, optionally after the static smoothing).
#
# Readings (the pages name the transform only): the KLT of a head is the eigenbasis of the
# covariance (mean removed) of that head's calibration keys, taken after the smoothing when
# both are selected, over the positions the smoothing calibration uses (position 0 excluded);
# columns in decreasing eigenvalue order, each signed so that its largest-magnitude entry is
# positive (entries within a relative 1e-6 of the largest count as ties, and the first of
# them decides, so that rounding noise cannot flip a sign); stored as fp32.  Keys are rotated z = B^T y with each
# output a chain of fp32 fused multiply-adds over the input index (one rounding per step), so
# that codes are reproducible bit for bit; the query side applies the same fp32 basis in
# fp64.  The Hadamard and KLT bases are not combined.
# ----------------------------------------------------------------------------------------
KLT_SIGN_TIE = 1e-6     # entries within this relative distance of the largest count as ties


def klt_basis(k_win: np.ndarray, r: np.ndarray | None, k_flags: int, exclude_pos0: bool = True):
    """k_win [W][T][Hkv][128] (bf16 values) -> (basis f32 [Hkv][128][128], eigenvalues f64
    [Hkv][128]); column i of basis[h] is the eigenvector of eigenvalue i (decreasing)."""
    y = key_transform(np.asarray(k_win, dtype=np.float32), None if r is None else r[None, None],
                      k_flags & FLAG_SMOOTH)
    y = y[:, 1:] if exclude_pos0 else y
    hkv = y.shape[2]
    X = y.astype(np.float64).reshape(-1, hkv, HEAD_DIM)
    basis = np.zeros((hkv, HEAD_DIM, HEAD_DIM), dtype=np.float32)
    lam_out = np.zeros((hkv, HEAD_DIM))
    for h in range(hkv):
        D = X[:, h] - X[:, h].mean(axis=0)
        C = D.T @ D / D.shape[0]
        lam, V = np.linalg.eigh(C)                  # increasing
        order = np.argsort(-lam, kind="stable")
        lam, V = lam[order], V[:, order]
        for i in range(HEAD_DIM):
            a = np.abs(V[:, i])
            j = int(np.argmax(a >= (1.0 - KLT_SIGN_TIE) * a.max()))   # first (near-)largest entry
            if V[j, i] < 0:
                V[:, i] = -V[:, i]
        basis[h] = V.astype(np.float32)
        lam_out[h] = lam
    return basis, lam_out


def _fma_f64_to_f32(p: np.ndarray, c64: np.ndarray) -> np.ndarray:
    """fl32(p + c) for an exact fp64 product p and fp32 values c held in fp64.

    The fp64 sum s is rounded to nearest; its exact error e comes from the two-sum identity.
    Where e != 0 and s has an even last bit, s moves one step towards e: that makes s the
    round-to-odd value of the exact sum, and a round-to-odd value with 53 >= 24 + 2 bits rounds
    to fp32 exactly as the exact sum would.  Valid away from fp64 overflow."""
    s = p + c64
    bb = s - p
    e = (p - (s - bb)) + (c64 - bb)
    fix = (e != 0) & ((s.view(np.int64) & 1) == 0)
    if fix.any():
        s = np.where(fix, np.nextafter(s, np.where(e > 0, np.inf, -np.inf)), s)
    return s.astype(np.float32)


def fma_f32(a: np.ndarray, b: np.ndarray, c: np.ndarray) -> np.ndarray:
    """fl32(a*b + c) with a single rounding (a fused multiply-add), for fp32 arrays: the
    product of two fp32 values is exact in fp64 (48 significant bits), then one correctly
    rounded addition (_fma_f64_to_f32)."""
    p = np.asarray(a, dtype=np.float32).astype(np.float64) * np.asarray(b, dtype=np.float32).astype(np.float64)
    c64 = np.asarray(c, dtype=np.float32).astype(np.float64)
    p, c64 = np.broadcast_arrays(p, c64)
    return _fma_f64_to_f32(p, c64)


def rotate_fp32(y: np.ndarray, basis: np.ndarray) -> np.ndarray:
    """z[..., h, i] = sum_j basis[h, j, i] * y[..., h, j], taken as a chain of fused
    multiply-adds over j = 0..127: z <- fl32(basis[h, j, i] * y_j + z) from z = 0, one rounding
    per step."""
    y64 = np.asarray(y, dtype=np.float32).astype(np.float64)
    B64 = np.asarray(basis, dtype=np.float32).astype(np.float64)
    acc = np.zeros(y64.shape, dtype=np.float64)            # fp32 values held in fp64
    for j in range(HEAD_DIM):
        acc = _fma_f64_to_f32(B64[:, j, :] * y64[..., :, j:j + 1], acc).astype(np.float64)
    return acc.astype(np.float32)


# ----------------------------------------------------------------------------------------
# Calibration ([cache post] smoothing row: sqrt(absmax) from 4 windows, position 0
# excluded; [OSFP4] section 3: a static calibration-based global scale lets blocks be
# quantised online before the whole tensor exists).
# ----------------------------------------------------------------------------------------
def calibrate(k_win: np.ndarray | None, v_win: np.ndarray | None,
              exclude_pos0: bool = True, k_flags: int = FLAG_SMOOTH):
    """k_win, v_win: [W][T][Hkv][128] arrays of bf16 values (as float).
    Returns (s [Hkv][128] f32, r [Hkv][128] f32, g [2] f32) with g = (g_K, g_V).
    A part whose windows are None is returned as None (s, r) / NaN (g entry).  With the KLT
    flag, g_K is taken over keys rotated by klt_basis of the same windows."""
    s = r = None
    g = np.array([np.nan, np.nan], dtype=np.float32)
    if k_win is not None:
        k = np.asarray(k_win, dtype=np.float64)
        kk = k[:, 1:] if exclude_pos0 else k
        a = np.abs(kk).max(axis=(0, 1)) if kk.shape[1] > 0 else np.zeros(k.shape[2:])
        # fp32 sqrt and reciprocal, each correctly rounded (fp64 then one rounding to fp32
        # is exact-rounding for sqrt and division: 53 >= 2*24 + 2).
        s = np.where(a == 0.0, 1.0, np.sqrt(a)).astype(np.float32)
        r = (np.float32(1.0) / s).astype(np.float32)
        basis = klt_basis(k_win, r, k_flags, exclude_pos0)[0] if k_flags & FLAG_KLT else None
        y = key_transform(np.asarray(k_win, dtype=np.float32), r[None, None], k_flags, basis)
        g[0] = _tensor_scale(np.abs(y.astype(np.float64)).max())
    if v_win is not None:
        g[1] = _tensor_scale(np.abs(np.asarray(v_win, dtype=np.float64)).max())
    return s, r, g


def _tensor_scale(amax: float) -> np.float32:
    """g = fl32(amax / 2688), or 1 when amax is 0."""
    if amax == 0.0:
        return np.float32(1.0)
    return np.float32(np.float64(np.float32(amax)) / TENSOR_SCALE_DIVISOR)


# ----------------------------------------------------------------------------------------
# NVFP4 encoding ([OSFP4] section 1: 16-entry groups, E4M3 scales, FP4 max 6, absmax-to-6
# flushes entries 24x below the block max; section 3: absmax-to-6 per 16-entry group at
# inference; [cache post] opening paragraph: 16-blocks along head_dim, post-RoPE K/V).
# ----------------------------------------------------------------------------------------
def absmax_scale_codes(A: np.ndarray, g64) -> np.ndarray:
    """E4M3 block-scale codes by the absmax-to-6 rule: RNE of the exact A/(6g), saturating
    at 448 (code 126)."""
    return rne_grid_index(A, 6.0 * g64, E4M3_GRID)


def encode_blocks(y32: np.ndarray, g: float, S: np.ndarray):
    """Rows of 128 fp32 values and a chosen E4M3 scale code per block ([..., 8]) -> (codes u8
    [..., 64], scales u8 [..., 8]).  Element magnitude code = E2M1 RNE of the exact
    |y|/(sigma_b g) (0 when sigma_b = 0); nibble = 0 for magnitude 0, else sign<<3 |
    magnitude.  Byte k = nibble(2k) | nibble(2k+1) << 4."""
    y32 = np.asarray(y32, dtype=np.float32)
    lead = y32.shape[:-1]
    y = y32.astype(np.float64).reshape(lead + (N_BLOCKS, BLOCK))
    g64 = np.float64(np.float32(g))
    S = np.asarray(S, dtype=np.int64)
    sigma = E4M3_GRID[S]
    unit = (sigma * g64)[..., None] * np.ones_like(y)
    mag = rne_grid_index(np.abs(y), unit, E2M1_MAG_GRID)
    mag = np.where((sigma == 0.0)[..., None], 0, mag)
    sign = np.signbit(y32.reshape(y.shape)).astype(np.int64)
    nib = np.where(mag == 0, 0, (sign << 3) | mag).reshape(lead + (HEAD_DIM,))
    codes = (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)
    return codes, S.astype(np.uint8)


def quantize_rows(y32: np.ndarray, g: float):
    """Rows of 128 fp32 values -> (codes u8 [..., 64], scales u8 [..., 8]).

    Block b = elements 16b..16b+15.  A_b = max |y|; scale code S_b = E4M3 RNE of the exact
    A_b/(6g), saturating at 448; sigma_b = value(S_b); the elements are then encoded by
    encode_blocks."""
    y32 = np.asarray(y32, dtype=np.float32)
    lead = y32.shape[:-1]
    y = y32.astype(np.float64).reshape(lead + (N_BLOCKS, BLOCK))
    g64 = np.float64(np.float32(g))
    return encode_blocks(y32, g, absmax_scale_codes(np.abs(y).max(axis=-1), g64))


# ----------------------------------------------------------------------------------------
# MSE-searched key block scales ([OSFP4] section 1: absmax-to-6 zeroes entries 24x below the
# block maximum and other scale choices can lower the distortion; appendix H: unweighted
# MSE-optimal E4M3 scales as a baseline; section 3 and appendix C: the deployed weight scales
# come from a search over valid E4M3 scales under the deterministic FP4 error, one block at a
# time for round-to-nearest; section 2.1 and appendix A (Lemma 1): the smoothed FP4 error is
# flat, at its minimum, for values between 7/4 and 7 times the scale).
#
# Readings (the pages give no candidate set): the candidates of a block are its absmax-to-6
# code and every E4M3 code c >= 1 whose scale puts the block maximum inside Lemma 1's
# interval, 7/4 <= A/(g sigma_c) <= 7; the chosen code minimises the block's squared error
# sum_j (y_j - y_hat_j)^2 over the candidates, with y_hat the round-to-nearest FP4
# dequantisation; ties go to the absmax-to-6 code, then to the smallest code.  The tensor
# scale g is the absmax-to-6 calibration's.
# ----------------------------------------------------------------------------------------
MSE_RATIO_LO = 1.75
MSE_RATIO_HI = 7.0


def mse_candidate_mask(A: np.ndarray, g64, c: int) -> np.ndarray:
    """Blocks (by absmax A) for which E4M3 code c >= 1 lies in the search interval.  Both
    products are exact in fp64 (24 + 4 + 3 significant bits)."""
    u = E4M3_GRID[c] * g64
    return (MSE_RATIO_LO * u <= A) & (A <= MSE_RATIO_HI * u)


def mse_block_sse(absy: np.ndarray, c: np.ndarray, g64) -> np.ndarray:
    """Squared FP4 error sum_j (|y_j| - y_hat_j)^2 of blocks |y| [n][16] encoded with scale
    codes c [n], y_hat_j = m_j g sigma_c with m_j the round-to-nearest E2M1 magnitude of
    |y_j| / (g sigma_c) (0 when sigma_c = 0), in fp64.

    For every block that has more than one candidate each difference is exact in fp64: a
    nonzero m_j needs |y_j| >= u/4 (u = g sigma_c) while |y_j| <= A <= 7u, and y_hat_j has at
    most 3 + 4 + 24 significant bits, so both operands lie within 35 bits; a zero m_j leaves
    |y_j|.  Each square rounds once and the sum of 16 non-negative terms at most 15 times,
    so the result is within MSE_SSE_REL_ERR (relative) of the exact sum."""
    c = np.asarray(c, dtype=np.int64)
    sigma = E4M3_GRID[c]
    unit = (sigma * g64)[:, None] * np.ones_like(absy)
    mag = rne_grid_index(absy, unit, E2M1_MAG_GRID)
    mag = np.where((sigma == 0.0)[:, None], 0, mag)
    d = absy - E2M1_MAG_GRID[mag] * unit
    return (d * d).sum(axis=-1)


MSE_SSE_REL_ERR = 2.0 ** -48


def mse_block_sse_exact(absy_row: np.ndarray, codes, g64) -> list:
    """The same squared errors of one block under each of `codes` (None for a code < 0), exact:
    |y_j| (an fp32 value) and y_hat_j = m_j * (g sigma_c) (at most 3 + 4 + 24 significant
    bits, so exact in fp64) are dyadic rationals, which are put over one power-of-two
    denominator D for all codes; each error is returned as the integer D^2 * sum_j
    (|y_j| - y_hat_j)^2, so the errors of the codes compare exactly."""
    absy_row = np.asarray(absy_row, np.float64)
    yhat = []
    for c in codes:
        c = int(c)
        if c < 0:
            yhat.append(None)
            continue
        unit = float(E4M3_GRID[c]) * float(g64)
        if unit == 0.0:
            yhat.append(np.zeros(BLOCK))
        else:
            mag = rne_grid_index(absy_row[None], np.full((1, BLOCK), unit), E2M1_MAG_GRID)[0]
            yhat.append(E2M1_MAG_GRID[mag] * unit)
    ratios_y = [float(v).as_integer_ratio() for v in absy_row]
    ratios_h = [None if h is None else [float(v).as_integer_ratio() for v in h] for h in yhat]
    den = max([q for _, q in ratios_y] + [q for r in ratios_h if r is not None for _, q in r])
    ys = [p_ * (den // q) for p_, q in ratios_y]
    out = []
    for r in ratios_h:
        out.append(None if r is None else sum((y - p_ * (den // q)) ** 2 for y, (p_, q) in zip(ys, r)))
    return out


def mse_candidates(A: np.ndarray, g64, s0: np.ndarray) -> np.ndarray:
    """Candidate codes of each block [n][1 + the longest run]: column 0 the absmax-to-6 code
    s0, then every other code c >= 1 with 7/4 <= A/(g sigma_c) <= 7 in increasing order (one
    run of at most 17 codes); -1 pads."""
    masks = [(c, mse_candidate_mask(A, g64, c) & (s0 != c)) for c in range(1, len(E4M3_GRID))]
    width = 1 + int(np.max(sum(mk.astype(np.int64) for _, mk in masks), initial=0))
    cand = np.full((A.shape[0], width), -1, dtype=np.int64)
    cand[:, 0] = s0
    cnt = np.ones(A.shape[0], dtype=np.int64)
    for c, mk in masks:
        idx = np.nonzero(mk)[0]
        cand[idx, cnt[idx]] = c
        cnt[idx] += 1
    return cand


def mse_pick(cand: np.ndarray, err) -> int:
    """Column of the chosen candidate among the valid columns of one block, from their squared
    errors (any exactly ordered numbers): the smallest error; ties keep column 0 (the
    absmax-to-6 code), then the smallest code."""
    cols = [k for k in range(cand.shape[0]) if cand[k] >= 0]
    return min(cols, key=lambda k: (err[k], -1 if k == 0 else int(cand[k])))


def mse_scale_codes(y32: np.ndarray, g: float) -> np.ndarray:
    """E4M3 scale code per block ([..., 8]) with the smallest squared FP4 error over the
    candidates described above (ties: the absmax-to-6 code, then the smallest code).  The
    errors are evaluated in fp64 (mse_block_sse); a block whose best error is not ahead of
    every other candidate's by more than the fp64 error bound is decided on the exact
    rational errors."""
    y32 = np.asarray(y32, dtype=np.float32)
    lead = y32.shape[:-1]
    absy = np.abs(y32.astype(np.float64)).reshape(-1, BLOCK)
    g64 = np.float64(np.float32(g))
    A = absy.max(axis=-1)
    s0 = absmax_scale_codes(A, g64)
    cand = mse_candidates(A, g64, s0)
    n, K = cand.shape
    sse = np.full((n, K), np.inf)
    for k in range(K):
        idx = np.nonzero(cand[:, k] >= 0)[0]
        if idx.size:
            sse[idx, k] = mse_block_sse(absy[idx], cand[idx, k], g64)
    # fp64 decision: the smallest error, ties to column 0 and then the smallest code
    m = sse.min(axis=1)
    rank = np.where(np.arange(K)[None, :] == 0, -1, cand)
    kbest = np.where(sse == m[:, None], rank, np.iinfo(np.int64).max).argmin(axis=1)
    rows = np.arange(n)
    best = cand[rows, kbest]
    # blocks where another candidate is within the rounding bound of the best are decided on
    # the exact rational errors
    close = sse <= (m * (1.0 + 4 * MSE_SSE_REL_ERR))[:, None]
    close[rows, kbest] = False
    for i in np.nonzero(close.any(axis=1))[0]:
        best[i] = cand[i, mse_pick(cand[i], mse_block_sse_exact(absy[i], cand[i], g64))]
    return best.reshape(lead + (N_BLOCKS,))


def quantize_rows_mse(y32: np.ndarray, g: float):
    """quantize_rows with each block's scale chosen by mse_scale_codes."""
    return encode_blocks(y32, g, mse_scale_codes(y32, g))


def quantize_keys(y32: np.ndarray, g: float, flags: int):
    """Transformed key rows -> NVFP4 with the block-scale rule selected by flags."""
    if flags & FLAG_MSE_SCALE:
        return quantize_rows_mse(y32, g)
    return quantize_rows(y32, g)


def unpack_nibbles(codes: np.ndarray) -> np.ndarray:
    """u8 [..., 64] -> nibbles [..., 128] (low nibble = even element)."""
    codes = np.asarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape[:-1] + (2 * codes.shape[-1],), dtype=np.int64)
    out[..., 0::2] = codes & 0xF
    out[..., 1::2] = codes >> 4
    return out


E2M1_ALL = np.array([e2m1_decode(c) for c in range(16)], dtype=np.float64)
E4M3_ALL = np.array([e4m3_decode(c) for c in range(256)], dtype=np.float64)


def dequantize(codes: np.ndarray, scales: np.ndarray, g: float) -> np.ndarray:
    """x_hat_j = e2m1(nibble_j) * sigma_b * g in fp64 (exact: 2 + 4 + 24 significant bits)."""
    nib = unpack_nibbles(codes)
    lead = nib.shape[:-1]
    vals = E2M1_ALL[nib].reshape(lead + (N_BLOCKS, BLOCK))
    sig = E4M3_ALL[np.asarray(scales, dtype=np.int64)][..., None]
    return (vals * sig * np.float64(np.float32(g))).reshape(lead + (HEAD_DIM,))


# ----------------------------------------------------------------------------------------
# Decode attention ([cache post] opening paragraph: attention runs over the fake-quantised
# post-RoPE cache; smoothing row: SmoothAttention, keys divided and queries multiplied by s;
# Hadamard rows: an orthogonal basis change on head_dim).
# ----------------------------------------------------------------------------------------
def query_transform(q: np.ndarray, s: np.ndarray | None, flags: int, basis: np.ndarray | None = None) -> np.ndarray:
    """q [..., 128] (bf16 values) -> q' in fp64: q*s, then H(q*s)/128 when Hadamard is on, or
    B^T (q*s) with the KLT basis.  ``s`` and ``basis`` ([..., 128, 128]) broadcast against q
    (one entry per KV head of each query head)."""
    qp = np.asarray(q, dtype=np.float64)
    if flags & FLAG_SMOOTH:
        qp = qp * np.asarray(s, dtype=np.float64)
    if flags & FLAG_HADAMARD:
        H = sylvester_hadamard(HEAD_DIM).astype(np.float64)
        qp = qp @ H.T / 128.0
    if flags & FLAG_KLT:
        B = np.asarray(basis, dtype=np.float64)
        qp = np.einsum("...j,...ji->...i", qp, B)
    return qp


def attention(qp: np.ndarray, k_hat: list, v_hat: list, seq_lens, sm_scale: float):
    """Textbook GQA decode attention in fp64.

    qp: [B][Hq][128] transformed queries; k_hat[b], v_hat[b]: [n_b][Hkv][128] dequantised
    cache of sequence b (n_b >= seq_lens[b]).  Query head hq reads KV head hq // (Hq/Hkv).
    Output [B][Hq][128]; a sequence with no cached tokens gives zeros."""
    qp = np.asarray(qp, dtype=np.float64)
    B, Hq, D = qp.shape
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        n = int(seq_lens[b])
        if n == 0:
            continue
        K = np.asarray(k_hat[b], dtype=np.float64)[:n]
        V = np.asarray(v_hat[b], dtype=np.float64)[:n]
        Hkv = K.shape[1]
        grp = Hq // Hkv
        for hq in range(Hq):
            h = hq // grp
            e = sm_scale * (K[:, h, :] @ qp[b, hq])
            p = np.exp(e - e.max())
            p /= p.sum()
            out[b, hq] = p @ V[:, h, :]
    return out


def causal_attention(qp: np.ndarray, k_hat: list, v_hat: list, seq_lens, sm_scale: float):
    """Textbook causal GQA attention of a block of query positions over the dequantised
    cache, in fp64 ([cache post] opening paragraph: the model is evaluated teacher-forced over
    full windows, with attention reading the fake-quantised post-RoPE cache; the mask is the
    causal mask of a decoder, each position attending to itself and earlier positions).

    qp: [B][Tq][Hq][128] transformed queries.  Query i of sequence b sits at position
    p = seq_lens[b] - Tq + i and attends to keys 0..p of k_hat[b], v_hat[b] ([n_b][Hkv][128],
    n_b >= seq_lens[b]); a row with p < 0 has no keys and is zero.  Query head hq reads KV
    head hq // (Hq/Hkv).  Output [B][Tq][Hq][128]."""
    qp = np.asarray(qp, dtype=np.float64)
    B, Tq, Hq, D = qp.shape
    out = np.zeros((B, Tq, Hq, D), dtype=np.float64)
    for b in range(B):
        n = int(seq_lens[b])
        K = np.asarray(k_hat[b], dtype=np.float64)
        V = np.asarray(v_hat[b], dtype=np.float64)
        Hkv = K.shape[1]
        grp = Hq // Hkv
        for i in range(Tq):
            p = n - Tq + i
            if p < 0:
                continue
            for hq in range(Hq):
                h = hq // grp
                e = sm_scale * (K[:p + 1, h, :] @ qp[b, i, hq])
                w = np.exp(e - e.max())
                w /= w.sum()
                out[b, i, hq] = w @ V[:p + 1, h, :]
    return out


# ----------------------------------------------------------------------------------------
# Sizes ([cache post] closing paragraph: BF16 cache size per token; [GPTQ thread] results
# table: NVFP4 at 4.50 bits per value).
# ----------------------------------------------------------------------------------------
def row_bytes(fmt: str, head_dim: int = HEAD_DIM) -> int:
    """Bytes of one (token, KV head) row: bf16 = 2*D; nvfp4 = D/2 code bytes + D/16 scales."""
    if fmt == "bf16":
        return 2 * head_dim
    if fmt == "nvfp4":
        return head_dim // 2 + head_dim // BLOCK
    raise ValueError(fmt)


def cache_bytes_per_token(k_fmt: str, v_fmt: str, num_kv_heads: int, num_layers: int,
                          head_dim: int = HEAD_DIM) -> int:
    return num_layers * num_kv_heads * (row_bytes(k_fmt, head_dim) + row_bytes(v_fmt, head_dim))


def bits_per_value(fmt: str, head_dim: int = HEAD_DIM) -> float:
    return 8.0 * row_bytes(fmt, head_dim) / head_dim
