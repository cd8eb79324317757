// NVFP4 encoder and key transform, one lane per 16-element block (8 lanes per 128-wide row).
// The key transform is part of the bit-exact encoding: every fp32 multiply and add below
// must round on its own, so each function turns floating-point contraction off for its own
// body (the including unit keeps its setting for everything else).
//
// Sources: [cache post] = rstation.ai post "NVFP4 attention cache on W4A4 Qwen3-8B: static
// key smoothing is near-lossless, key rotations hurt" (cache-config table: per-channel
// smoothing sqrt(absmax) and Hadamard-128 on head_dim); [OSFP4] = paperlayer.ai summary of
// arXiv 2610.08231v1 (section 1: 16-entry groups, E4M3 scales, FP4 max 6, absmax-to-6;
// section 3: absmax-to-6 per 16-entry group with a calibration-based global scale).
#pragma once

#include "nvkv_device.hpp"


namespace nvkv {

// Block b of a row sits in the lane whose block index is b; the lanes of one row are
// LANE_STRIDE apart (see hadamard_row).
__device__ __forceinline__ float xor_lanes(float v, int mask) { return __shfl_xor(v, mask, 64); }

// Smoothing: y_j = fl32(x_j * r_j) for the 16 elements of this lane's block.
__device__ __forceinline__ void smooth_block(float (&y)[kBlock], const float* __restrict__ r16) {
#pragma clang fp contract(off)
  const float4* rp = reinterpret_cast<const float4*>(r16);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 rv = rp[q];
    y[4 * q + 0] = y[4 * q + 0] * rv.x;
    y[4 * q + 1] = y[4 * q + 1] * rv.y;
    y[4 * q + 2] = y[4 * q + 2] * rv.z;
    y[4 * q + 3] = y[4 * q + 3] * rv.w;
  }
}

// Unnormalised Sylvester Hadamard over the 128-element row, stages h = 1, 2, ..., 64 in that
// order; a stage maps the pair (i, i+h) with (i & h) == 0 to (y_i + y_{i+h}, y_i - y_{i+h}).
// Stages 1..8 stay inside a lane's block; stages 16, 32, 64 pair block b with b ^ 1, 2, 4,
// which sits LANE_STRIDE lanes times that apart.
template <int LANE_STRIDE = 1>
__device__ __forceinline__ void hadamard_row(float (&y)[kBlock], int blk) {
#pragma clang fp contract(off)
#pragma unroll
  for (int h = 1; h < kBlock; h <<= 1) {
#pragma unroll
    for (int i = 0; i < kBlock; ++i) {
      if ((i & h) == 0) {
        const float a = y[i], b = y[i + h];
        y[i] = a + b;
        y[i + h] = a - b;
      }
    }
  }
#pragma unroll
  for (int d = 1; d < 8; d <<= 1) {
    const bool upper = (blk & d) != 0;
#pragma unroll
    for (int i = 0; i < kBlock; ++i) {
      const float p = xor_lanes(y[i], d * LANE_STRIDE);
      y[i] = upper ? (p - y[i]) : (y[i] + p);
    }
  }
}

// Is the midpoint between E4M3 codes k and k+1 (k <= 125) passed by the exact quotient
// A/(6g)?  6 * midpoint = 3 * (v_k + v_{k+1}) is exact in fp32, and the sign of the fused
// A - t6*g is that of the exact difference; at an exact midpoint the even code wins.
__device__ __forceinline__ bool e4m3_mid_passed(uint32_t k, float A, float g) {
#pragma clang fp contract(off)
  const float t6 = 3.0f * (e4m3_value(k) + e4m3_value(k + 1));
  const float d = __builtin_fmaf(-t6, g, A);
  return (d > 0.0f) | ((d == 0.0f) & (((k + 1) & 1u) == 0u));    // no short-circuit branches
}

// E4M3 block-scale code: round-to-nearest-even of the exact A/(6g), saturating at 448
// (code 0x7E); g > 0 and normal.  A candidate is the code nearest to the rounded fp32 quotient (its
// error is a few ulp, far below the 1/16 relative spacing of the codes, so the exact answer
// is the candidate or a neighbour); the exact midpoint tests on both sides settle it.
__device__ __forceinline__ uint32_t e4m3_scale_code(float A, float g) {
#pragma clang fp contract(off)
  // straight-line code (selects, no short-circuit operators): it runs on every lane
  const float x = A * __builtin_amdgcn_rcpf(6.0f * g);                // A = 0 gives x = 0 -> code 0
  const int c_sub = static_cast<int>(__builtin_rintf(x * 512.0f));    // subnormal codes: x * 2^9
  // normal codes: (exponent field - 120) * 8 + 3 mantissa bits, rounded at mantissa bit 20
  const uint32_t rn = (__float_as_uint(x) + 0x80000u) >> 20;
  const int c_norm = rn > 1086u ? 126 : static_cast<int>(rn) - 960;    // also catches inf
  int c = x < 0.015625f ? c_sub : c_norm;
  c = c > 126 ? 126 : c;
  const uint32_t cu = static_cast<uint32_t>(c);
  const bool up = (c < 126) & e4m3_mid_passed(cu < 125u ? cu : 125u, A, g);
  const bool down = (!up) & (c > 0) & !e4m3_mid_passed(cu > 0u ? cu - 1u : 0u, A, g);
  return static_cast<uint32_t>(c + (up ? 1 : 0) - (down ? 1 : 0));
}

// The same decision with the two neighbouring midpoints read from a table of 6x midpoints,
// t6[k] = 3 (v_k + v_{k+1}) for k = 0..125 (the values e4m3_mid_passed forms, so the result
// is the same bit for bit); the kernels that encode many blocks keep the table in LDS.
__device__ __forceinline__ void fill_e4m3_tables(float* val, float* t6, int tid, int nthreads) {
#pragma clang fp contract(off)
  for (int k = tid; k < 127; k += nthreads) {
    val[k] = e4m3_value(static_cast<uint32_t>(k));
    if (k < 126) t6[k] = 3.0f * (e4m3_value(static_cast<uint32_t>(k)) + e4m3_value(static_cast<uint32_t>(k + 1)));
  }
}

__device__ __forceinline__ bool e4m3_mid_passed_t(uint32_t k, float A, float g, const float* t6) {
#pragma clang fp contract(off)
  const float d = __builtin_fmaf(-t6[k], g, A);
  return (d > 0.0f) | ((d == 0.0f) & (((k + 1) & 1u) == 0u));
}

__device__ __forceinline__ uint32_t e4m3_scale_code_t(float A, float g, const float* t6) {
#pragma clang fp contract(off)
  const float x = A * __builtin_amdgcn_rcpf(6.0f * g);
  const int c_sub = static_cast<int>(__builtin_rintf(x * 512.0f));
  const uint32_t rn = (__float_as_uint(x) + 0x80000u) >> 20;
  const int c_norm = rn > 1086u ? 126 : static_cast<int>(rn) - 960;
  int c = x < 0.015625f ? c_sub : c_norm;
  c = c > 126 ? 126 : c;
  const uint32_t cu = static_cast<uint32_t>(c);
  const bool up = (c < 126) & e4m3_mid_passed_t(cu < 125u ? cu : 125u, A, g, t6);
  const bool down = (!up) & (c > 0) & !e4m3_mid_passed_t(cu > 0u ? cu - 1u : 0u, A, g, t6);
  return static_cast<uint32_t>(c + (up ? 1 : 0) - (down ? 1 : 0));
}

// Per-block E2M1 decision bounds.  The midpoints of the magnitude grid {0, .5, 1, 1.5, 2,
// 3, 4, 6} are t = .25, .75, 1.25, 1.75, 2.5, 3.5, 5, and the exact threshold of midpoint k is
// T_k = t_k sigma g.  A tie goes to the even code: up at odd k (0.75, 1.75, 3.5: the value
// passes when a >= T_k) and down at even k (it passes when a > T_k).  For an fp32 value a,
// "a >= T" is "a >= RU(T)" and "a > T" is "a > RD(T)", with RU / RD the fp32 values next
// above / below T (both T when T is an fp32 value; otherwise no fp32 value lies between them,
// so neither comparison can meet T itself).  Each bound comes once per block from the rounded
// product and the sign of its exact error (one FMA), so an element costs three plain compares.
// Valid for products far above the fp32 subnormal range, as everywhere in this encoder.
__device__ __forceinline__ float bound_rd(float P, float g) {
#pragma clang fp contract(off)
  const float p = P * g;
  const float e = __builtin_fmaf(P, g, -p);                 // exact P*g - p
  return e < 0.0f ? __uint_as_float(__float_as_uint(p) - 1u) : p;
}
__device__ __forceinline__ float bound_ru(float P, float g) {
#pragma clang fp contract(off)
  const float p = P * g;
  const float e = __builtin_fmaf(P, g, -p);
  return e > 0.0f ? __uint_as_float(__float_as_uint(p) + 1u) : p;
}

struct E2m1Thresholds {
  float u0, u1, u2, u3, u4, u5, u6;       // RD, RU, RD, RU, RD, RU, RD of T_0 .. T_6
  __device__ __forceinline__ E2m1Thresholds(float sigma, float g)
      : u0(bound_rd(0.25f * sigma, g)), u1(bound_ru(0.75f * sigma, g)), u2(bound_rd(1.25f * sigma, g)),
        u3(bound_ru(1.75f * sigma, g)), u4(bound_rd(2.5f * sigma, g)), u5(bound_ru(3.5f * sigma, g)),
        u6(bound_rd(5.0f * sigma, g)) {
    // keep the seven bounds in registers: left to itself the compiler re-forms them at every
    // use and turns the bound selects of all 16 elements into branches
    asm volatile("" : "+v"(u0), "+v"(u1), "+v"(u2), "+v"(u3), "+v"(u4), "+v"(u5), "+v"(u6));
  }
};

// E2M1 magnitude code (0..7) of a = |y| >= 0 in a block with scale sigma > 0: round to nearest
// (ties to the even code) of the exact a/(sigma g), saturating at 6.  Binary search with the
// comparison type of each level fixed (levels 1, 2: ties up, >=; level 3: ties down, >).
__device__ __forceinline__ uint32_t e2m1_mag(float a, const E2m1Thresholds& t) {
  const bool b2 = a >= t.u3;
  // bound choices as bit selects on all-ones / all-zero masks (nested conditional
  // expressions are compiled to branches here)
  const uint32_t m2 = b2 ? 0xFFFFFFFFu : 0u;
  const float t1 = __uint_as_float((__float_as_uint(t.u5) & m2) | (__float_as_uint(t.u1) & ~m2));
  const bool b1 = a >= t1;
  const uint32_t m1 = b1 ? 0xFFFFFFFFu : 0u;
  const uint32_t hi2 = (__float_as_uint(t.u6) & m1) | (__float_as_uint(t.u4) & ~m1);
  const uint32_t lo2 = (__float_as_uint(t.u2) & m1) | (__float_as_uint(t.u0) & ~m1);
  const float t0 = __uint_as_float((hi2 & m2) | (lo2 & ~m2));
  const bool b0 = a > t0;
  return (uint32_t(b2) << 2) | (uint32_t(b1) << 1) | uint32_t(b0);
}

// Signed E2M1 nibble of y: magnitude code, sign bit 3, a zero magnitude stored as code 0.
__device__ __forceinline__ uint32_t e2m1_nibble(float y, const E2m1Thresholds& t) {
  const uint32_t m = e2m1_mag(fabsf(y), t);
  const uint32_t sign = (__float_as_uint(y) >> 28) & 8u;
  return m | (m ? sign : 0u);
}

// Eight signed nibbles packed in a word (nibble i = element i): the sign bits are set for
// every element and then cleared where the magnitude is zero, once per word.
__device__ __forceinline__ uint32_t e2m1_pack8(const float* y, const E2m1Thresholds& t) {
  uint32_t w = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) w |= (e2m1_mag(fabsf(y[i]), t) | ((__float_as_uint(y[i]) >> 28) & 8u)) << (4 * i);
  const uint32_t z = ~(w | (w >> 1) | (w >> 2)) & 0x11111111u;     // bit 0 of nibbles with magnitude 0
  return w & ~(z << 3);
}

// Clear the sign bit of every nibble whose magnitude is zero (a zero is stored as code 0).
__device__ __forceinline__ uint32_t clear_zero_signs(uint32_t w) {
  const uint32_t z = ~(w | (w >> 1) | (w >> 2)) & 0x11111111u;     // bit 0 of nibbles with magnitude 0
  return w & ~(z << 3);
}

// Eight elements through the hardware E2M1 converter: nibble i = RNE(y_i * Rs) with ties to
// the even code, saturating at 6, sign from y_i (so a zero magnitude may carry a sign bit).
// The converter divides by the power of two of its scale operand; 1 leaves the input as is.
__device__ __forceinline__ uint32_t cvt_pack8(const float* y, float Rs) {
#pragma clang fp contract(off)
  uint32_t w = 0u;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[0] * Rs, y[1] * Rs, 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[2] * Rs, y[3] * Rs, 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[4] * Rs, y[5] * Rs, 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[6] * Rs, y[7] * Rs, 1.0f, 3);
  return w;
}

// Relative margins of the bracketing quotients: 1 -/+ 2^-20.
constexpr float kBracketDown = 1.0f - 0x1p-20f;
constexpr float kBracketUp = 1.0f + 0x1p-20f;

// Midpoint screen, for a block that is encoded under many scales.  The E2M1 rounding
// midpoints are 1/4, 3/4, 5/4, 7/4, 5/2, 7/2 and 5: an odd number up to 7 times a power of
// two.  An E4M3 value has at most 4 significant bits, so every midpoint of the quotient
// |y| / (sigma g), over every scale sigma, is a point |y| / g = N with N of at most 7
// significant bits.  W = fl(|y| rcp(g) + tiny) is within 3 * 2^-24 (relative) of |y| / g (the
// reciprocal 1 ulp, the multiply-add half an ulp).  When the 17 significand bits of W below
// its top 7 are at least kScreenUlps = 16 away from 0 and from 2^17, W is at least 16 ulps
// from every number with 7 significant bits, which is at least 16 * 2^-24 relative; then
// |y| / (sigma g) stays at least 12 * 2^-24 (relative) away from every midpoint of every scale,
// twice the 6 * 2^-24 error of the converter's quotient |y| R, so that quotient rounds like
// the exact one.  An element that can take a nonzero code under a scale has W >= sigma / 4 >=
// 2^-11, far above the tiny addend (2^-126); a zero element gives W = tiny, whose low bits
// pass.  The screen fails for about one block in 250 of generic data (and for data on a
// coarse grid relative to g); those blocks keep the bracketed pass.
constexpr uint32_t kScreenUlps = 16u;
__device__ __forceinline__ bool clear_of_midpoints(const float (&y)[kBlock], float rg) {
  constexpr float kTiny = 0x1.008p-126f;                 // normal; low 17 bits 0x4000
  bool clear = true;
#pragma unroll
  for (int i = 0; i < kBlock; ++i) {
    const uint32_t b = __float_as_uint(__builtin_fmaf(fabsf(y[i]), rg, kTiny));
    clear &= (b << 15) + (kScreenUlps << 15) >= ((2u * kScreenUlps) << 15);
  }
  return clear;
}

// Encode one block with a given scale code S: writes the 16 nibbles packed in two dwords
// (byte k = nibble 2k | nibble 2k+1 << 4); a zero scale gives an all-zero block.
//
// Fast path: the exact quotient Q = |y| / (sigma g) is bracketed by q1 = |y| R (1 - 2^-20) and
// q2 = |y| R (1 + 2^-20), R = rcp(fl(sigma g)): the reciprocal (1 ulp), the product sigma g
// and the two multiplications stay within 3 ulp (3 * 2^-23) of the exact factors, far inside
// the 2^-20 margin, so q1 < Q < q2 whenever sigma g is a normal number.  Round to nearest is
// monotonic, so when the converter gives both brackets the same code that code is RNE(Q),
// exactly the decision of the bound-based encoder.  Where they differ (Q within about 2^-20
// of a midpoint, a few elements in a million) the block takes the exact bound-based encoder.
__device__ __forceinline__ void encode_block_sigma(const float (&y)[kBlock], float g, float sigma, uint32_t& lo,
                                                   uint32_t& hi) {
#pragma clang fp contract(off)
  const float u = sigma * g;
  const float R = __builtin_amdgcn_rcpf(u);
  const float r1 = R * kBracketDown, r2 = R * kBracketUp;
  const uint32_t l1 = cvt_pack8(&y[0], r1), l2 = cvt_pack8(&y[0], r2);
  const uint32_t h1 = cvt_pack8(&y[8], r1), h2 = cvt_pack8(&y[8], r2);
  uint32_t l = l1, h = h1;
  const bool exact = sigma > 0.0f && !(l1 == l2 && h1 == h2 && u >= 0x1p-125f);
  if (__builtin_expect(exact, 0)) {
    const E2m1Thresholds t(sigma, g);
    l = e2m1_pack8(&y[0], t);
    h = e2m1_pack8(&y[8], t);
  }
  l = clear_zero_signs(l);
  h = clear_zero_signs(h);
  lo = sigma > 0.0f ? l : 0u;
  hi = sigma > 0.0f ? h : 0u;
}

__device__ __forceinline__ void encode_block_with(const float (&y)[kBlock], float g, uint32_t S, uint32_t& lo,
                                                  uint32_t& hi) {
  encode_block_sigma(y, g, e4m3_value(S), lo, hi);
}

__device__ __forceinline__ float block_absmax(const float (&y)[kBlock]) {
  float A = 0.0f;
#pragma unroll
  for (int i = 0; i < kBlock; ++i) A = fmaxf(A, fabsf(y[i]));
  return A;
}

// Encode one block with the absmax-to-6 scale: returns the scale code.
__device__ __forceinline__ uint32_t encode_block(const float (&y)[kBlock], float g, uint32_t& lo,
                                                 uint32_t& hi) {
  const uint32_t S = e4m3_scale_code(block_absmax(y), g);
  encode_block_with(y, g, S, lo, hi);
  return S;
}

// Absmax-to-6 scale code through gfx950's E4M3 converter (OCP E4M3, round to nearest even),
// on the same bracketing argument as the E2M1 codes: x = A rcp(fl(6g)) is within 2^-22 of
// the exact A/(6g) (fl(6g), the reciprocal and the product), so x (1 -/+ 2^-20) bracket it,
// and where the converter gives both the same code that code is RNE of the exact quotient.
// Both are clamped to 448 first, where the code saturates (the converter is not told to
// saturate).  Returns false where the two differ (the quotient within about 2^-20 of a
// midpoint between codes); S is then unset.
__device__ __forceinline__ bool e4m3_scale_code_cvt(float A, float r6g, uint32_t& S) {
#pragma clang fp contract(off)
  const float x = A * r6g;
  const float b0 = fminf(x * kBracketDown, 448.0f), b1 = fminf(x * kBracketUp, 448.0f);
  const uint32_t w = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(b0, b1, 0, false));
  S = w & 0xFFu;
  return S == ((w >> 8) & 0xFFu);
}

// The same with the 6x midpoints (t6) read from a table: the converter decides, and the exact
// midpoint tests decide where its two brackets differ.  The scale value comes from the
// converter too (codes 0..126 are exact in fp32).
__device__ __forceinline__ uint32_t encode_block_t(const float (&y)[kBlock], float g, float r6g, const float* t6,
                                                   uint32_t& lo, uint32_t& hi) {
  const float A = block_absmax(y);
  uint32_t S;
  if (!e4m3_scale_code_cvt(A, r6g, S)) S = e4m3_scale_code_t(A, g, t6);
  encode_block_sigma(y, g, __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(S), 0), lo, hi);
  return S;
}

// ---------------------------------------------------------------------------------------
// MSE-searched key block scale ([OSFP4] section 1: other scales than absmax-to-6 can lower
// the FP4 distortion; section 3 and appendix C: a deterministic search over valid E4M3
// scales, block by block for round-to-nearest; appendix H: MSE-optimal E4M3 scales; section
// 2.1 and appendix A, Lemma 1: the smoothed FP4 error is flat for values between 7/4 and 7
// times the scale).  Candidates: the absmax-to-6 code S0 and every code c >= 1 with
// 7/4 <= A/(g sigma_c) <= 7; they form one run of at most kMseMaxCand codes that starts no
// lower than S0 - 2.  The smallest squared error wins; ties keep S0, then the smaller code.
//
// Ranking criterion: with u = g sigma, FP4 magnitudes m_j and y_hat_j = m_j u (sign of y_j),
//   sum (y - y_hat)^2 = sum y^2 + g J,   J = sigma (u M2 - 2P),  P = sum m_j |y_j|,  M2 = sum m_j^2.
// Each step is exact in fp64: a nonzero m_j needs |y_j| >= u/4 and every compared block has
// |y_j| <= A <= 9u, so the products m_j |y_j| lie within 37 bits of each other and their sum
// is exact in any order; u M2 has at most 28 + 12 bits, u M2 - 2P at most 42, times the 4-bit
// sigma at most 46.  So J is the exact real number and the decision needs no rounding rule.
// ---------------------------------------------------------------------------------------
constexpr int kMseMaxCand = 17;

// Twice the E2M1 magnitude of a 3-bit magnitude code: 0, 1, 2, 3, 4, 6, 8, 12.
__device__ __forceinline__ uint32_t e2m1_twice_mag(uint32_t m) { return (0xC8643210u >> (4u * m)) & 15u; }

// 2P and 4 M2 over N elements of a block (|y| given in fp64) for scale sigma > 0.  The
// magnitude codes come from the bracketing converter pass of encode_block_with when its two
// brackets agree, else from the exact bound-based encoder.
template <int N>
__device__ __forceinline__ void mse_partials(const float (&y)[N], const double (&ay)[N], float sigma, float g,
                                             double& p2, uint32_t& m4) {
#pragma clang fp contract(off)
  static_assert(N % 8 == 0, "whole packed words");
  const float u = sigma * g;
  const float R = __builtin_amdgcn_rcpf(u);
  const float r1 = R * kBracketDown, r2 = R * kBracketUp;
  uint32_t w[N / 8];
  bool same = u >= 0x1p-125f;
#pragma unroll
  for (int j = 0; j < N / 8; ++j) {
    w[j] = cvt_pack8(&y[8 * j], r1);
    same &= w[j] == cvt_pack8(&y[8 * j], r2);
  }
  if (__builtin_expect(!same, 0)) {
    const E2m1Thresholds t(sigma, g);
#pragma unroll
    for (int j = 0; j < N / 8; ++j) w[j] = e2m1_pack8(&y[8 * j], t);
  }
  p2 = 0.0;
  m4 = 0u;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const uint32_t v2 = e2m1_twice_mag((w[i / 8] >> (4 * (i % 8))) & 7u);
    p2 = __builtin_fma(static_cast<double>(v2), ay[i], p2);   // exact (see above)
    m4 += v2 * v2;
  }
}

__device__ __forceinline__ double mse_criterion(float sigma, float g, double p2, uint32_t m4) {
  const double u = static_cast<double>(g) * static_cast<double>(sigma);
  return static_cast<double>(sigma) * (u * static_cast<double>(m4) * 0.25 - p2);
}

// Is code c's scale too small for the block maximum (A > 7 g sigma_c)?  Too large (A <
// 7/4 g sigma_c)?  Both products are exact in fp32 (7 and 1.75 have 3 significant bits).
__device__ __forceinline__ bool mse_below(float s, float A, float g) { return __builtin_fmaf(-7.0f * s, g, A) > 0.0f; }
__device__ __forceinline__ bool mse_above(float s, float A, float g) { return __builtin_fmaf(-1.75f * s, g, A) < 0.0f; }

// First code of the candidate run (or a code past it when the run is empty).
__device__ __forceinline__ uint32_t mse_first_code(uint32_t S0, float A, float g) {
  uint32_t c = S0 >= 3u ? S0 - 2u : 1u;
#pragma unroll
  for (int k = 0; k < 3; ++k) c += (c < 126u && mse_below(e4m3_value(c), A, g)) ? 1u : 0u;
  return c;
}

// Criterion J of code c for a block held by one lane (c >= 1).
__device__ __forceinline__ double mse_code_criterion(const float (&y)[kBlock], const double (&ay)[kBlock], uint32_t c,
                                                     float g) {
  const float s = e4m3_value(c);
  double p2;
  uint32_t m4;
  mse_partials<kBlock>(y, ay, s, g, p2, m4);
  return mse_criterion(s, g, p2, m4);
}

// Integer form of 2P for the one-lane search.  With E = floor(log2 A), every element that
// can take a nonzero code under a scale u >= A/8 has |y_j| > u/4 >= A/32 >= 2^(E-5), so
// |y_j| = Y_j 2^(E-28) with an integer Y_j < 2^29 (smaller elements keep code 0 and their
// truncated Y_j is multiplied by 0).  The codes' twice-magnitudes k_j (0..12) are packed four
// to a dword in the order of the packed nibble words (dword 0: elements 0, 2, 4, 6; 1: 1, 3,
// 5, 7; 2: 8, 10, 12, 14; 3: 9, 11, 13, 15), and Y_j is split into bytes regrouped the same
// way, so 2P = sum over bytes b of 2^(8b) sum_j k_j byte_b(Y_j) comes from 16 four-way byte
// dot products (each partial sum below 2^16, the total below 2^40: exact in fp64), and 4 M2 =
// sum k_j^2 from 4 more.  The result equals mse_partials' exactly.
struct MseAligned {
  uint32_t yb[4][4];    // [dword d][byte b]: byte b of Y_j for the four elements of dword d
  int shift;            // E - 28
};

__device__ __forceinline__ void mse_align(const float (&y)[kBlock], float A, MseAligned& m) {
  const int E = __builtin_amdgcn_frexp_expf(A) - 1;          // A in [2^E, 2^(E+1))
  uint32_t Y[kBlock];
#pragma unroll
  for (int i = 0; i < kBlock; ++i) Y[i] = static_cast<uint32_t>(__builtin_ldexpf(fabsf(y[i]), 28 - E));
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const int e0 = 8 * (d >> 1) + (d & 1);                  // elements e0, e0 + 2, e0 + 4, e0 + 6
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      // bytes b of two elements side by side, then the two pairs side by side
      const uint32_t sel = static_cast<uint32_t>(b) | (static_cast<uint32_t>(b + 4) << 8);
      const uint32_t lo = __builtin_amdgcn_perm(Y[e0 + 2], Y[e0], sel);
      const uint32_t hi = __builtin_amdgcn_perm(Y[e0 + 6], Y[e0 + 4], sel);
      m.yb[d][b] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
    }
  }
  m.shift = E - 28;
}

// 2P and 4 M2 of one candidate from its packed codes (nibble i = element i, words w0, w1).
__device__ __forceinline__ void mse_partials_aligned(uint32_t w0, uint32_t w1, const MseAligned& m, double& p2,
                                                     uint32_t& m4) {
  // twice-magnitude of each 3-bit magnitude code by a byte table lookup: 0 1 2 3 4 6 8 12
  const uint32_t kd[4] = {__builtin_amdgcn_perm(0x0C080604u, 0x03020100u, w0 & 0x07070707u),
                          __builtin_amdgcn_perm(0x0C080604u, 0x03020100u, (w0 >> 4) & 0x07070707u),
                          __builtin_amdgcn_perm(0x0C080604u, 0x03020100u, w1 & 0x07070707u),
                          __builtin_amdgcn_perm(0x0C080604u, 0x03020100u, (w1 >> 4) & 0x07070707u)};
  uint32_t q = 0u;
  uint32_t pb[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    q = __builtin_amdgcn_udot4(kd[d], kd[d], q, false);
#pragma unroll
    for (int b = 0; b < 4; ++b) pb[b] = __builtin_amdgcn_udot4(kd[d], m.yb[d][b], pb[b], false);
  }
  m4 = q;
  const uint32_t lo = pb[0] + (pb[1] << 8), hi = pb[2] + (pb[3] << 8);     // each below 2^25
  p2 = __builtin_ldexp(__builtin_fma(static_cast<double>(hi), 65536.0, static_cast<double>(lo)), m.shift);
}

// Criterion J of code c (c >= 1, u = g sigma_c >= A/8) from the aligned block.
// A block that passed the midpoint screen (clear) takes one converter pass.
__device__ __forceinline__ double mse_code_criterion_aligned(const float (&y)[kBlock], const MseAligned& m, uint32_t c,
                                                             float g, bool clear) {
#pragma clang fp contract(off)
  const float s = e4m3_value(c);
  const float u = s * g;
  const float R = __builtin_amdgcn_rcpf(u);
  const bool fast = clear && u >= 0x1p-125f;
  const float r1 = fast ? R : R * kBracketDown;
  uint32_t w0 = cvt_pack8(&y[0], r1), w1 = cvt_pack8(&y[8], r1);
  bool same = true;
  if (!fast) {
    const float r2 = R * kBracketUp;
    same = u >= 0x1p-125f && w0 == cvt_pack8(&y[0], r2) && w1 == cvt_pack8(&y[8], r2);
  }
  if (__builtin_expect(!same, 0)) {
    const E2m1Thresholds t(s, g);
    w0 = e2m1_pack8(&y[0], t);
    w1 = e2m1_pack8(&y[8], t);
  }
  double p2;
  uint32_t m4;
  mse_partials_aligned(w0, w1, m, p2, m4);
  return mse_criterion(s, g, p2, m4);
}

// Search for a block held by one lane, in the order of the definition: S0 first, then the run
// in increasing code order, a candidate replacing the best only when strictly better.  When S0
// lies in the run (its scale maps the absmax near 6, so nearly always) it is evaluated at its
// place in the run instead, and it takes a tie with the best so far: the same result with one
// evaluation fewer.  The run's codes all have g sigma >= A/7, so they take the integer form;
// S0 outside the run does too unless its scale is below A/8 (a saturated block), where it
// takes the fp64 form.
__device__ __forceinline__ uint32_t mse_scale_code(const float (&y)[kBlock], float A, float g, uint32_t S0,
                                                  bool clear) {
#pragma clang fp contract(off)
  MseAligned m;
  mse_align(y, A, m);
  uint32_t best = S0;
  double best_j = 0.0;
  if (S0) {
    const float s0 = e4m3_value(S0);
    if (!mse_below(s0, A, g) && !mse_above(s0, A, g)) {
      best_j = __builtin_inf();                       // S0 comes up in the run
    } else if (__builtin_fmaf(-8.0f * s0, g, A) <= 0.0f) {      // A <= 8 g sigma_0, exactly
      best_j = mse_code_criterion_aligned(y, m, S0, g, clear);
    } else {
      double ay[kBlock];
#pragma unroll
      for (int i = 0; i < kBlock; ++i) ay[i] = static_cast<double>(fabsf(y[i]));
      best_j = mse_code_criterion(y, ay, S0, g);
    }
  }
  uint32_t c = mse_first_code(S0, A, g);
  for (int k = 0; k < kMseMaxCand; ++k, ++c) {
    if (c > 126u) break;
    const float s = e4m3_value(c);
    if (mse_above(s, A, g)) break;                 // this code and every larger one
    if (mse_below(s, A, g)) continue;
    const double j = mse_code_criterion_aligned(y, m, c, g, clear);
    if (j < best_j || (c == S0 && j == best_j)) {
      best_j = j;
      best = c;
    }
  }
  return best;
}

// Keep the smaller (J, rank) of this lane's and the lane that DPP control CTRL names.
template <int CTRL>
__device__ __forceinline__ void mse_keep_best_dpp(double& best_j, int& best_rank, uint32_t& best) {
  const uint64_t jb = __builtin_bit_cast(uint64_t, best_j);
  const uint32_t jlo = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(jb), CTRL, 0xF, 0xF, true));
  const uint32_t jhi =
      static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(jb >> 32), CTRL, 0xF, 0xF, true));
  const double oj = __builtin_bit_cast(double, static_cast<uint64_t>(jlo) | (static_cast<uint64_t>(jhi) << 32));
  const int orank = __builtin_amdgcn_mov_dpp(best_rank, CTRL, 0xF, 0xF, true);
  const uint32_t oc = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(best), CTRL, 0xF, 0xF, true));
  if (oj < best_j || (oj == best_j && orank < best_rank)) {
    best_j = oj;
    best_rank = orank;
    best = oc;
  }
}

// Search for the 8 blocks of a 128-element row staged in LDS (row[128]), by a whole
// wavefront: lane L takes block L >> 3 and evaluates entries v = (L & 7) + 8t, t = 0, 1, 2,
// of the block's candidate list: entry v < kMseMaxCand is code first + v of the run, entry
// kMseMaxCand is S0 when S0 lies outside the run (inside it, S0 is one of the run's
// entries).  The block's eight lanes then keep the smallest (J, rank), rank = -1 for S0 and
// the code otherwise, which is the order of the one-lane search.  A run spans a factor of 4
// in scale, which holds 16 E4M3 values unless both ends are values, and S0 maps the absmax
// near 6, inside the run, so the third round usually has no entry in any block: it runs only
// when some lane has one.  The call must be reached by all 64 lanes; every lane returns its
// block's code.
__device__ __forceinline__ uint32_t mse_scale_code_row(const float* row, float g, int lane) {
#pragma clang fp contract(off)
  const int sub = lane & 7;
  float y[kBlock];
  const float4* src = reinterpret_cast<const float4*>(row + kBlock * (lane >> 3));
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 v = src[q];
    y[4 * q] = v.x;
    y[4 * q + 1] = v.y;
    y[4 * q + 2] = v.z;
    y[4 * q + 3] = v.w;
  }
  double ay[kBlock];
#pragma unroll
  for (int i = 0; i < kBlock; ++i) ay[i] = static_cast<double>(fabsf(y[i]));
  const float A = block_absmax(y);
  const uint32_t S0 = e4m3_scale_code(A, g);
  const uint32_t first = mse_first_code(S0, A, g);
  bool s0_in_run = false;
  if (S0) {
    const float s = e4m3_value(S0);
    s0_in_run = !mse_below(s, A, g) && !mse_above(s, A, g);
  }
  double best_j = __builtin_inf();
  int best_rank = 0x7FFFFFFF;
  uint32_t best = S0;
  static_assert(2 * 8 < kMseMaxCand && 3 * 8 > kMseMaxCand, "two full rounds, then the rest");
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    const int v = sub + 8 * t;
    uint32_t c = S0;
    bool valid = v == kMseMaxCand && !s0_in_run;
    if (v < kMseMaxCand) {
      c = first + static_cast<uint32_t>(v);
      valid = false;
      if (c <= 126u) {
        const float s = e4m3_value(c);
        valid = !mse_below(s, A, g) && !mse_above(s, A, g);
      }
    }
    if (!valid) continue;                   // the third round: skipped when no lane has an entry
    const double j = c == 0u ? 0.0 : mse_code_criterion(y, ay, c, g);
    const int rank = c == S0 ? -1 : static_cast<int>(c);
    if (j < best_j || (j == best_j && rank < best_rank)) {
      best_j = j;
      best_rank = rank;
      best = c;
    }
  }
  // the block's eight lanes by DPP: pairs (xor 1), quads (xor 2), then the mirrored half row
  // (lane i of the eight takes lane 7 - i, in the other quad)
  mse_keep_best_dpp<0xB1>(best_j, best_rank, best);
  mse_keep_best_dpp<0x4E>(best_j, best_rank, best);
  mse_keep_best_dpp<0x141>(best_j, best_rank, best);
  return best;
}

// Encode one block with the MSE-searched scale: returns the scale code.
__device__ __forceinline__ uint32_t encode_block_mse(const float (&y)[kBlock], float g, uint32_t& lo,
                                                     uint32_t& hi) {
  const float A = block_absmax(y);
  const bool clear = clear_of_midpoints(y, __builtin_amdgcn_rcpf(g));
  uint32_t S0;
  if (!e4m3_scale_code_cvt(A, __builtin_amdgcn_rcpf(6.0f * g), S0)) S0 = e4m3_scale_code(A, g);
  const uint32_t S = mse_scale_code(y, A, g, S0, clear);
  encode_block_with(y, g, S, lo, hi);
  return S;
}

// The 16 bf16 elements of a block, held as two 16-byte words, as fp32 (exact).
__device__ __forceinline__ void unpack_bf16_block(const uint4& raw0, const uint4& raw1, float (&y)[kBlock]) {
  const uint32_t w[8] = {raw0.x, raw0.y, raw0.z, raw0.w, raw1.x, raw1.y, raw1.z, raw1.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    y[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
    y[2 * i + 1] = bf16_to_f32(w[i] >> 16);
  }
}

// Load this lane's 16 bf16 elements as fp32.
__device__ __forceinline__ void load_block_bf16(const uint16_t* __restrict__ src, float (&y)[kBlock],
                                                uint4& raw0, uint4& raw1) {
  const uint4* p = reinterpret_cast<const uint4*>(src);
  raw0 = p[0];
  raw1 = p[1];
  unpack_bf16_block(raw0, raw1, y);
}

}  // namespace nvkv

