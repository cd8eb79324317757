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

// Per-block E2M1 thresholds P_k = t_k * sigma (exact), t = midpoints of the magnitude grid
// {0, .5, 1, 1.5, 2, 3, 4, 6}.
struct E2m1Thresholds {
  float p0, p1, p2, p3, p4, p5, p6;
  __device__ __forceinline__ explicit E2m1Thresholds(float sigma)
      : p0(0.25f * sigma), p1(0.75f * sigma), p2(1.25f * sigma), p3(1.75f * sigma),
        p4(2.5f * sigma), p5(3.5f * sigma), p6(5.0f * sigma) {
    // keep the seven products in registers: left to itself the compiler re-forms them at
    // every use and turns the threshold selects of all 16 elements into branches
    asm volatile("" : "+v"(p0), "+v"(p1), "+v"(p2), "+v"(p3), "+v"(p4), "+v"(p5), "+v"(p6));
  }
};

// Signed E2M1 nibble of y in a block with scale sigma > 0 and tensor scale g: magnitude =
// round-to-nearest (ties to the even code) of the exact |y|/(sigma g), saturating at 6;
// a zero magnitude is stored as code 0.  Three exact comparisons (binary search).
__device__ __forceinline__ uint32_t e2m1_nibble(float y, const E2m1Thresholds& t, float g) {
#pragma clang fp contract(off)
  const float a = fabsf(y);
  const bool b2 = __builtin_fmaf(-t.p3, g, a) >= 0.0f;            // 1.75: tie -> code 4
  // threshold choices as bit selects on all-ones / all-zero masks (nested conditional
  // expressions are compiled to branches here)
  const uint32_t m2 = b2 ? 0xFFFFFFFFu : 0u;
  const float t1 = __uint_as_float((__float_as_uint(t.p5) & m2) | (__float_as_uint(t.p1) & ~m2));  // 3.5 / 0.75: tie -> up
  const bool b1 = __builtin_fmaf(-t1, g, a) >= 0.0f;
  const uint32_t m1 = b1 ? 0xFFFFFFFFu : 0u;
  const uint32_t hi2 = (__float_as_uint(t.p6) & m1) | (__float_as_uint(t.p4) & ~m1);
  const uint32_t lo2 = (__float_as_uint(t.p2) & m1) | (__float_as_uint(t.p0) & ~m1);
  const float t0 = __uint_as_float((hi2 & m2) | (lo2 & ~m2));      // 5, 2.5, 1.25, 0.25: tie -> down
  const bool b0 = __builtin_fmaf(-t0, g, a) > 0.0f;
  const uint32_t m = (uint32_t(b2) << 2) | (uint32_t(b1) << 1) | uint32_t(b0);
  const uint32_t sign = (__float_as_uint(y) >> 28) & 8u;
  return m | (m ? sign : 0u);
}

// Encode one block: returns the scale code, writes the 16 nibbles packed in two dwords
// (byte k = nibble 2k | nibble 2k+1 << 4).
__device__ __forceinline__ uint32_t encode_block(const float (&y)[kBlock], float g, uint32_t& lo,
                                                 uint32_t& hi) {
#pragma clang fp contract(off)
  float A = 0.0f;
#pragma unroll
  for (int i = 0; i < kBlock; ++i) A = fmaxf(A, fabsf(y[i]));
  const uint32_t S = e4m3_scale_code(A, g);
  const float sigma = e4m3_value(S);
  // straight-line: a zero scale (underflowing block) masks the codes to 0 afterwards
  const E2m1Thresholds t(sigma);
  uint32_t l = 0u, h = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) l |= e2m1_nibble(y[i], t, g) << (4 * i);
#pragma unroll
  for (int i = 0; i < 8; ++i) h |= e2m1_nibble(y[8 + i], t, g) << (4 * i);
  lo = sigma > 0.0f ? l : 0u;
  hi = sigma > 0.0f ? h : 0u;
  return S;
}

// Load this lane's 16 bf16 elements as fp32.
__device__ __forceinline__ void load_block_bf16(const uint16_t* __restrict__ src, float (&y)[kBlock],
                                                uint4& raw0, uint4& raw1) {
#pragma clang fp contract(off)
  const uint4* p = reinterpret_cast<const uint4*>(src);
  raw0 = p[0];
  raw1 = p[1];
  const uint32_t w[8] = {raw0.x, raw0.y, raw0.z, raw0.w, raw1.x, raw1.y, raw1.z, raw1.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    y[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
    y[2 * i + 1] = bf16_to_f32(w[i] >> 16);
  }
}

}  // namespace nvkv

