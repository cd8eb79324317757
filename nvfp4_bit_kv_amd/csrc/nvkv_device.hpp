// Device-side building blocks shared by the quantise, calibrate and decode kernels (gfx950).
//
// Number formats ([OSFP4] = paperlayer.ai summary of arXiv 2610.08231v1, "OSFP4: Joint
// Optimization of Diagonal Smoothing and Block Scales for NVFP4 Quantization"):
//   E2M1 element codes (largest magnitude 6, section 1), E4M3 scale per 16 elements and an
//   fp32 tensor scale (appendix D.1); the scale constellation is the positive E4M3 points
//   (appendix I).  E4M3 here is the OCP E4M3FN variant (bias 7, max 448, no infinities).
//
// Every quantisation decision is taken on the EXACT real quotient.  A quotient a/(t*g)
// against a grid midpoint t is decided by the sign of fma(-t, g, a): the product t*g is
// formed exactly inside the FMA and the single rounding of the difference cannot change its
// sign (for the operand ranges met here the exact difference is far above the smallest
// subnormal).  All midpoint-times-scale constants are exact fp32 values (at most 7
// significant bits), so no division or reciprocal enters a decision.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvkv {

constexpr int kHeadDim = 128;
constexpr int kBlock = 16;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16 bits, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Value of a non-negative E4M3FN code 0..126, exact in fp32.  Normal codes (exponent field
// e >= 1, mantissa m) are 2^(e-7) (1 + m/8): the fp32 pattern with exponent e + 120 and the
// three mantissa bits on top, i.e. (c + 960) << 20.  Subnormal codes are m * 2^-9.
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const float sub = static_cast<float>(c) * 0x1p-9f;
  const float nrm = __uint_as_float((c + 960u) << 20);
  return c < 8u ? sub : nrm;
}

// Neighbours of a positive finite fp32 value (bit-pattern steps).
__device__ __forceinline__ float next_up_pos(float x) { return __uint_as_float(__float_as_uint(x) + 1u); }
__device__ __forceinline__ float next_down_pos(float x) { return __uint_as_float(__float_as_uint(x) - 1u); }

// Correctly rounded fp32 square root of a > 0.  A candidate from the fp64 square root is
// moved to the neighbour whose rounding interval holds sqrt(a): the interval ends are the
// midpoints to the adjacent fp32 values (at most 26 significant bits), so their squares are
// exact in fp64 and each comparison with a is exact.  No exact tie exists (a midpoint's
// square has at least 49 significant bits, a has 24).
__device__ __forceinline__ float sqrt_rn_f32(float a) {
  const double ad = a;
  float s = static_cast<float>(sqrt(ad));
  for (int i = 0; i < 3; ++i) {
    const double hi = 0.5 * (static_cast<double>(s) + static_cast<double>(next_up_pos(s)));
    if (ad > hi * hi) { s = next_up_pos(s); continue; }
    const double lo = 0.5 * (static_cast<double>(s) + static_cast<double>(next_down_pos(s)));
    if (s > 0.0f && ad < lo * lo) { s = next_down_pos(s); continue; }
    break;
  }
  return s;
}

// Correctly rounded fp32 quotient n/d for n, d > 0, by the same midpoint test: a midpoint
// (<= 26 bits) times d (24 bits) is exact in fp64; no exact tie exists.
__device__ __forceinline__ float div_rn_f32(float n, float d) {
  const double nd = n, dd = d;
  float q = static_cast<float>(nd / dd);
  for (int i = 0; i < 3; ++i) {
    const double hi = 0.5 * (static_cast<double>(q) + static_cast<double>(next_up_pos(q)));
    if (nd > hi * dd) { q = next_up_pos(q); continue; }
    const double lo = 0.5 * (static_cast<double>(q) + static_cast<double>(next_down_pos(q)));
    if (q > 0.0f && nd < lo * dd) { q = next_down_pos(q); continue; }
    break;
  }
  return q;
}

}  // namespace nvkv
