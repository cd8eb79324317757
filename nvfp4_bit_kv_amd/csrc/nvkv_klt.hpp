// Static per-head KLT key basis: device helpers shared by the calibration, append, decode
// and prefill kernels (gfx950).
//
// Source: [cache post] = rstation.ai post "NVFP4 attention cache on W4A4 Qwen3-8B: static key
// smoothing is near-lossless, key rotations hurt", cache-config table rows "K: static
// per-head KLT" and "K: static KLT + smoothing".  The basis B of a KV head is fp32 [128][128]
// (element (j, i) at j*128 + i; column i = basis vector i).  Keys are rotated z = B^T y with a
// fixed rounding order (rotate_cols: a chain of fused multiply-adds), which is part of the
// bit-exact encoding; the query side q' = B^T (q * s) is not an encoding step and may round in
// any order.
#pragma once

#include "nvkv_device.hpp"

namespace nvkv {

constexpr int kBasisFloats = kHeadDim * kHeadDim;

// Copy one head's basis into LDS with every thread of the workgroup (no barrier inside).
__device__ __forceinline__ void load_basis_lds(const float* __restrict__ basis_h, float* lds, int tid,
                                               int nthreads) {
  const float4* src = reinterpret_cast<const float4*>(basis_h);
  float4* dst = reinterpret_cast<float4*>(lds);
  for (int i = tid; i < kBasisFloats / 4; i += nthreads) dst[i] = src[i];
}

// One wavefront copies a quarter of the basis (rows 32q .. 32q+31), all 16 of each lane's
// loads issued before its stores.
__device__ __forceinline__ void load_basis_quarter(const float* __restrict__ basis_h, float* lds, int quarter,
                                                   int lane) {
  const float4* src = reinterpret_cast<const float4*>(basis_h) + quarter * (kBasisFloats / 16);
  float4* dst = reinterpret_cast<float4*>(lds) + quarter * (kBasisFloats / 16);
  float4 v[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) v[k] = src[64 * k + lane];
#pragma unroll
  for (int k = 0; k < 16; ++k) dst[64 * k + lane] = v[k];
}

// z_k = sum over j = 0..127 of B[j][c0 + k] * row[j], k < N (a multiple of 4, c0 a multiple
// of 4), as a chain of fp32 fused multiply-adds in j: z <- fl32(B[j][c0 + k] * row[j] + z)
// from z = 0, one rounding per step: the key rotation's rounding order.  B and row may be in
// LDS or global memory.
template <int N>
__device__ __forceinline__ void rotate_cols(const float* B, const float* row, int c0, float (&z)[N]) {
#pragma unroll
  for (int k = 0; k < N; ++k) z[k] = 0.0f;
#pragma unroll 4
  for (int j = 0; j < kHeadDim; ++j) {
    const float yj = row[j];
    const float4* bj = reinterpret_cast<const float4*>(B + j * kHeadDim + c0);
#pragma unroll
    for (int k = 0; k < N / 4; ++k) {
      const float4 b = bj[k];
      z[4 * k + 0] = __builtin_fmaf(b.x, yj, z[4 * k + 0]);
      z[4 * k + 1] = __builtin_fmaf(b.y, yj, z[4 * k + 1]);
      z[4 * k + 2] = __builtin_fmaf(b.z, yj, z[4 * k + 2]);
      z[4 * k + 3] = __builtin_fmaf(b.w, yj, z[4 * k + 3]);
    }
  }
}

}  // namespace nvkv
