// Calibration of the static per-head KLT key basis (gfx950).  Compiled with
// -ffp-contract=off (the g_K pass applies the key rotation in its fixed rounding order).
//
// Source: [cache post] = rstation.ai post "NVFP4 attention cache on W4A4 Qwen3-8B: static key
// smoothing is near-lossless, key rotations hurt", cache-config table rows "K: static
// per-head KLT" and "K: static KLT + smoothing": a fixed per-head basis computed once from
// calibration keys (after the static smoothing when both are selected).
//
// Three steps per head, each one workgroup per head except the last:
//   1. covariance: the mean of the (smoothed) keys over the calibration rows, then the fp64
//      sum of outer products of the centred rows, in row order (deterministic);
//   2. eigendecomposition: cyclic two-sided Jacobi in fp64 with the round-robin ordering (64
//      disjoint rotations per round, 127 rounds per sweep), the matrix in LDS and the
//      eigenvectors in the workspace; then columns sorted by decreasing eigenvalue, signed so
//      the largest-magnitude entry is positive (ties within a relative 1e-6: the first), and
//      rounded to fp32;
//   3. g_K: the keys of every position smoothed and rotated by the fp32 basis (the append
//      kernel's rounding order), max |z| -> g_K = fl32(A_K / 2688).
#include "nvkv_klt.hpp"
#include "nvkv_internal.hpp"

namespace nvkv {

constexpr int kCovRows = 32;             // rows staged per chunk
constexpr int kJacobiMaxSweeps = 24;
constexpr int kAStride = kHeadDim + 1;   // padded LDS row (column accesses spread over banks)
constexpr double kSignTie = 1e-6;

// x (bf16 bits) -> fp32 key, smoothed by r when smooth (one fp32 multiply).
__device__ __forceinline__ float smoothed_key(uint16_t bits, const float* r, int j, bool smooth) {
#pragma clang fp contract(off)
  const float x = bf16_to_f32(bits);
  return smooth ? x * r[j] : x;
}

// grid: Hkv, block 256.  cov[h] = (1/n) sum (y - mean)(y - mean)^T over the n = W (T - t_begin)
// calibration rows of head h.
__global__ void __launch_bounds__(256) k_klt_covariance(const uint16_t* __restrict__ k_win, int W, int T, int hkv,
                                                        int t_begin, const float* __restrict__ r, int smooth,
                                                        double* __restrict__ cov) {
  const int h = blockIdx.x, tid = threadIdx.x;
  __shared__ float rows[kCovRows][kHeadDim];
  __shared__ double mean[kHeadDim];
  const int per_w = T - t_begin;
  const int64_t n_rows = static_cast<int64_t>(W) * per_w;
  const float* rh = smooth ? r + h * kHeadDim : nullptr;

  auto stage = [&](int64_t r0) {
    for (int e = tid; e < kCovRows * kHeadDim; e += 256) {
      const int rr = e >> 7, j = e & 127;
      const int64_t gr = r0 + rr;
      float y = 0.0f;
      if (gr < n_rows) {
        const int64_t w = gr / per_w, t = t_begin + gr % per_w;
        y = smoothed_key(k_win[((w * T + t) * hkv + h) * kHeadDim + j], rh, j, smooth != 0);
      }
      rows[rr][j] = y;
    }
  };

  double msum = 0.0;
  for (int64_t r0 = 0; r0 < n_rows; r0 += kCovRows) {
    stage(r0);
    __syncthreads();
    const int n = static_cast<int>(min<int64_t>(kCovRows, n_rows - r0));
    if (tid < kHeadDim)
      for (int rr = 0; rr < n; ++rr) msum += static_cast<double>(rows[rr][tid]);
    __syncthreads();
  }
  if (tid < kHeadDim) mean[tid] = msum / static_cast<double>(n_rows);
  __syncthreads();

  const int i0 = (tid >> 4) * 8, j0 = (tid & 15) * 8;
  double mi[8], mj[8];
#pragma unroll
  for (int a = 0; a < 8; ++a) {
    mi[a] = mean[i0 + a];
    mj[a] = mean[j0 + a];
  }
  double acc[8][8];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[a][b] = 0.0;
  for (int64_t r0 = 0; r0 < n_rows; r0 += kCovRows) {
    stage(r0);
    __syncthreads();
    const int n = static_cast<int>(min<int64_t>(kCovRows, n_rows - r0));
    for (int rr = 0; rr < n; ++rr) {
      double di[8], dj[8];
#pragma unroll
      for (int a = 0; a < 8; ++a) {
        di[a] = static_cast<double>(rows[rr][i0 + a]) - mi[a];
        dj[a] = static_cast<double>(rows[rr][j0 + a]) - mj[a];
      }
#pragma unroll
      for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int b = 0; b < 8; ++b) acc[a][b] = __builtin_fma(di[a], dj[b], acc[a][b]);
    }
    __syncthreads();
  }
  const double inv_n = 1.0 / static_cast<double>(n_rows);
  double* out = cov + static_cast<int64_t>(h) * kBasisFloats;
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) out[(i0 + a) * kHeadDim + j0 + b] = acc[a][b] * inv_n;
}

// Block-wide sum of two values over 256 threads (every thread gets the totals).
__device__ __forceinline__ void block_sum2(double& x, double& y, double* red) {
  const int tid = threadIdx.x;
  red[tid] = x;
  red[256 + tid] = y;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) {
      red[tid] += red[tid + s];
      red[256 + tid] += red[256 + tid + s];
    }
    __syncthreads();
  }
  x = red[0];
  y = red[256];
  __syncthreads();
}

// grid: Hkv, block 256.  Jacobi eigendecomposition of cov[h]; writes basis_out[h] (fp32).
// vmat: fp64 [Hkv][128][128] workspace for the eigenvectors; row i is read and written only by
// thread i during the sweeps.
__global__ void __launch_bounds__(256) k_klt_jacobi(const double* __restrict__ cov, double* __restrict__ vmat,
                                                    float* __restrict__ basis_out) {
  const int h = blockIdx.x, tid = threadIdx.x;
  __shared__ double A[kHeadDim * kAStride];
  __shared__ double red[512];
  __shared__ double cs[64], sn[64];
  __shared__ int pp[64], qq[64];
  __shared__ double lam[kHeadDim];
  const double* C = cov + static_cast<int64_t>(h) * kBasisFloats;
  double* V = vmat + static_cast<int64_t>(h) * kBasisFloats;
  for (int e = tid; e < kBasisFloats; e += 256) A[(e >> 7) * kAStride + (e & 127)] = C[e];
  if (tid < kHeadDim)
    for (int j = 0; j < kHeadDim; ++j) V[tid * kHeadDim + j] = j == tid ? 1.0 : 0.0;
  __syncthreads();

  for (int sweep = 0; sweep < kJacobiMaxSweeps; ++sweep) {
    double off = 0.0, dg = 0.0;
    for (int e = tid; e < kBasisFloats; e += 256) {
      const int i = e >> 7, j = e & 127;
      const double a = A[i * kAStride + j];
      if (i != j) off += a * a; else dg += a * a;
    }
    block_sum2(off, dg, red);
    if (!(off > 1e-30 * dg)) break;                  // uniform: converged (or a zero matrix)
    for (int round = 0; round < kHeadDim - 1; ++round) {
      if (tid < 64) {
        // round-robin pairing: player 127 meets `round`; the others pair round +- k (mod 127)
        int p = tid == 0 ? kHeadDim - 1 : (round + tid) % (kHeadDim - 1);
        int q = tid == 0 ? round : (round + (kHeadDim - 1) - tid) % (kHeadDim - 1);
        if (p > q) {
          const int t = p;
          p = q;
          q = t;
        }
        const double apq = A[p * kAStride + q];
        double c = 1.0, s = 0.0;
        if (apq != 0.0) {
          const double theta = (A[q * kAStride + q] - A[p * kAStride + p]) / (2.0 * apq);
          const double t = (theta >= 0.0 ? 1.0 : -1.0) / (fabs(theta) + sqrt(theta * theta + 1.0));
          c = 1.0 / sqrt(t * t + 1.0);
          s = t * c;
        }
        cs[tid] = c;
        sn[tid] = s;
        pp[tid] = p;
        qq[tid] = q;
      }
      __syncthreads();
      for (int e = tid; e < 64 * kHeadDim; e += 256) {     // rows p, q: A <- P^T A
        const int k = e >> 7, j = e & 127;
        const int p = pp[k], q = qq[k];
        const double c = cs[k], s = sn[k];
        const double a = A[p * kAStride + j], b = A[q * kAStride + j];
        A[p * kAStride + j] = c * a - s * b;
        A[q * kAStride + j] = s * a + c * b;
      }
      __syncthreads();
      for (int e = tid; e < 64 * kHeadDim; e += 256) {     // columns p, q: A <- A P
        const int k = e >> 7, i = e & 127;
        const int p = pp[k], q = qq[k];
        const double c = cs[k], s = sn[k];
        const double a = A[i * kAStride + p], b = A[i * kAStride + q];
        A[i * kAStride + p] = c * a - s * b;
        A[i * kAStride + q] = s * a + c * b;
      }
      if (tid < kHeadDim) {                                // V <- V P, row tid
        double* vr = V + tid * kHeadDim;
        for (int k0 = 0; k0 < 64; k0 += 16) {
          double va[16], vb[16];
#pragma unroll
          for (int k = 0; k < 16; ++k) {
            va[k] = vr[pp[k0 + k]];
            vb[k] = vr[qq[k0 + k]];
          }
#pragma unroll
          for (int k = 0; k < 16; ++k) {
            const double c = cs[k0 + k], s = sn[k0 + k];
            vr[pp[k0 + k]] = c * va[k] - s * vb[k];
            vr[qq[k0 + k]] = s * va[k] + c * vb[k];
          }
        }
      }
      __syncthreads();
    }
  }

  // eigenvalues; eigenvector rows into LDS (the matrix is no longer needed)
  if (tid < kHeadDim) lam[tid] = A[tid * kAStride + tid];
  __syncthreads();
  if (tid < kHeadDim)
    for (int j = 0; j < kHeadDim; ++j) A[tid * kAStride + j] = V[tid * kHeadDim + j];
  __syncthreads();
  if (tid < kHeadDim) {
    const int c = tid;
    const double lc = lam[c];
    int rank = 0;
    for (int j = 0; j < kHeadDim; ++j) rank += (lam[j] > lc) || (lam[j] == lc && j < c);
    double amax = 0.0;
    for (int j = 0; j < kHeadDim; ++j) amax = fmax(amax, fabs(A[j * kAStride + c]));
    int jsel = 0;
    for (int j = kHeadDim - 1; j >= 0; --j)
      if (fabs(A[j * kAStride + c]) >= (1.0 - kSignTie) * amax) jsel = j;
    const double sgn = A[jsel * kAStride + c] < 0.0 ? -1.0 : 1.0;
    float* out = basis_out + static_cast<int64_t>(h) * kBasisFloats;
    for (int j = 0; j < kHeadDim; ++j) out[j * kHeadDim + rank] = static_cast<float>(sgn * A[j * kAStride + c]);
  }
}

// grid: (ceil(W*T / 128), Hkv), block 256 (4 wavefronts x 4 passes x 8 rows).  Max |z| of the
// smoothed, rotated keys of every position -> atomicMax on the fp32 bits of g_bits[0].
__global__ void __launch_bounds__(256) k_klt_key_amax(const uint16_t* __restrict__ k_win, int64_t n_rows, int hkv,
                                                      const float* __restrict__ r, int smooth,
                                                      const float* __restrict__ basis, uint32_t* g_bits) {
  const int h = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int blk = lane >> 3, tok = lane & 7;
  __shared__ __attribute__((aligned(16))) float B[kBasisFloats];
  __shared__ __attribute__((aligned(16))) float rows[4][8][kHeadDim];
  load_basis_lds(basis + static_cast<int64_t>(h) * kBasisFloats, B, tid, 256);
  __syncthreads();
  const float* rh = smooth ? r + h * kHeadDim : nullptr;
  float m = 0.0f;
  for (int pass = 0; pass < 4; ++pass) {
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 128 + wave * 32 + pass * 8 + tok;
    const int64_t rw = row < n_rows ? row : n_rows - 1;       // clamped copy; counted anyway (a real row)
    const uint16_t* src = k_win + (rw * hkv + h) * kHeadDim + blk * kBlock;
#pragma unroll
    for (int i = 0; i < kBlock; ++i) rows[wave][tok][blk * kBlock + i] = smoothed_key(src[i], rh, blk * kBlock + i, smooth != 0);
    float z[kBlock];
    rotate_cols<kBlock>(B, rows[wave][tok], blk * kBlock, z);
#pragma unroll
    for (int i = 0; i < kBlock; ++i) m = fmaxf(m, fabsf(z[i]));
  }
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) m = fmaxf(m, __shfl_xor(m, d, 64));
  if (lane == 0) atomicMax(g_bits, __float_as_uint(m));
}

__global__ void k_klt_clear_g(uint32_t* g_bits) {
  if (threadIdx.x == 0) g_bits[0] = 0u;
}

// g_K = fl32(A / 2688), 1 where A = 0 (correctly rounded).
__global__ void k_klt_finalize_g(float* g_out) {
  if (threadIdx.x != 0) return;
  const float A = __uint_as_float(reinterpret_cast<uint32_t*>(g_out)[0]);
  g_out[0] = A == 0.0f ? 1.0f : div_rn_f32(A, 2688.0f);
}

size_t klt_workspace_bytes(int32_t hkv) {
  return static_cast<size_t>(hkv) * kBasisFloats * sizeof(double) * 2;
}

hipError_t launch_calibrate_basis(const uint16_t* k_win, int32_t W, int32_t T, int32_t hkv, int32_t exclude_pos0,
                                  uint32_t k_flags, const float* r, float* basis_out, float* g_out, void* workspace,
                                  hipStream_t stream) {
  double* cov = static_cast<double*>(workspace);
  double* vmat = cov + static_cast<size_t>(hkv) * kBasisFloats;
  const int smooth = (k_flags & NVKV_K_SMOOTH) ? 1 : 0;
  const int t_begin = exclude_pos0 ? 1 : 0;
  hipLaunchKernelGGL(k_klt_covariance, dim3(hkv), dim3(256), 0, stream, k_win, W, T, hkv, t_begin, r, smooth, cov);
  hipLaunchKernelGGL(k_klt_jacobi, dim3(hkv), dim3(256), 0, stream, cov, vmat, basis_out);
  uint32_t* g_bits = reinterpret_cast<uint32_t*>(g_out);
  hipLaunchKernelGGL(k_klt_clear_g, dim3(1), dim3(64), 0, stream, g_bits);
  const int64_t rows = static_cast<int64_t>(W) * T;
  hipLaunchKernelGGL(k_klt_key_amax, dim3(static_cast<unsigned>((rows + 127) / 128), hkv), dim3(256), 0, stream,
                     k_win, rows, hkv, r, smooth, basis_out, g_bits);
  hipLaunchKernelGGL(k_klt_finalize_g, dim3(1), dim3(64), 0, stream, g_out);
  return hipGetLastError();
}

}  // namespace nvkv
