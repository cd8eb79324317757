// Quantise/append and calibration kernels (gfx950).  Compiled with -ffp-contract=off.
//
// [cache post] = rstation.ai post "NVFP4 attention cache on W4A4 Qwen3-8B: static key
// smoothing is near-lossless, key rotations hurt": post-RoPE keys/values are quantised to
// NVFP4 in 16-blocks along head_dim (opening paragraph); keys are smoothed per channel by
// sqrt(absmax) calibrated on 4 windows without position 0, optionally in a Hadamard-128 basis
// (cache-config table).  [OSFP4] = paperlayer.ai summary of arXiv 2610.08231v1: the global
// scale is static and calibration-based so blocks can be quantised as they arrive (section 3).
//
// Every lane handles one 16-element block of a 128-element row.  The append kernel puts the
// 8 blocks of a row 8 lanes apart (lane = 8 * block + token); the calibration kernels put
// them in 8 consecutive lanes (8 rows per wavefront, 32 per workgroup).  The only cross-lane
// traffic is the Hadamard butterfly's three block-pair stages.
#include "nvkv_encode.hpp"
#include "nvkv_internal.hpp"
#include "nvkv_klt.hpp"

namespace nvkv {

// Append layout: a wavefront takes 8 consecutive new tokens of one KV head per pass, lane
// = 8 * block + token, and makes kPasses passes; a workgroup is 4 wavefronts.  The
// smoothing factors of a lane's block are loaded once and serve every pass.  Adjacent lanes
// hold adjacent tokens, so the scale bytes and value words of a token quad are written by
// adjacent lanes to adjacent bytes.
constexpr int kTokPerPass = 8;
constexpr int kPasses = 4;
constexpr int kAppendWaves = 4;
constexpr int kTokPerWg = kTokPerPass * kPasses * kAppendWaves;

struct AppendArgs {
  const uint16_t* src;        // bf16 [N][Hkv][128]
  uint8_t* codes;             // NVFP4 codes or BF16 rows
  uint8_t* scales;            // NVFP4 scales (unused for BF16)
  const float* inv_smooth;    // r [Hkv][128]
  const float* gscale;        // &g_K or &g_V
  uint32_t flags;             // key transform flags (0 for V)
  int32_t fmt;                // NVKV_FMT_*
  int32_t quad_words;         // 1: codes in the quad-interleaved word layout (NVFP4 values)
  const float* basis;         // KLT basis [Hkv][128][128] (keys with NVKV_K_KLT), else unused
};

struct AppendPair {
  AppendArgs a[2];            // [0] = keys, [1] = values
  const int32_t* slots;       // [N]; nullptr: see below
  // slots == nullptr: token n is the new token of sequence n, at position min(seq_lens[n],
  // seq_cap) - 1 of the paged sequence (nothing is written when that length is 0)
  const int32_t* page_table;  // [B][max_pages_per_seq]
  const int32_t* seq_lens;    // [B]
  int32_t max_pages_per_seq;
  int32_t seq_cap;
  int32_t n_tokens;           // N
  int32_t hkv;
  int32_t page_size;
  int64_t max_slot;           // num_pages * page_size
};

__device__ __forceinline__ int32_t append_slot(const AppendPair& p, int n) {
  if (p.slots) return p.slots[n];
  int32_t len = p.seq_lens[n];
  len = len > p.seq_cap ? p.seq_cap : len;
  if (len <= 0) return -1;
  const int32_t pos = len - 1;
  const int64_t pg = p.page_table[static_cast<int64_t>(n) * p.max_pages_per_seq + pos / p.page_size];
  const int64_t s64 = pg * p.page_size + pos % p.page_size;
  return (pg < 0 || s64 >= p.max_slot) ? -1 : static_cast<int32_t>(s64);
}

// grid: x = token chunks of kTokPerWg, y = KV head (y < Hkv: keys, else values).  MSE:
// compiled with the key block-scale search (which needs more registers than the plain
// encoder, so the plain launch does not carry it).  KLT: compiled with the key basis
// rotation (the head's basis in LDS, each wavefront's 8 rows staged in LDS).
template <bool MSE, bool KLT>
__global__ void __launch_bounds__(256) k_quantize_append(AppendPair p) {
  const int which = static_cast<int>(blockIdx.y) >= p.hkv ? 1 : 0;
  const AppendArgs a = which ? p.a[1] : p.a[0];   // uniform select, no dynamic indexing
  const int h = static_cast<int>(blockIdx.y) - (which ? p.hkv : 0);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int blk = lane >> 3, tok = lane & 7;
  __shared__ __attribute__((aligned(16))) float basis_lds[KLT ? kBasisFloats : 4];
  __shared__ __attribute__((aligned(16))) float row_lds[KLT ? kAppendWaves : 1][KLT ? kTokPerPass : 1][kHeadDim];
  const bool klt = KLT && a.fmt != NVKV_FMT_BF16 && (a.flags & NVKV_K_KLT);   // uniform per workgroup
  if constexpr (KLT) {
    if (klt) load_basis_lds(a.basis + static_cast<int64_t>(h) * kBasisFloats, basis_lds, threadIdx.x, 256);
    __syncthreads();
  }
  const bool smooth = a.fmt != NVKV_FMT_BF16 && (a.flags & 1u);
  float r[kBlock];
  if (smooth) {
    const float4* rp = reinterpret_cast<const float4*>(a.inv_smooth + h * kHeadDim + blk * kBlock);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 v = rp[q];
      r[4 * q] = v.x;
      r[4 * q + 1] = v.y;
      r[4 * q + 2] = v.z;
      r[4 * q + 3] = v.w;
    }
  }
  const float gsc = a.fmt == NVKV_FMT_BF16 ? 1.0f : *a.gscale;
  const int n_wave = static_cast<int>(blockIdx.x) * kTokPerWg + wave * (kTokPerPass * kPasses);
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {   // unrolled: a pass's loads overlap the previous encode
    const int n0 = n_wave + pass * kTokPerPass;
    if (n0 >= p.n_tokens) break;                        // uniform
    // tokens past the end compute on a clamped copy (every lane takes part in the
    // cross-lane steps) and store nothing
    const int n = n0 + tok < p.n_tokens ? n0 + tok : p.n_tokens - 1;
    const bool live = n0 + tok < p.n_tokens;
    // independent loads first (row block, slot); the slot check comes after
    float y[kBlock];
    uint4 raw0, raw1;
    load_block_bf16(a.src + (static_cast<int64_t>(n) * p.hkv + h) * kHeadDim + blk * kBlock, y, raw0, raw1);
    const int32_t slot = append_slot(p, n);
    const bool ok = live && slot >= 0 && static_cast<int64_t>(slot) < p.max_slot;
    const int32_t page = ok ? slot / p.page_size : 0;
    const int32_t off = ok ? slot - page * p.page_size : 0;
    const int64_t row_index = (static_cast<int64_t>(page) * p.hkv + h) * p.page_size + off;
    if (a.fmt == NVKV_FMT_BF16) {  // BF16 keys: plain copy of the row
      if (ok) {
        uint4* dst = reinterpret_cast<uint4*>(a.codes + row_index * (kHeadDim * 2) + blk * 32);
        dst[0] = raw0;
        dst[1] = raw1;
      }
      continue;
    }
    if (smooth) {
#pragma unroll
      for (int i = 0; i < kBlock; ++i) y[i] = y[i] * r[i];
    }
    if (a.flags & 2u) hadamard_row<8>(y, blk);
    if constexpr (KLT) {
      if (klt) {   // z = B^T y: the row through LDS, this lane's 16 outputs in the fixed order
        float4* dst = reinterpret_cast<float4*>(&row_lds[wave][tok][blk * kBlock]);
#pragma unroll
        for (int q = 0; q < 4; ++q) dst[q] = make_float4(y[4 * q], y[4 * q + 1], y[4 * q + 2], y[4 * q + 3]);
        rotate_cols<kBlock>(basis_lds, row_lds[wave][tok], blk * kBlock, y);
      }
    }
    uint32_t lo, hi;
    const uint32_t S = (MSE && (a.flags & NVKV_K_MSE_SCALE)) ? encode_block_mse(y, gsc, lo, hi)
                                                             : encode_block(y, gsc, lo, hi);
    if (!ok) continue;
    if (!a.quad_words) {
      *reinterpret_cast<uint2*>(a.codes + row_index * 64 + blk * 8) = make_uint2(lo, hi);
    } else {
      // words 2blk, 2blk+1 of token `off`: byte ((off/4)*16 + w)*16 + (off%4)*4 of the
      // (page, head) block, which starts at the same place as in the row-major layout
      uint8_t* wq = a.codes + (row_index - (off & 3)) * 64 + 32 * blk + 4 * (off & 3);
      *reinterpret_cast<uint32_t*>(wq) = lo;
      *reinterpret_cast<uint32_t*>(wq + 16) = hi;
    }
    const int64_t sbase = (static_cast<int64_t>(page) * p.hkv + h) * p.page_size * 8;
    a.scales[sbase + ((off >> 2) * 8 + blk) * 4 + (off & 3)] = static_cast<uint8_t>(S);
  }
}

constexpr int kRowsPerWg = 32;   // calibration kernels: rows per workgroup

// ---------------------------------------------------------------------------------------
// Calibration.  Max reductions over non-negative fp32 use unsigned atomicMax on the bit
// patterns (order-preserving, deterministic).  s_out and g_out serve as the reduction
// buffers and are rewritten in place by the finalise kernels.
// ---------------------------------------------------------------------------------------
__global__ void k_calib_clear(uint32_t* s_bits, int n, uint32_t* g_bits, int clear_gk, int clear_gv) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) s_bits[i] = 0u;
  if (i == 0) {
    if (clear_gk) g_bits[0] = 0u;
    if (clear_gv) g_bits[1] = 0u;
  }
}

constexpr int kCalibTokChunk = 32;

// grid: (ceil(T / 32), W); each thread owns channel pairs c2 = tid, tid+256, ...
__global__ void __launch_bounds__(256) k_calib_channel_absmax(const uint16_t* __restrict__ k_win, int T,
                                                              int hkv, int t_begin, uint32_t* s_bits) {
  const int C2 = hkv * kHeadDim / 2;
  const int w = blockIdx.y;
  const int t0 = max(static_cast<int>(blockIdx.x) * kCalibTokChunk, t_begin);
  const int t1 = min(static_cast<int>(blockIdx.x + 1) * kCalibTokChunk, T);
  const uint32_t* base = reinterpret_cast<const uint32_t*>(k_win) + static_cast<int64_t>(w) * T * C2;
  for (int c2 = threadIdx.x; c2 < C2; c2 += blockDim.x) {
    float m0 = 0.0f, m1 = 0.0f;
    for (int t = t0; t < t1; ++t) {
      const uint32_t v = base[static_cast<int64_t>(t) * C2 + c2];
      m0 = fmaxf(m0, fabsf(bf16_to_f32(v & 0xFFFFu)));
      m1 = fmaxf(m1, fabsf(bf16_to_f32(v >> 16)));
    }
    if (t0 < t1) {
      atomicMax(&s_bits[2 * c2], __float_as_uint(m0));
      atomicMax(&s_bits[2 * c2 + 1], __float_as_uint(m1));
    }
  }
}

// s = fl32(sqrt(a)) (1 where a = 0), r = fl32(1/s); both correctly rounded.
__global__ void k_calib_finalize_sr(float* s_out, float* r_out, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float a = __uint_as_float(reinterpret_cast<uint32_t*>(s_out)[i]);
  const float s = (a == 0.0f) ? 1.0f : sqrt_rn_f32(a);
  s_out[i] = s;
  r_out[i] = div_rn_f32(1.0f, s);
}

// Row absmax of the transformed keys (all positions) or the raw values; one atomic per
// 8-row group.  Rows: W*T*Hkv.
__global__ void __launch_bounds__(256) k_calib_transform_amax(const uint16_t* __restrict__ src, int64_t n_rows,
                                                              int hkv, const float* __restrict__ r,
                                                              uint32_t flags, uint32_t* g_bits) {
  const int lane = threadIdx.x & 63;
  const int blk = lane & 7;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kRowsPerWg + (threadIdx.x >> 3);
  if (row >= n_rows) return;
  const int h = static_cast<int>(row % hkv);
  float y[kBlock];
  uint4 raw0, raw1;
  load_block_bf16(src + row * kHeadDim + blk * kBlock, y, raw0, raw1);
  if (flags & 1u) smooth_block(y, r + h * kHeadDim + blk * kBlock);
  if (flags & 2u) hadamard_row(y, blk);
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < kBlock; ++i) m = fmaxf(m, fabsf(y[i]));
  m = fmaxf(m, xor_lanes(m, 1));
  m = fmaxf(m, xor_lanes(m, 2));
  m = fmaxf(m, xor_lanes(m, 4));
  if (blk == 0) atomicMax(g_bits, __float_as_uint(m));
}

// g = fl32(A / 2688) (1 where A = 0), correctly rounded.
__global__ void k_calib_finalize_g(float* g_out, int do_k, int do_v) {
  const int i = threadIdx.x;
  if (i > 1 || (i == 0 && !do_k) || (i == 1 && !do_v)) return;
  const float A = __uint_as_float(reinterpret_cast<uint32_t*>(g_out)[i]);
  g_out[i] = (A == 0.0f) ? 1.0f : div_rn_f32(A, 2688.0f);
}

// ---------------------------------------------------------------------------------------
// Host launchers (argument validation happens in the C ABI layer before these run).
// ---------------------------------------------------------------------------------------
hipError_t launch_quantize_append(const nvkv_layer& L, const uint16_t* k_new, const uint16_t* v_new,
                                  const int32_t* slots, int32_t N, hipStream_t stream) {
  return launch_quantize_append_rows(L, k_new, v_new, slots, N, nullptr, nullptr, 0, 0, stream);
}

hipError_t launch_quantize_append_rows(const nvkv_layer& L, const uint16_t* k_new, const uint16_t* v_new,
                                       const int32_t* slots, int32_t N, const int32_t* page_table,
                                       const int32_t* seq_lens, int32_t max_pages_per_seq, int32_t seq_cap,
                                       hipStream_t stream) {
  AppendPair p{};
  p.a[0] = AppendArgs{k_new, static_cast<uint8_t*>(L.k_data), L.k_scales, L.k_inv_smooth, L.global_scale + 0,
                      L.k_fmt == NVKV_FMT_NVFP4 ? L.k_flags : 0u, L.k_fmt, 0, L.k_basis};
  p.a[1] = AppendArgs{v_new, static_cast<uint8_t*>(L.v_data), L.v_scales, nullptr, L.global_scale + 1, 0u,
                      L.v_fmt, 1, nullptr};
  p.slots = slots;
  p.page_table = page_table;
  p.seq_lens = seq_lens;
  p.max_pages_per_seq = max_pages_per_seq;
  p.seq_cap = seq_cap;
  p.n_tokens = N;
  p.hkv = L.num_kv_heads;
  p.page_size = L.page_size;
  p.max_slot = static_cast<int64_t>(L.num_pages) * L.page_size;
  const dim3 grid((N + kTokPerWg - 1) / kTokPerWg, 2 * L.num_kv_heads);
  const bool mse = p.a[0].flags & NVKV_K_MSE_SCALE, klt = p.a[0].flags & NVKV_K_KLT;
  using Kernel = void (*)(AppendPair);
  const Kernel kern = klt ? (mse ? k_quantize_append<true, true> : k_quantize_append<false, true>)
                          : (mse ? k_quantize_append<true, false> : k_quantize_append<false, false>);
  hipLaunchKernelGGL(kern, grid, dim3(64 * kAppendWaves), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_calibrate(const uint16_t* k_win, const uint16_t* v_win, int32_t W, int32_t T, int32_t hkv,
                            int32_t exclude_pos0, uint32_t k_flags, float* s_out, float* r_out, float* g_out,
                            hipStream_t stream) {
  const int C = hkv * kHeadDim;
  uint32_t* s_bits = reinterpret_cast<uint32_t*>(s_out);
  uint32_t* g_bits = reinterpret_cast<uint32_t*>(g_out);
  const int do_k = k_win != nullptr, do_v = v_win != nullptr;
  const int do_gk = do_k && !(k_flags & NVKV_K_KLT);     // with the KLT basis, g_K comes after the basis
  hipLaunchKernelGGL(k_calib_clear, dim3((C + 255) / 256), dim3(256), 0, stream, s_bits, do_k ? C : 0, g_bits,
                     do_gk, do_v);
  const int64_t rows = static_cast<int64_t>(W) * T * hkv;
  const int64_t wg_rows = (rows + kRowsPerWg - 1) / kRowsPerWg;
  if (do_k) {
    const int t_begin = exclude_pos0 ? 1 : 0;
    hipLaunchKernelGGL(k_calib_channel_absmax, dim3((T + kCalibTokChunk - 1) / kCalibTokChunk, W), dim3(256), 0,
                       stream, k_win, T, hkv, t_begin, s_bits);
    hipLaunchKernelGGL(k_calib_finalize_sr, dim3((C + 255) / 256), dim3(256), 0, stream, s_out, r_out, C);
    if (do_gk)
      hipLaunchKernelGGL(k_calib_transform_amax, dim3(static_cast<unsigned>(wg_rows)), dim3(256), 0, stream, k_win,
                         rows, hkv, r_out, k_flags, g_bits + 0);
  }
  if (do_v) {
    hipLaunchKernelGGL(k_calib_transform_amax, dim3(static_cast<unsigned>(wg_rows)), dim3(256), 0, stream, v_win,
                       rows, hkv, nullptr, 0u, g_bits + 1);
  }
  hipLaunchKernelGGL(k_calib_finalize_g, dim3(1), dim3(64), 0, stream, g_out, do_gk, do_v);
  return hipGetLastError();
}

}  // namespace nvkv
