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
#include <algorithm>

#include "nvkv_encode.hpp"
#include "nvkv_internal.hpp"
#include "nvkv_klt.hpp"

namespace nvkv {

// Append layout: a wavefront takes 32 consecutive new tokens of one KV head; lane = 8 * block
// + quad, and the lane encodes its block of tokens 4 * quad + t, t = 0..3 (one token quad),
// in four passes.  All eight row loads of a lane are issued before the first encode.  When a
// quad's four slots are consecutive and quad-aligned (pages filled in order, as in a
// prefill), the lane writes the quad's four scale bytes as one word and, for the
// quad-interleaved value codes, its two 16-byte code runs; otherwise each token is stored on
// its own.  The smoothing factors of a lane's block are loaded once.  A workgroup is 4
// wavefronts.
constexpr int kQuad = 4;
constexpr int kAppendWaves = 4;
constexpr int kTokPerWave = 8 * kQuad;
constexpr int kTokPerWg = kTokPerWave * kAppendWaves;

struct AppendArgs {
  const uint16_t* src;        // bf16 [N][Hkv][128]
  uint8_t* codes;             // NVFP4 codes or BF16 rows
  uint8_t* scales;            // NVFP4 scales (unused for BF16)
  const float* inv_smooth;    // r [Hkv][128]
  const float* gscale;        // &g_K or &g_V
  uint32_t flags;             // key transform flags (0 for V)
  int32_t fmt;                // NVKV_FMT_*
  int32_t quad_words;         // 1: codes in the quad-interleaved word layout (NVFP4 values)
  int32_t wide_stores;        // 1: scales 4-byte and codes 16-byte aligned (quad stores allowed)
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

// One wavefront's share of a (K or V, head) pair of rows in the plain layout: tokens
// n_first .. n_first + 31, lane = 8 * block + quad.  Tokens past the end compute on a clamped
// copy (every lane takes part in the cross-lane steps) and store nothing.
struct QuadLoads {
  uint4 raw[kQuad][2];        // the lane's block of the quad's four rows (bf16)
  int32_t slot[kQuad];        // their cache slots (-1: past the end)
};

// The independent loads of append_quads: the quad's rows and slots.
__device__ __forceinline__ void quads_load(const AppendPair& p, const AppendArgs& a, int h, int n_first, int lane,
                                           QuadLoads& L) {
  const int blk = lane >> 3, qd = lane & 7;
  const int nq = n_first + kQuad * qd;                  // this lane's token quad
#pragma unroll
  for (int t = 0; t < kQuad; ++t) {
    const int n = nq + t < p.n_tokens ? nq + t : p.n_tokens - 1;
    const uint4* src = reinterpret_cast<const uint4*>(a.src + (static_cast<int64_t>(n) * p.hkv + h) * kHeadDim +
                                                      blk * kBlock);
    L.raw[t][0] = src[0];
    L.raw[t][1] = src[1];
    L.slot[t] = nq + t < p.n_tokens ? append_slot(p, n) : -1;
  }
}

// The encode and stores of append_quads, from its loads.
// TAB: block-scale decisions from the E4M3 tables in LDS (tval, tt6), else computed in registers.
template <bool MSE, bool TAB>
__device__ __forceinline__ void quads_finish(const AppendPair& p, const AppendArgs& a, int h, int lane,
                                             const QuadLoads& L, const float* tval, const float* tt6) {
  const int blk = lane >> 3;
  const auto& raw = L.raw;
  const auto& slot = L.slot;
  bool ok[kQuad];
#pragma unroll
  for (int t = 0; t < kQuad; ++t) ok[t] = slot[t] >= 0 && static_cast<int64_t>(slot[t]) < p.max_slot;
  if (a.fmt == NVKV_FMT_BF16) {  // BF16 keys: plain copy of the rows
#pragma unroll
    for (int t = 0; t < kQuad; ++t) {
      if (!ok[t]) continue;
      const int32_t page = slot[t] / p.page_size, off = slot[t] - page * p.page_size;
      const int64_t ri = (static_cast<int64_t>(page) * p.hkv + h) * p.page_size + off;
      uint4* dst = reinterpret_cast<uint4*>(a.codes + ri * (kHeadDim * 2) + blk * 32);
      dst[0] = raw[t][0];
      dst[1] = raw[t][1];
    }
    return;
  }
  float r[kBlock];
  const bool smooth = (a.flags & 1u) != 0;
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
  const float gsc = *a.gscale;
  const float r6g = __builtin_amdgcn_rcpf(6.0f * gsc);
  uint32_t lo[kQuad], hi[kQuad], S[kQuad];
#pragma unroll
  for (int t = 0; t < kQuad; ++t) {
    float y[kBlock];
    unpack_bf16_block(raw[t][0], raw[t][1], y);
    if (smooth) {
#pragma unroll
      for (int i = 0; i < kBlock; ++i) y[i] = y[i] * r[i];
    }
    if (a.flags & 2u) hadamard_row<8>(y, blk);
    if (MSE && (a.flags & NVKV_K_MSE_SCALE))
      S[t] = encode_block_mse(y, gsc, lo[t], hi[t]);
    else if (TAB)
      S[t] = encode_block_t(y, gsc, r6g, tt6, lo[t], hi[t]);
    else
      S[t] = encode_block(y, gsc, lo[t], hi[t]);
  }
  const bool quad = a.wide_stores && ok[0] && ok[1] && ok[2] && ok[3] && (slot[0] & 3) == 0 &&
                    slot[1] == slot[0] + 1 && slot[2] == slot[0] + 2 && slot[3] == slot[0] + 3;
  if (quad) {   // page_size is a multiple of 16, so an aligned quad lies in one page
    const int32_t page = slot[0] / p.page_size, off = slot[0] - page * p.page_size;
    const int64_t ri = (static_cast<int64_t>(page) * p.hkv + h) * p.page_size + off;
    if (!a.quad_words) {
#pragma unroll
      for (int t = 0; t < kQuad; ++t)
        *reinterpret_cast<uint2*>(a.codes + (ri + t) * 64 + blk * 8) = make_uint2(lo[t], hi[t]);
    } else {
      // word 2blk of the quad's tokens: 16 bytes at 32 blk of the quad's 256-byte group,
      // word 2blk+1 the next 16
      uint4* wq = reinterpret_cast<uint4*>(a.codes + ri * 64 + 32 * blk);
      wq[0] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
      wq[1] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    }
    const int64_t sbase = (static_cast<int64_t>(page) * p.hkv + h) * p.page_size * 8;
    *reinterpret_cast<uint32_t*>(a.scales + sbase + ((off >> 2) * 8 + blk) * 4) =
        S[0] | (S[1] << 8) | (S[2] << 16) | (S[3] << 24);
    return;
  }
#pragma unroll
  for (int t = 0; t < kQuad; ++t) {
    if (!ok[t]) continue;
    const int32_t page = slot[t] / p.page_size, off = slot[t] - page * p.page_size;
    const int64_t ri = (static_cast<int64_t>(page) * p.hkv + h) * p.page_size + off;
    if (!a.quad_words) {
      *reinterpret_cast<uint2*>(a.codes + ri * 64 + blk * 8) = make_uint2(lo[t], hi[t]);
    } else {
      // words 2blk, 2blk+1 of token `off`: byte ((off/4)*16 + w)*16 + (off%4)*4 of the
      // (page, head) block, which starts at the same place as in the row-major layout
      uint8_t* wq = a.codes + (ri - (off & 3)) * 64 + 32 * blk + 4 * (off & 3);
      *reinterpret_cast<uint32_t*>(wq) = lo[t];
      *reinterpret_cast<uint32_t*>(wq + 16) = hi[t];
    }
    const int64_t sbase = (static_cast<int64_t>(page) * p.hkv + h) * p.page_size * 8;
    a.scales[sbase + ((off >> 2) * 8 + blk) * 4 + (off & 3)] = static_cast<uint8_t>(S[t]);
  }
}

template <bool MSE>
__device__ __forceinline__ void append_quads(const AppendPair& p, const AppendArgs& a, int h, int n_first,
                                             int lane, const float* tval, const float* tt6) {
  QuadLoads L;
  quads_load(p, a, h, n_first, lane, L);
  quads_finish<MSE, true>(p, a, h, lane, L, tval, tt6);
}

// grid: x = token chunks of kTokPerWg, y = KV head row (< Hkv: keys, else values).  MSE:
// compiled with the key block-scale search (which needs more registers than the plain
// encoder, so the plain launch does not carry it).  Four workgroups per CU: the search
// instance fits 128 registers without spills, four wavefronts per SIMD instead of three.
template <bool MSE>
__global__ void __launch_bounds__(256, 4) k_quantize_append(AppendPair p) {
  const int row = static_cast<int>(blockIdx.y);
  const int which = row >= p.hkv ? 1 : 0;
  // the selected half of the arguments, read from the kernel-argument segment (p, the only
  // argument, is at its start) at a uniform offset: a select between the two copies in
  // registers keeps both alive up to the stores, and their scalar registers spill
  const AppendArgs a = ((const AppendPair*)__builtin_amdgcn_kernarg_segment_ptr())->a[which];
  const int h = row - (which ? p.hkv : 0);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // E4M3 values and 6x midpoints for the block-scale decisions
  __shared__ float tval[128], tt6[128];
  fill_e4m3_tables(tval, tt6, threadIdx.x, 64 * kAppendWaves);
  __syncthreads();
  const int n_first = static_cast<int>(blockIdx.x) * kTokPerWg + wave * kTokPerWave;
  if (n_first >= p.n_tokens) return;                   // uniform per wavefront
  append_quads<MSE>(p, a, h, n_first, lane, tval, tt6);
}

// KLT keys ([cache post] cache-config table, KLT rows).  A workgroup of 8 wavefronts owns
// one head and walks its 128-token chunks with the head's basis resident in LDS (64 KB), so
// the basis is read from memory once per workgroup.  Per chunk:
//   staging: wavefront w converts tokens 64 (w & 1) .. + 63, dims 32 (w >> 1) .. + 31 to
//     y = fl32(x r) and writes them element-major, ybuf[j][token] (64 KB);
//   rotation: lane (column group cb, token quad tq) forms z for 8 columns 8 cb .. 8 cb + 7 and
//     the quad's 4 tokens as rotate_cols does, z <- fl32(B[j][col] y_j + z) over j = 0..127,
//     from one 16-byte read of y and two of B per j: 32 multiply-adds per 48 bytes read;
//   encode: the two lanes of a block (cb = 2b, 2b + 1, adjacent lanes) swap halves so that
//     each holds the block's 16 columns for two of the quad's tokens, then encode and store.
// The next chunk's key rows are loaded during the rotation, and wavefronts 0..3 load the
// chunk's value rows before it and encode them after it (the plain quad path), so the
// memory traffic overlaps the multiply-adds.
constexpr int kKltWaves = 8;
constexpr int kKltTok = 128;
constexpr int kKltResidentWgs = 256;      // one per CU

__device__ __forceinline__ float swap_adjacent_lanes(float v) {   // lane l <-> lane l ^ 1
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}

template <bool MSE>
__global__ void __launch_bounds__(64 * kKltWaves) k_quantize_append_klt(AppendPair p) {
  const int h = static_cast<int>(blockIdx.y);
  const AppendArgs& ka = p.a[0];
  const AppendArgs& va = p.a[1];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // one LDS object, the basis first: every rotation read is then a base register plus a
  // constant offset below 64 KiB
  __shared__ __attribute__((aligned(16))) float lds[kBasisFloats + kHeadDim * kKltTok];
  float* const basis_lds = lds;
  float (*const ybuf)[kKltTok] = reinterpret_cast<float (*)[kKltTok]>(lds + kBasisFloats);
  load_basis_lds(ka.basis + static_cast<int64_t>(h) * kBasisFloats, basis_lds, tid, 64 * kKltWaves);
  const int st_tok = 64 * (wave & 1) + lane, st_d0 = 32 * (wave >> 1);     // staging role
  const int cb = 8 * (wave & 1) + (lane & 7), tq = 8 * (wave >> 1) + (lane >> 3);   // rotation role
  const bool odd = (cb & 1) != 0;
  // the smoothing factors of the wavefront's 32 staging dims (1 without smoothing: x * 1 = x)
  float rs[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) rs[i] = (ka.flags & 1u) ? ka.inv_smooth[h * kHeadDim + st_d0 + i] : 1.0f;
  const float gk = *ka.gscale;
  const int n_chunks = (p.n_tokens + kKltTok - 1) / kKltTok;
  uint4 kraw[4];
  auto load_keys = [&](int chunk) {
    const int n0 = chunk * kKltTok + st_tok;
    const int n = n0 < p.n_tokens ? n0 : p.n_tokens - 1;
    const uint4* src = reinterpret_cast<const uint4*>(ka.src + (static_cast<int64_t>(n) * p.hkv + h) * kHeadDim + st_d0);
#pragma unroll
    for (int i = 0; i < 4; ++i) kraw[i] = src[i];
  };
  int chunk = static_cast<int>(blockIdx.x);
  if (chunk < n_chunks) load_keys(chunk);
  for (; chunk < n_chunks; chunk += static_cast<int>(gridDim.x)) {
    const int base = chunk * kKltTok;
    QuadLoads vl;
    if (wave < 4) quads_load(p, va, h, base + kTokPerWave * wave, lane, vl);
    // staging (the first chunk's barrier also publishes the basis)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w[4] = {kraw[i].x, kraw[i].y, kraw[i].z, kraw[i].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = bf16_to_f32(e & 1 ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xFFFFu));
        ybuf[st_d0 + 8 * i + e][st_tok] = x * rs[8 * i + e];
      }
    }
    __syncthreads();
    if (chunk + static_cast<int>(gridDim.x) < n_chunks) load_keys(chunk + static_cast<int>(gridDim.x));
    float z[kQuad][8];
#pragma unroll
    for (int t = 0; t < kQuad; ++t)
#pragma unroll
      for (int k = 0; k < 8; ++k) z[t][k] = 0.0f;
    // software pipelined: the reads of step j + 2 are issued before the multiply-adds of step j
    float4 yq[3], b0[3], b1[3];
    auto read_step = [&](int j, int slot) {
      yq[slot] = *reinterpret_cast<const float4*>(&ybuf[j][kQuad * tq]);
      b0[slot] = *reinterpret_cast<const float4*>(&basis_lds[j * kHeadDim + 8 * cb]);
      b1[slot] = *reinterpret_cast<const float4*>(&basis_lds[j * kHeadDim + 8 * cb + 4]);
    };
    read_step(0, 0);
    read_step(1, 1);
#pragma unroll
    for (int j = 0; j < kHeadDim; ++j) {
      if (j + 2 < kHeadDim) read_step(j + 2, (j + 2) % 3);
      const int c = j % 3;
      const float bv[8] = {b0[c].x, b0[c].y, b0[c].z, b0[c].w, b1[c].x, b1[c].y, b1[c].z, b1[c].w};
      const float yv[4] = {yq[c].x, yq[c].y, yq[c].z, yq[c].w};
#pragma unroll
      for (int t = 0; t < kQuad; ++t)
#pragma unroll
        for (int k = 0; k < 8; ++k) z[t][k] = __builtin_fmaf(bv[k], yv[t], z[t][k]);
    }
    __syncthreads();                      // ybuf is free for the next chunk
    // halves: the even lane keeps tokens 0, 1 of the quad, the odd lane tokens 2, 3
    float blkz[2][kBlock];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float keep = odd ? z[2 + u][k] : z[u][k];
        const float recv = swap_adjacent_lanes(odd ? z[u][k] : z[2 + u][k]);
        blkz[u][k] = odd ? recv : keep;           // columns 16b .. 16b + 7
        blkz[u][k + 8] = odd ? keep : recv;       // columns 16b + 8 .. 16b + 15
      }
    const int b = cb >> 1;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int n = base + kQuad * tq + (odd ? 2 : 0) + u;
      uint32_t lo, hi;
      const uint32_t S = (MSE && (ka.flags & NVKV_K_MSE_SCALE)) ? encode_block_mse(blkz[u], gk, lo, hi)
                                                                : encode_block(blkz[u], gk, lo, hi);
      const int32_t slot = n < p.n_tokens ? append_slot(p, n) : -1;
      if (slot >= 0 && static_cast<int64_t>(slot) < p.max_slot) {
        const int32_t page = slot / p.page_size, off = slot - page * p.page_size;
        const int64_t ri = (static_cast<int64_t>(page) * p.hkv + h) * p.page_size + off;
        *reinterpret_cast<uint2*>(ka.codes + ri * 64 + b * 8) = make_uint2(lo, hi);
        const int64_t sbase = (static_cast<int64_t>(page) * p.hkv + h) * p.page_size * 8;
        ka.scales[sbase + ((off >> 2) * 8 + b) * 4 + (off & 3)] = static_cast<uint8_t>(S);
      }
    }
    if (wave < 4 && base + kTokPerWave * wave < p.n_tokens)
      quads_finish<false, false>(p, va, h, lane, vl, nullptr, nullptr);
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
  auto wide = [](const void* codes, const void* scales) {
    return static_cast<int32_t>((reinterpret_cast<uintptr_t>(codes) & 15u) == 0 &&
                                (reinterpret_cast<uintptr_t>(scales) & 3u) == 0);
  };
  AppendPair p{};
  p.a[0] = AppendArgs{k_new, static_cast<uint8_t*>(L.k_data), L.k_scales, L.k_inv_smooth, L.global_scale + 0,
                      L.k_fmt == NVKV_FMT_NVFP4 ? L.k_flags : 0u, L.k_fmt, 0, wide(L.k_data, L.k_scales), L.k_basis};
  p.a[1] = AppendArgs{v_new, static_cast<uint8_t*>(L.v_data), L.v_scales, nullptr, L.global_scale + 1, 0u,
                      L.v_fmt, 1, wide(L.v_data, L.v_scales), nullptr};
  p.slots = slots;
  p.page_table = page_table;
  p.seq_lens = seq_lens;
  p.max_pages_per_seq = max_pages_per_seq;
  p.seq_cap = seq_cap;
  p.n_tokens = N;
  p.hkv = L.num_kv_heads;
  p.page_size = L.page_size;
  p.max_slot = static_cast<int64_t>(L.num_pages) * L.page_size;
  const unsigned chunks = static_cast<unsigned>((N + kTokPerWg - 1) / kTokPerWg);
  const bool mse = p.a[0].flags & NVKV_K_MSE_SCALE, klt = p.a[0].flags & NVKV_K_KLT;
  using Kernel = void (*)(AppendPair);
  if (klt) {
    // one resident workgroup per CU (the basis and the staged rows fill its LDS), each
    // walking the chunks of one head
    const int kchunks = (N + kKltTok - 1) / kKltTok;
    const int per_head = std::max(1, std::min(kchunks, kKltResidentWgs / L.num_kv_heads));
    const Kernel kk = mse ? k_quantize_append_klt<true> : k_quantize_append_klt<false>;
    hipLaunchKernelGGL(kk, dim3(per_head, L.num_kv_heads), dim3(64 * kKltWaves), 0, stream, p);
  } else {
    const Kernel kk = mse ? k_quantize_append<true> : k_quantize_append<false>;
    hipLaunchKernelGGL(kk, dim3(chunks, 2 * L.num_kv_heads), dim3(64 * kAppendWaves), 0, stream, p);
  }
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
