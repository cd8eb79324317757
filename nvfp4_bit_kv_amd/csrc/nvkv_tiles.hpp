// Cache tiles of the attention kernels (gfx950): buffer descriptors and loads of 32-token
// iterations of the packed paged cache, and the exact dequantisation into MFMA operands.
// Shared by the split-K decode kernel and the causal prefill-attention kernel.
//
// Layout read here (one layer, per (page, KV head) block of page_size tokens):
//   K codes  [page][Hkv][page_size][64 B]   (BF16 keys: [page][Hkv][page_size][256 B])
//   K scales [page][Hkv][page_size/4][8 blocks][4 tokens]
//   V codes  [page][Hkv][page_size/4][16 words][4 tokens][4 B]   (quad-interleaved)
//   V scales as K scales.
// The argument structs of the kernels provide k_codes, k_scales, v_codes, v_scales,
// num_pages, hkv, page_size and page_shift.
#pragma once

#include "../../include/nvfp4kv.h"
#include "nvkv_device.hpp"

namespace nvkv {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kIterTok = 32;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazyMax = 8.0f;

__device__ __forceinline__ float dpp_xor1(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float dpp_xor2(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));
}
// rotate right within a row of 16 lanes by 4 / 8 (with xor 1, 2 first: max over the row)
__device__ __forceinline__ float dpp_row_ror4(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x124, 0xF, 0xF, true));
}
__device__ __forceinline__ float dpp_row_ror8(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, true));
}

// Max over the four 16-lane rows (lanes l, l^16, l^32, l^48) with the gfx950 row-swap
// permutes: pure VALU, so it never waits on outstanding scalar loads.
__device__ __forceinline__ float rows_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
}

__device__ __forceinline__ half2v as_half2(uint32_t u) { return __builtin_bit_cast(half2v, u); }
__device__ __forceinline__ uint32_t as_u32(half2v h) { return __builtin_bit_cast(uint32_t, h); }

// 8 key elements of one code dword (dims 8u..8u+7 relative) times the block scale pair.
// The gfx950 scaled FP4 convert applies only the exponent of its f32 scale, so it is asked
// for value * 2^8 (exact) and one packed f16 multiply by sigma * 2^-8 gives code * sigma.
// Byte k (constant) of a code dword -> two fp16 values * 2^8.
template <int K>
__device__ __forceinline__ half2v fp4_pair_x256(uint32_t d) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 256.0f, K);
}

__device__ __forceinline__ half8 dequant_dword(uint32_t d, half2v sig2) {
  const half2v v0 = fp4_pair_x256<0>(d) * sig2, v1 = fp4_pair_x256<1>(d) * sig2;
  const half2v v2 = fp4_pair_x256<2>(d) * sig2, v3 = fp4_pair_x256<3>(d) * sig2;
  return half8{v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
}

// E4M3 scale byte (masked to 7 bits) -> fp16 bits of sigma * 2^-8, duplicated in both halves.
__device__ __forceinline__ half2v scale_pair_same(uint32_t s) { return as_half2((s & 0x7Fu) * 0x00800080u); }

// Per-lane constants: lane (c, g) = (lane & 15, lane >> 4).  All cache loads of an iteration
// are a wave-uniform base (scalar registers, from the page table) plus one of these
// loop-invariant 32-bit lane offsets.
struct Lane {
  int c, g;
  uint32_t k_off;       // K codes: token c, dims 32g..32g+31 (16 B); BF16 keys: 64 B
  uint32_t ks_off;      // K scales: the quad of token c, blocks 2g and 2g+1 (8 B)
  uint32_t ks_shift;    // bit position of token c's byte in those scale dwords
  uint32_t v_off;       // V codes: words c (dims 8c..8c+7) of tokens 4g..4g+3 of the half (16 B)
  uint32_t vs_off;      // V scales: quad g of the half, block c >> 1 (4 B)
};

// Registers of one 32-token iteration, filled by issue_loads() well before they are used.
template <bool KBF16> struct KLoads;
template <> struct KLoads<false> {
  u32x4 kc[2];          // codes of dims 32g..32g+31 of token c of half eta
  u32x2 ks[2];          // scale dwords of blocks 2g, 2g+1 (4 tokens each) of half eta
};
template <> struct KLoads<true> {
  u32x4 kr[2][4];       // bf16 dims 32g..32g+31 of token c of half eta
};
template <bool KBF16> struct IterLoads {
  KLoads<KBF16> k;
  uint32_t vd[8];       // V code dword (dims 8c..8c+7) of token 4g+j of half eta, at [2j + eta]
  uint32_t vs[2];       // V scale dword of half eta (tokens 4g..4g+3, block c >> 1)
};

// Wave-uniform buffer descriptors of the two 16-token halves of an iteration: base = the
// half's first token in each cache array, so every load is descriptor + 32-bit lane offset
// + instruction offset.
struct HalfBase {
  __amdgpu_buffer_rsrc_t kc, ks, vc, vs;
  bool ok;              // page index in range (otherwise page 0 is read and the tokens masked)
};

// Raw-buffer descriptor word 3 for gfx9-family parts (32-bit data format, no swizzle); the
// record count is left unbounded because every offset is derived from checked indices.
constexpr int kRsrcWord3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const uint8_t* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, -1, kRsrcWord3);
}
constexpr int kNonTemporal = 2;   // cache-policy bit of the buffer-load intrinsics: nt

// Page-table entries of the two 16-token halves of an iteration (scalar loads, issued one
// iteration before the cache loads that need them).  Tokens at or beyond t_hi are mapped
// into [0, t_hi) so every access stays inside the sequence's pages.
struct IterPages {
  int32_t pg[2];
  int off16[2];
};

// The page table is read-only for the whole kernel: reading it through the constant address
// space lets the compiler use scalar loads for these wave-uniform entries.
typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;

template <class Args>
__device__ __forceinline__ IterPages load_pages(const Args& a, const_i32_ptr ptab, int t, int t_hi) {
  IterPages r;
  int tb[2], idx[2];
#pragma unroll
  for (int eta = 0; eta < 2; ++eta) {
    tb[eta] = t + 16 * eta;
    if (tb[eta] >= t_hi) tb[eta] = (t_hi - 1) & ~15;
    if (tb[eta] < 0) tb[eta] = 0;
  }
  // one branch for both halves
  if (a.page_shift >= 0) {
#pragma unroll
    for (int eta = 0; eta < 2; ++eta) {
      idx[eta] = tb[eta] >> a.page_shift;
      r.off16[eta] = tb[eta] & (a.page_size - 1);
    }
  } else {
#pragma unroll
    for (int eta = 0; eta < 2; ++eta) {
      idx[eta] = tb[eta] / a.page_size;
      r.off16[eta] = tb[eta] % a.page_size;
    }
  }
  r.pg[0] = ptab[idx[0]];
  r.pg[1] = ptab[idx[1]];
  return r;
}

template <bool KBF16, class Args>
__device__ __forceinline__ void half_bases(const Args& a, const IterPages& P, int h, HalfBase (&hb)[2]) {
#pragma unroll
  for (int eta = 0; eta < 2; ++eta) {
    const int32_t pg = P.pg[eta];
    hb[eta].ok = static_cast<uint32_t>(pg) < static_cast<uint32_t>(a.num_pages);
    const int64_t ph = static_cast<int64_t>(hb[eta].ok ? pg : 0) * a.hkv + h;   // (page, head) block
    const int64_t row0 = ph * a.page_size + P.off16[eta];
    const int64_t sc0 = ph * a.page_size * 8 + (P.off16[eta] >> 2) * 32;
    hb[eta].kc = make_rsrc(a.k_codes + row0 * (KBF16 ? kHeadDim * 2 : 64));
    if constexpr (!KBF16) hb[eta].ks = make_rsrc(a.k_scales + sc0);
    hb[eta].vc = make_rsrc(a.v_codes + row0 * 64);
    hb[eta].vs = make_rsrc(a.v_scales + sc0);
  }
}

template <bool KBF16>
__device__ __forceinline__ void issue_loads(const HalfBase (&hb)[2], const Lane& ln, IterLoads<KBF16>& L) {
#pragma unroll
  for (int eta = 0; eta < 2; ++eta) {
    if constexpr (!KBF16) {
      L.k.kc[eta] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(hb[eta].kc, ln.k_off, 0, kNonTemporal));
      L.k.ks[eta] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(hb[eta].ks, ln.ks_off, 0, 0));
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        L.k.kr[eta][u] =
            __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(hb[eta].kc, ln.k_off + 16 * u, 0, kNonTemporal));
    }
    const u32x4 v4 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(hb[eta].vc, ln.v_off, 0, kNonTemporal));
#pragma unroll
    for (int j = 0; j < 4; ++j) L.vd[2 * j + eta] = v4[j];
    L.vs[eta] = __builtin_amdgcn_raw_buffer_load_b32(hb[eta].vs, ln.vs_off, 0, 0);
  }
}

// Per-block nibble interleave of the V codes of two tokens A, B (dims 8c..8c+7 each): byte k
// of ev holds dim 8c+2k of (A, B), byte k of od holds dim 8c+2k+1 of (A, B), so one FP4 pair
// convert yields a (token, token) pair of one dim -- the PV B-operand order.
__device__ __forceinline__ uint32_t nib_even(uint32_t A, uint32_t B) { return (A & 0x0F0F0F0Fu) | ((B << 4) & 0xF0F0F0F0u); }
__device__ __forceinline__ uint32_t nib_odd(uint32_t A, uint32_t B) { return ((A >> 4) & 0x0F0F0F0Fu) | (B & 0xF0F0F0F0u); }

// Sum / max over the 16 lanes of a row (DPP within the row).
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_xor1(x));
  x = fmaxf(x, dpp_xor2(x));
  x = fmaxf(x, dpp_row_ror4(x));
  return fmaxf(x, dpp_row_ror8(x));
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_xor1(x);
  x += dpp_xor2(x);
  x += dpp_row_ror4(x);
  return x + dpp_row_ror8(x);
}

__device__ __forceinline__ void valid_tokens(const HalfBase (&hb)[2], int t0, int t_end, int c, bool (&v)[2]) {
  v[0] = hb[0].ok && (t0 + c < t_end);
  v[1] = hb[1].ok && (t0 + 16 + c < t_end);
}


// Query transform of one row (lane l holds dims 2l, 2l+1 as the bf16 pair qw): q' = q * s,
// then H(q * s) / 128 when the keys are in the Hadamard basis ([QServe rec]: the smoothing
// factor is folded into the query; [cache post] Hadamard-128 rows), times sm_scale * log2(e)
// and the key tensor scale g_K.  BF16 keys take neither transform.  The row is then split
// into exact operand terms: NVFP4 keys -- a power-of-two prescale 2^p2 puts max |q'| in
// [2^13, 2^14) and two fp16 terms (hi, lo) keep ~22 bits; BF16 keys -- three bf16 terms.
// w0..w2 receive the terms of the lane's two dims (w2 = 0 for fp16); returns the descale
// 2^-p2 to apply to the scores.  With the KLT key basis ([cache post] table rows "static
// per-head KLT"), q' = B^T (q * s) with the head's basis B in LDS (basis_lds, fp32
// [128][128]); this side of the scores is not an encoding step, so it rounds in any order.
template <bool KBF16>
__device__ __forceinline__ float query_terms(uint32_t qw, float2 sv, uint32_t k_flags, float sm_scale, float gk,
                                           int lane, uint32_t& w0, uint32_t& w1, uint32_t& w2,
                                           const float* basis_lds = nullptr, float* row_lds = nullptr) {
  float x0 = bf16_to_f32(qw & 0xFFFFu), x1 = bf16_to_f32(qw >> 16);
  float scale = sm_scale * kLog2e;
  if (!KBF16) {
    x0 *= sv.x;
    x1 *= sv.y;
    if (k_flags & NVKV_K_HADAMARD) {
      const float u0 = x0 + x1, u1 = x0 - x1;
      x0 = u0;
      x1 = u1;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const float p0 = __shfl_xor(x0, d, 64), p1 = __shfl_xor(x1, d, 64);
        const bool up = (lane & d) != 0;
        x0 = up ? p0 - x0 : x0 + p0;
        x1 = up ? p1 - x1 : x1 + p1;
      }
      scale *= (1.0f / 128.0f);
    }
    if (k_flags & NVKV_K_KLT) {
      // the row through this wavefront's LDS slot (row_lds, 128 floats); lane l forms outputs
      // 2l, 2l + 1 as four interleaved partial sums each
      *reinterpret_cast<float2*>(row_lds + 2 * lane) = make_float2(x0, x1);
      float y0[4] = {0.0f, 0.0f, 0.0f, 0.0f}, y1[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      // the reads of step j4 + 1 go out before the multiply-adds of step j4
      float4 q4 = *reinterpret_cast<const float4*>(row_lds);
      float2 bj[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) bj[u] = *reinterpret_cast<const float2*>(basis_lds + u * kHeadDim + 2 * lane);
#pragma unroll
      for (int j4 = 0; j4 < kHeadDim / 4; ++j4) {
        float4 q4n = q4;
        float2 bn[4] = {bj[0], bj[1], bj[2], bj[3]};
        if (j4 + 1 < kHeadDim / 4) {
          q4n = *reinterpret_cast<const float4*>(row_lds + 4 * (j4 + 1));
#pragma unroll
          for (int u = 0; u < 4; ++u)
            bn[u] = *reinterpret_cast<const float2*>(basis_lds + (4 * (j4 + 1) + u) * kHeadDim + 2 * lane);
        }
        const float qv[4] = {q4.x, q4.y, q4.z, q4.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          y0[u] = __builtin_fmaf(bj[u].x, qv[u], y0[u]);
          y1[u] = __builtin_fmaf(bj[u].y, qv[u], y1[u]);
        }
        q4 = q4n;
#pragma unroll
        for (int u = 0; u < 4; ++u) bj[u] = bn[u];
      }
      x0 = (y0[0] + y0[1]) + (y0[2] + y0[3]);
      x1 = (y1[0] + y1[1]) + (y1[2] + y1[3]);
    }
    scale *= gk;
  }
  x0 *= scale;
  x1 *= scale;
  float m = fmaxf(fabsf(x0), fabsf(x1));
  m = fmaxf(m, dpp_xor1(m));
  m = fmaxf(m, dpp_xor2(m));
  m = fmaxf(m, dpp_row_ror4(m));
  m = fmaxf(m, dpp_row_ror8(m));
  m = rows_max(m);
  int e = 0;
  if (m > 0.0f) frexpf(m, &e);
  const int p2 = KBF16 ? 0 : 14 - e;           // max |x| * 2^p2 in [2^13, 2^14)
  x0 = ldexpf(x0, p2);
  x1 = ldexpf(x1, p2);
  if constexpr (!KBF16) {
    const _Float16 h0 = static_cast<_Float16>(x0), h1 = static_cast<_Float16>(x1);
    const _Float16 l0 = static_cast<_Float16>(x0 - static_cast<float>(h0));
    const _Float16 l1 = static_cast<_Float16>(x1 - static_cast<float>(h1));
    w0 = __builtin_bit_cast(uint16_t, h0) | (uint32_t(__builtin_bit_cast(uint16_t, h1)) << 16);
    w1 = __builtin_bit_cast(uint16_t, l0) | (uint32_t(__builtin_bit_cast(uint16_t, l1)) << 16);
    w2 = 0u;
  } else {
    const uint32_t a0 = f32_to_bf16_rne(x0), a1 = f32_to_bf16_rne(x1);
    const float r0 = x0 - bf16_to_f32(a0), r1 = x1 - bf16_to_f32(a1);
    const uint32_t b0 = f32_to_bf16_rne(r0), b1 = f32_to_bf16_rne(r1);
    const uint32_t c0 = f32_to_bf16_rne(r0 - bf16_to_f32(b0)), c1 = f32_to_bf16_rne(r1 - bf16_to_f32(b1));
    w0 = a0 | (a1 << 16);
    w1 = b0 | (b1 << 16);
    w2 = c0 | (c1 << 16);
  }
  return ldexpf(1.0f, -p2);
}

}  // namespace nvkv
