// Split-K GQA decode attention over the packed NVFP4 cache (gfx950, MFMA).
//
// [cache post] = rstation.ai post "NVFP4 attention cache on W4A4 Qwen3-8B: static key
// smoothing is near-lossless, key rotations hurt": attention over the NVFP4 post-RoPE cache,
// keys smoothed per channel (queries carry the factor) and optionally in a Hadamard-128 basis.
// [QServe rec] = inference-research record "QServe SmoothAttention (4-bit KV cache ...)":
// the smoothing factor is folded into the query; attention is kept memory-bound so the 4-bit
// cache pays off.
//
// Work decomposition: one workgroup (4 wavefronts) per (split, KV head, sequence); the split's
// tokens are cut into 32-token iterations dealt round-robin to the 4 wavefronts.  Per
// iteration a wavefront does:
//   QK  S^T[32 tok x 16 col] = Khat[32 x 128] Q'^T: 2 x 4 MFMA 16x16x32 f16.  Khat = code *
//       sigma (exact in fp16); the 16 columns are (query head i, term t): the query is split
//       into hi + lo fp16 terms (t = 0, 1; columns t = 2, 3 are zero) so the product keeps
//       ~22 bits.  BF16 keys use the bf16 MFMA with a 3-term bf16 split instead.
//   online softmax in the base-2 domain with a lazily updated running max (the reference
//       max moves only when a block max exceeds it by more than 8, so p <= 256).
//   PV  O[16 row x 128] += P[16 x 32 tok] Vhat[32 tok x 128]: 8 MFMA 16x16x32 f16; rows are
//       (query head i, term t) with p split into hi + lo fp16 terms.
// The score layout produced by QK (lane (c, g) holds tokens 4g..4g+3 of each 16-token half
// for column c) is exactly the A-operand layout PV needs, so no transpose is required.
// V codes are read token-major: lane (c, g) fetches the dword of dims 8c..8c+7 of its 8
// tokens and serves column c of PV instruction v as dim 8c + v.
// Dequantisation: nibble -> fp16 (value * 2^8) through a v_perm byte table, E4M3 scale ->
// fp16 (sigma * 2^-8) by a bit shift, one v_pk_mul_f16 per element pair; the product is the
// exact code * sigma.
// Partials (unnormalised O, running max m, sum l) are merged across wavefronts in LDS and,
// when a sequence has several splits, across workgroups by k_decode_merge.
#include "nvkv_device.hpp"
#include "nvkv_internal.hpp"

namespace nvkv {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kIterTok = 32;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazyMax = 8.0f;

struct DecodeArgs {
  const uint8_t* k_codes;     // NVFP4 key codes, or BF16 key rows
  const uint8_t* k_scales;
  const uint8_t* v_codes;
  const uint8_t* v_scales;
  const float* smooth;        // s [Hkv][128]
  const float* gscale;        // {g_K, g_V}
  const uint16_t* q;          // bf16 [B][Hq][128]
  const int32_t* page_table;  // [B][max_pages_per_seq]
  const int32_t* seq_lens;    // [B]
  float* out;                 // fp32 [B][Hq][128]
  float* ws_o;                // [B][Hkv][n_splits][4][128]
  float* ws_ml;               // [B][Hkv][n_splits][4][2]
  int32_t hkv, hq, page_size, num_pages, max_pages_per_seq, seq_cap;
  int32_t split_tokens, n_splits;
  uint32_t k_flags;
  float sm_scale;
};

__device__ __forceinline__ float dpp_xor1(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float dpp_xor2(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));
}

// fp16 high bytes of e2m1 magnitude * 256 for magnitude codes 0..7:
// {0, 128, 256, 384, 512, 768, 1024, 1536} -> 0x00 0x58 0x5C 0x5E | 0x60 0x62 0x64 0x66.
constexpr uint32_t kLutLo = 0x5E5C5800u;
constexpr uint32_t kLutHi = 0x66646260u;

// High bytes (sign included) of the fp16 images of the even / odd nibbles of a code dword.
__device__ __forceinline__ void nibble_high_bytes(uint32_t d, uint32_t& even, uint32_t& odd) {
  even = __builtin_amdgcn_perm(kLutHi, kLutLo, d & 0x07070707u) | ((d << 4) & 0x80808080u);
  odd = __builtin_amdgcn_perm(kLutHi, kLutLo, (d >> 4) & 0x07070707u) | (d & 0x80808080u);
}

// [0x00, lo.byte k, 0x00, hi.byte k]: two fp16 values with zero low bytes.
__device__ __forceinline__ uint32_t pair_bytes(uint32_t hi_src, uint32_t lo_src, int k) {
  const uint32_t sel = 0x0Cu | (uint32_t(k) << 8) | (0x0Cu << 16) | (uint32_t(4 + k) << 24);
  return __builtin_amdgcn_perm(hi_src, lo_src, sel);
}

__device__ __forceinline__ half2v as_half2(uint32_t u) { return __builtin_bit_cast(half2v, u); }
__device__ __forceinline__ uint32_t as_u32(half2v h) { return __builtin_bit_cast(uint32_t, h); }

// 8 key elements of one code dword (dims 8u..8u+7 relative) times the block scale pair.
__device__ __forceinline__ half8 dequant_dword(uint32_t d, half2v sig2) {
  uint32_t ev, od;
  nibble_high_bytes(d, ev, od);
  half8 r;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const half2v v = as_half2(pair_bytes(od, ev, k)) * sig2;
    r[2 * k] = v[0];
    r[2 * k + 1] = v[1];
  }
  return r;
}

// E4M3 scale byte (masked to 7 bits) -> fp16 bits of sigma * 2^-8, duplicated in both halves.
__device__ __forceinline__ half2v scale_pair_same(uint32_t s) { return as_half2((s & 0x7Fu) * 0x00800080u); }

template <bool KBF16>
__global__ void __launch_bounds__(256) k_decode(DecodeArgs a) {
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, g = lane >> 4;

  __shared__ __attribute__((aligned(16))) uint16_t q_lds[4][4][kHeadDim];   // [head][term][dim]
  __shared__ float q_descale[4];
  __shared__ float red_m[kWaves][4], red_l[kWaves][4];
  __shared__ __attribute__((aligned(16))) float red_o[kWaves][4][kHeadDim];

  int seq_len = a.seq_lens[b];
  seq_len = seq_len < 0 ? 0 : (seq_len > a.seq_cap ? a.seq_cap : seq_len);
  const int t_begin = split * a.split_tokens;
  const int t_end = min(t_begin + a.split_tokens, seq_len);
  const int64_t unit = static_cast<int64_t>(b) * a.hkv + h;

  if (t_begin >= t_end) {      // empty split (uniform across the workgroup)
    if (a.n_splits == 1) {
      for (int i = tid; i < 4 * kHeadDim; i += 256)
        a.out[(static_cast<int64_t>(b) * a.hq + 4 * h) * kHeadDim + i] = 0.0f;
    } else if (tid < 4) {
      float* ml = a.ws_ml + ((unit * a.n_splits + split) * 4 + tid) * 2;
      ml[0] = -INFINITY;
      ml[1] = 0.0f;
    }
    return;
  }

  // ---------------- query prologue: wavefront w prepares query head 4h + w ----------------
  {
    const int hq = 4 * h + wave;
    const uint32_t qw = reinterpret_cast<const uint32_t*>(a.q + (static_cast<int64_t>(b) * a.hq + hq) * kHeadDim)[lane];
    float x0 = bf16_to_f32(qw & 0xFFFFu), x1 = bf16_to_f32(qw >> 16);
    float scale = a.sm_scale * kLog2e;
    if (!KBF16) {
      if (a.k_flags & NVKV_K_SMOOTH) {
        const float2 sv = reinterpret_cast<const float2*>(a.smooth + h * kHeadDim)[lane];
        x0 *= sv.x;
        x1 *= sv.y;
      }
      if (a.k_flags & NVKV_K_HADAMARD) {
        float u0 = x0 + x1, u1 = x0 - x1;
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
      scale *= a.gscale[0];
    }
    x0 *= scale;
    x1 *= scale;
    float m = fmaxf(fabsf(x0), fabsf(x1));
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) m = fmaxf(m, __shfl_xor(m, d, 64));
    int e = 0;
    if (m > 0.0f) frexpf(m, &e);
    const int p2 = KBF16 ? 0 : 14 - e;           // max |x| * 2^p2 in [2^13, 2^14)
    x0 = ldexpf(x0, p2);
    x1 = ldexpf(x1, p2);
    uint32_t t0, t1, t2;
    if (!KBF16) {
      const _Float16 h0 = static_cast<_Float16>(x0), h1 = static_cast<_Float16>(x1);
      const _Float16 l0 = static_cast<_Float16>(x0 - static_cast<float>(h0));
      const _Float16 l1 = static_cast<_Float16>(x1 - static_cast<float>(h1));
      t0 = __builtin_bit_cast(uint16_t, h0) | (uint32_t(__builtin_bit_cast(uint16_t, h1)) << 16);
      t1 = __builtin_bit_cast(uint16_t, l0) | (uint32_t(__builtin_bit_cast(uint16_t, l1)) << 16);
      t2 = 0u;
    } else {
      const uint32_t a0 = f32_to_bf16_rne(x0), a1 = f32_to_bf16_rne(x1);
      const float r0 = x0 - bf16_to_f32(a0), r1 = x1 - bf16_to_f32(a1);
      const uint32_t b0 = f32_to_bf16_rne(r0), b1 = f32_to_bf16_rne(r1);
      const uint32_t c0 = f32_to_bf16_rne(r0 - bf16_to_f32(b0)), c1 = f32_to_bf16_rne(r1 - bf16_to_f32(b1));
      t0 = a0 | (a1 << 16);
      t1 = b0 | (b1 << 16);
      t2 = c0 | (c1 << 16);
    }
    reinterpret_cast<uint32_t*>(q_lds[wave][0])[lane] = t0;
    reinterpret_cast<uint32_t*>(q_lds[wave][1])[lane] = t1;
    reinterpret_cast<uint32_t*>(q_lds[wave][2])[lane] = t2;
    reinterpret_cast<uint32_t*>(q_lds[wave][3])[lane] = 0u;
    if (lane == 0) q_descale[wave] = ldexpf(1.0f, -p2);
  }
  __syncthreads();

  // B operand of QK (Q'^T): lane (c, g) = column c = (head c>>2, term c&3); instruction u,
  // item e <-> dim 32g + 8u + e.
  u32x4 qb[4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
    qb[u] = *reinterpret_cast<const u32x4*>(&q_lds[c >> 2][c & 3][32 * g + 8 * u]);
  const float descale = q_descale[c >> 2];
  const int term = c & 3;

  float m_ref = -INFINITY;   // running (lazy) max of this lane's head, base-2 units
  float l_acc = 0.0f;        // this lane's share of the softmax denominator
  floatx4 acc[8];
#pragma unroll
  for (int v = 0; v < 8; ++v) acc[v] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

  const int32_t* ptab = a.page_table + static_cast<int64_t>(b) * a.max_pages_per_seq;
  const int ps = a.page_size;

  for (int t0 = t_begin + kIterTok * wave; t0 < t_end; t0 += kIterTok * kWaves) {
    // ---- page lookup per 16-token half (clamped into the valid range for addressing) ----
    int64_t kv_row[2];       // (page * Hkv + h) * ps + page offset of the half's first token
    int64_t sc_base[2];      // byte base of the (page, head) scale array
    int off16[2];
    bool page_ok[2];
#pragma unroll
    for (int eta = 0; eta < 2; ++eta) {
      int tb = t0 + 16 * eta;
      if (tb >= t_end) tb = (t_end - 1) & ~15;
      const int32_t pg = ptab[tb / ps];
      page_ok[eta] = static_cast<uint32_t>(pg) < static_cast<uint32_t>(a.num_pages);
      const int64_t pgc = page_ok[eta] ? pg : 0;
      off16[eta] = tb % ps;
      kv_row[eta] = (pgc * a.hkv + h) * ps + off16[eta];
      sc_base[eta] = (pgc * a.hkv + h) * ps * 8;
    }

    // ---- QK^T ----
    floatx4 sacc[2];
#pragma unroll
    for (int eta = 0; eta < 2; ++eta) {
      sacc[eta] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
      const int64_t row = kv_row[eta] + c;          // A row m = c: token t0 + 16 eta + c
      if (!KBF16) {
        const u32x4 kc = *reinterpret_cast<const u32x4*>(a.k_codes + row * 64 + 16 * g);
        const int tok = off16[eta] + c;
        const uint8_t* sb = a.k_scales + sc_base[eta] + ((tok >> 2) * 8 + 2 * g) * 4 + (tok & 3);
        const half2v s0 = scale_pair_same(sb[0]);
        const half2v s1 = scale_pair_same(sb[4]);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const half8 ak = dequant_dword(kc[u], u < 2 ? s0 : s1);
          sacc[eta] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ak, __builtin_bit_cast(half8, qb[u]), sacc[eta], 0, 0, 0);
        }
      } else {
        const u32x4* kr = reinterpret_cast<const u32x4*>(a.k_codes + row * (kHeadDim * 2) + 64 * g);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const u32x4 kw = kr[u];
          sacc[eta] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kw),
                                                               __builtin_bit_cast(bf16x8, qb[u]), sacc[eta], 0, 0, 0);
        }
      }
    }

    // ---- scores: sum the query terms (columns 4i..4i+3), descale, mask ----
    float s[8];
    float bmax = -INFINITY;
#pragma unroll
    for (int eta = 0; eta < 2; ++eta) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float x = sacc[eta][r];
        x += dpp_xor1(x);
        x += dpp_xor2(x);
        x *= descale;
        const int tok = t0 + 16 * eta + 4 * g + r;
        const bool ok = tok < t_end && page_ok[eta];
        x = ok ? x : -INFINITY;
        s[4 * eta + r] = x;
        bmax = fmaxf(bmax, x);
      }
    }
    bmax = fmaxf(bmax, __shfl_xor(bmax, 16, 64));
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32, 64));

    // ---- lazy running max: move it only when the block max exceeds it by > 8 ----
    const bool need = bmax > m_ref + kLazyMax;
    if (__any(need)) {
      const float m_new = need ? bmax : m_ref;
      const float alpha = exp2f(m_ref - m_new);       // 0 on the first block
      m_ref = m_new;
      l_acc *= alpha;
      const float alpha_row = __shfl(alpha, 4 * g, 64);   // PV rows of lane group g = head g
#pragma unroll
      for (int v = 0; v < 8; ++v) acc[v] *= alpha_row;
    }

    // ---- probabilities -> A operand of PV (row c: head c>>2, term c&3) ----
    const float m_sub = (m_ref == -INFINITY) ? 0.0f : m_ref;   // a fully masked block keeps p = 0
    half8 ap;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = exp2f(s[e] - m_sub);
      l_acc += p;
      const _Float16 ph = static_cast<_Float16>(p);
      const _Float16 pl = static_cast<_Float16>(p - static_cast<float>(ph));
      ap[e] = term == 0 ? ph : (term == 1 ? pl : static_cast<_Float16>(0.0f));
    }

    // ---- V: codes of dims 8c..8c+7 for tokens T(g, e) = 16*(e>>2) + 4g + (e&3) ----
    uint32_t vd[8];
    uint32_t vsc[2];
#pragma unroll
    for (int eta = 0; eta < 2; ++eta) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int tok_rel = 4 * g + j;
        const bool ok = (t0 + 16 * eta + tok_rel) < t_end && page_ok[eta];
        const uint32_t w = *reinterpret_cast<const uint32_t*>(a.v_codes + (kv_row[eta] + tok_rel) * 64 + 4 * c);
        vd[4 * eta + j] = ok ? w : 0u;
      }
      const int quad = (off16[eta] >> 2) + g;
      vsc[eta] = *reinterpret_cast<const uint32_t*>(a.v_scales + sc_base[eta] + (quad * 8 + (c >> 1)) * 4) & 0x7F7F7F7Fu;
    }
    half2v sig[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t w = vsc[p >> 1];
      const int j0 = 2 * (p & 1);
      const uint32_t sel = 0x0Cu | (uint32_t(j0) << 8) | (0x0Cu << 16) | (uint32_t(j0 + 1) << 24);
      sig[p] = as_half2(__builtin_amdgcn_perm(w, w, sel) >> 1);
    }
    uint32_t hev[8], hod[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) nibble_high_bytes(vd[e], hev[e], hod[e]);

#pragma unroll
    for (int v = 0; v < 8; ++v) {
      half8 bv;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t lo = (v & 1) ? hod[2 * p] : hev[2 * p];
        const uint32_t hi = (v & 1) ? hod[2 * p + 1] : hev[2 * p + 1];
        const half2v x = as_half2(pair_bytes(hi, lo, v >> 1)) * sig[p];
        bv[2 * p] = x[0];
        bv[2 * p + 1] = x[1];
      }
      acc[v] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ap, bv, acc[v], 0, 0, 0);
    }
  }

  // ---------------- wavefront partials -> LDS -> workgroup partial ----------------
  float l_tot = l_acc;
  l_tot += __shfl_xor(l_tot, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  if (g == 0 && term == 0) {
    red_m[wave][c >> 2] = m_ref;
    red_l[wave][c >> 2] = l_tot;
  }
  {
    float o8[8];
#pragma unroll
    for (int v = 0; v < 8; ++v) o8[v] = acc[v][0] + acc[v][1];   // rows (head g, terms 0,1)
    float4* dst = reinterpret_cast<float4*>(&red_o[wave][g][8 * c]);
    dst[0] = make_float4(o8[0], o8[1], o8[2], o8[3]);
    dst[1] = make_float4(o8[4], o8[5], o8[6], o8[7]);
  }
  __syncthreads();

  {
    const int i = tid >> 6;              // head
    const int d0 = 2 * (tid & 63);       // dims d0, d0+1
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, red_m[w][i]);
    float L = 0.0f, o0 = 0.0f, o1 = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      if (red_l[w][i] > 0.0f) {
        const float wt = exp2f(red_m[w][i] - M);
        L += wt * red_l[w][i];
        o0 += wt * red_o[w][i][d0];
        o1 += wt * red_o[w][i][d0 + 1];
      }
    }
    const float gv = a.gscale[1];
    if (a.n_splits == 1) {
      const float f = L > 0.0f ? gv / L : 0.0f;
      float2* o = reinterpret_cast<float2*>(a.out + (static_cast<int64_t>(b) * a.hq + 4 * h + i) * kHeadDim + d0);
      *o = make_float2(o0 * f, o1 * f);
    } else {
      const int64_t slot = (unit * a.n_splits + split) * 4 + i;
      *reinterpret_cast<float2*>(a.ws_o + slot * kHeadDim + d0) = make_float2(o0 * gv, o1 * gv);
      if ((tid & 63) == 0) {
        a.ws_ml[slot * 2 + 0] = M;
        a.ws_ml[slot * 2 + 1] = L;
      }
    }
  }
}

// Cross-split log-sum-exp merge: grid (Hkv, B), 256 threads = 4 heads x 64 dim pairs.
__global__ void __launch_bounds__(256) k_decode_merge(DecodeArgs a) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int i = threadIdx.x >> 6, d0 = 2 * (threadIdx.x & 63);
  const int64_t unit = static_cast<int64_t>(b) * a.hkv + h;
  float M = -INFINITY;
  for (int s = 0; s < a.n_splits; ++s) {
    const float* ml = a.ws_ml + ((unit * a.n_splits + s) * 4 + i) * 2;
    if (ml[1] > 0.0f) M = fmaxf(M, ml[0]);
  }
  float L = 0.0f, o0 = 0.0f, o1 = 0.0f;
  for (int s = 0; s < a.n_splits; ++s) {
    const int64_t slot = (unit * a.n_splits + s) * 4 + i;
    const float l = a.ws_ml[slot * 2 + 1];
    if (l > 0.0f) {
      const float wt = exp2f(a.ws_ml[slot * 2] - M);
      const float2 o = *reinterpret_cast<const float2*>(a.ws_o + slot * kHeadDim + d0);
      L += wt * l;
      o0 += wt * o.x;
      o1 += wt * o.y;
    }
  }
  const float f = L > 0.0f ? 1.0f / L : 0.0f;
  *reinterpret_cast<float2*>(a.out + (static_cast<int64_t>(b) * a.hq + 4 * h + i) * kHeadDim + d0) =
      make_float2(o0 * f, o1 * f);
}

// ---------------------------------------------------------------------------------------
// Split plan and launcher
// ---------------------------------------------------------------------------------------
DecodePlan plan_decode(int32_t B, int32_t Hkv, int32_t max_seq_len, int32_t split_tokens) {
  DecodePlan p{};
  const int32_t len = max_seq_len > 0 ? max_seq_len : 1;
  if (split_tokens <= 0) {
    // Aim at ~1024 workgroups in flight (4 per CU over 256 CUs) without cutting a split below
    // one iteration per wavefront.
    const int64_t iters = (len + kIterTok - 1) / kIterTok;
    const int64_t units = static_cast<int64_t>(B) * Hkv;
    int64_t per = (units * iters + 1023) / 1024;
    if (per < kWaves) per = kWaves;
    if (per > iters) per = iters;
    split_tokens = static_cast<int32_t>(per * kIterTok);
  }
  p.split_tokens = split_tokens;
  p.n_splits = (len + split_tokens - 1) / split_tokens;
  return p;
}

size_t decode_workspace_bytes(int32_t B, int32_t Hkv, const DecodePlan& plan) {
  const size_t slots = static_cast<size_t>(B) * Hkv * plan.n_splits * 4;
  const size_t o_bytes = (slots * kHeadDim * sizeof(float) + 255) & ~size_t(255);
  const size_t ml_bytes = (slots * 2 * sizeof(float) + 255) & ~size_t(255);
  return o_bytes + ml_bytes;
}

hipError_t launch_decode(const nvkv_layer& L, const uint16_t* q, int32_t B, int32_t Hq, const int32_t* page_table,
                         int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t max_seq_len, float sm_scale,
                         float* out, void* workspace, const DecodePlan& plan, hipStream_t stream) {
  DecodeArgs a{};
  a.k_codes = static_cast<const uint8_t*>(L.k_data);
  a.k_scales = L.k_scales;
  a.v_codes = static_cast<const uint8_t*>(L.v_data);
  a.v_scales = L.v_scales;
  a.smooth = L.k_smooth;
  a.gscale = L.global_scale;
  a.q = q;
  a.page_table = page_table;
  a.seq_lens = seq_lens;
  a.out = out;
  const size_t slots = static_cast<size_t>(B) * L.num_kv_heads * plan.n_splits * 4;
  a.ws_o = static_cast<float*>(workspace);
  a.ws_ml = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) +
                                     ((slots * kHeadDim * sizeof(float) + 255) & ~size_t(255)));
  a.hkv = L.num_kv_heads;
  a.hq = Hq;
  a.page_size = L.page_size;
  a.num_pages = L.num_pages;
  a.max_pages_per_seq = max_pages_per_seq;
  const int64_t cap_pages = static_cast<int64_t>(max_pages_per_seq) * L.page_size;
  a.seq_cap = static_cast<int32_t>(cap_pages < max_seq_len ? cap_pages : max_seq_len);
  a.split_tokens = plan.split_tokens;
  a.n_splits = plan.n_splits;
  a.k_flags = L.k_flags;
  a.sm_scale = sm_scale;
  const dim3 grid(plan.n_splits, L.num_kv_heads, B);
  if (L.k_fmt == NVKV_FMT_BF16)
    hipLaunchKernelGGL(k_decode<true>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(k_decode<false>, grid, dim3(256), 0, stream, a);
  if (plan.n_splits > 1)
    hipLaunchKernelGGL(k_decode_merge, dim3(L.num_kv_heads, B), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace nvkv
