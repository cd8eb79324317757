// Causal multi-query attention over the packed NVFP4 cache (gfx950, MFMA): the attention of
// a block of Tq query positions per sequence, each position seeing the cached keys up to and
// including its own.  This is the teacher-forced evaluation of [cache post] (opening
// paragraph: the model is scored over full windows while attention reads the quantised
// post-RoPE cache), and the attention of a prefill chunk whose keys were just appended.
//
// [cache post] = rstation.ai post "NVFP4 attention cache on W4A4 Qwen3-8B: static key
// smoothing is near-lossless, key rotations hurt"; [QServe rec] = inference-research record
// "QServe SmoothAttention (4-bit KV cache ...)" (the smoothing factor rides on the query).
//
// Work decomposition: one workgroup of 4 wavefronts per (8 query positions, KV head,
// sequence).  Its 32 rows are (position, query head) of the KV head's group of 4; a row
// block of 16 rows holds 4 positions x 4 heads.  The keys 0..p_last of the tile are cut into
// 32-token iterations dealt round-robin to the wavefronts (split-K inside the workgroup), and
// the four partial softmax states are merged pairwise in LDS at the end, so no workspace is
// needed.
// Per iteration a wavefront does, for both row blocks:
//   QK  S[16 rows x 32 tok] = Q'[16 x 128] Khat^T: the query is held as exact operand terms
//       (two fp16 terms with a power-of-two row prescale, or three bf16 terms for BF16 keys)
//       and each term is one MFMA 16x16x32 per 32 dims, accumulating into the same S.
//       Khat = code * sigma is exact in fp16 (the decode kernel's dequantisation).
//   online softmax per row in the base-2 domain with the lazily moved running max of the
//       decode kernel (threshold 8, so p <= 256); the causal mask drops keys beyond a row's
//       position.
//   PV  O[16 x 128] += P[16 x 32] Vhat[32 x 128]: P split into hi + lo fp16 terms by
//       round-toward-zero packed converts, one MFMA per term and 16-dim tile; P goes from
//       the score layout to the A-operand layout through the wavefront's LDS rows.
// The cache loads, page lookups and V operand construction are those of the decode kernel
// (nvkv_tiles.hpp); tiles are processed longest first (the last query positions).
#include "nvkv_device.hpp"
#include "nvkv_internal.hpp"
#include "nvkv_klt.hpp"
#include "nvkv_tiles.hpp"

namespace nvkv {

struct PrefillArgs {
  const uint8_t* k_codes;     // NVFP4 key codes, or BF16 key rows
  const uint8_t* k_scales;
  const uint8_t* v_codes;
  const uint8_t* v_scales;
  const float* smooth;        // s [Hkv][128]
  const float* gscale;        // {g_K, g_V}
  const uint16_t* q;          // bf16 [B][Tq][Hq][128]
  const int32_t* page_table;  // [B][max_pages_per_seq]
  const int32_t* seq_lens;    // [B]: cached tokens, the Tq query positions included
  float* out;                 // fp32 [B][Tq][Hq][128]
  int32_t hkv, hq, page_size, num_pages, max_pages_per_seq, seq_cap;
  int32_t page_shift;         // log2(page_size) when it is a power of two, else -1
  int32_t tq;                 // query positions per sequence
  uint32_t k_flags;
  float sm_scale;
  const float* basis;         // KLT basis [Hkv][128][128] (NVKV_K_KLT)
};

constexpr int kPfPos = 8;                   // query positions per workgroup
constexpr int kPfRows = 4 * kPfPos;         // rows (position, head)
constexpr int kPfWaves = 4;
constexpr int kPfStride = 20;               // P row stride in dwords (32 fp16 + padding)
constexpr int kPfPWords = 16 * kPfStride;   // one P term of one row block

// LDS: the query terms and per-wavefront P buffers live while the iterations run; the
// partial states of the four wavefronts reuse the same bytes for the final merge.
template <int NT>
struct PfLoopSmem {
  // query terms in QK A-operand order: block (row block, term, instruction u) holds, for
  // lane L = c + 16 g, dims 32g + 8u .. 32g + 8u + 7 of row c (16 B), so a wavefront reads
  // each operand as one contiguous 1 KB
  u32x4 qa[2][NT][4][64];
  float desc[kPfRows];                        // score descale of row R
  uint32_t p[kPfWaves][2][2][kPfPWords];      // [wave][row block][term hi/lo]
};
// Per-wavefront softmax state for the two row blocks: lane (c, g) holds rows 4g..4g+3 of
// each block (one query position, its four heads) in the score layout.
struct PfState {
  float m_ref[2][4];
  float thr[2][4];            // raw-score threshold of the lazy max: (m_ref + 8) / descale
  float l_acc[2][4];
  floatx4 acc[2][8];          // O rows 4g+j, column c <-> dim 8c + v
};

// Pairwise merge of the wavefront states in two rounds through two slots, each holding one
// wavefront's state in its own register layout (per lane: m, l of rows 4g+j of both row
// blocks, and the 16 accumulator quads).
struct PfMergeSmem {
  float m[2][2][4][64];
  float l[2][2][4][64];
  floatx4 o[2][2][8][64];
};
// Fold the state held in merge slot k into this wavefront's state (same lane layout).
__device__ __forceinline__ void pf_merge_from(const PfMergeSmem& ms, int k, int lane, PfState& st) {
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float m1 = st.m_ref[rb][j], m2 = ms.m[k][rb][j][lane];
      const float M = fmaxf(m1, m2);
      const float a1 = m1 == -INFINITY ? 0.0f : exp2f(m1 - M);
      const float a2 = m2 == -INFINITY ? 0.0f : exp2f(m2 - M);
      st.m_ref[rb][j] = M;
      st.l_acc[rb][j] = st.l_acc[rb][j] * a1 + ms.l[k][rb][j][lane] * a2;
#pragma unroll
      for (int v = 0; v < 8; ++v) st.acc[rb][v][j] = st.acc[rb][v][j] * a1 + ms.o[k][rb][v][lane][j] * a2;
    }
}

__device__ __forceinline__ void pf_merge_to(PfMergeSmem& ms, int k, int lane, const PfState& st) {
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ms.m[k][rb][j][lane] = st.m_ref[rb][j];
      ms.l[k][rb][j][lane] = st.l_acc[rb][j];
    }
#pragma unroll
    for (int v = 0; v < 8; ++v) ms.o[k][rb][v][lane] = st.acc[rb][v];
  }
}

template <int NT>
union PfSmem {
  PfLoopSmem<NT> loop;
  PfMergeSmem merge;
  float basis[NT == 2 ? kBasisFloats : 4];    // KLT key basis, query prologue only (NVFP4 keys)
};


// Key part of an iteration's loads (codes and scales, or BF16 rows).
template <bool KBF16>
__device__ __forceinline__ void issue_k_loads(const HalfBase (&hb)[2], const Lane& ln, KLoads<KBF16>& K) {
#pragma unroll
  for (int eta = 0; eta < 2; ++eta) {
    if constexpr (!KBF16) {
      K.kc[eta] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(hb[eta].kc, ln.k_off, 0, kNonTemporal));
      K.ks[eta] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(hb[eta].ks, ln.ks_off, 0, 0));
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        K.kr[eta][u] =
            __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(hb[eta].kc, ln.k_off + 16 * u, 0, kNonTemporal));
    }
  }
}

// Value part of an iteration's loads (codes and scales).
template <bool KBF16>
__device__ __forceinline__ void issue_v_loads(const HalfBase (&hb)[2], const Lane& ln, IterLoads<KBF16>& L) {
#pragma unroll
  for (int eta = 0; eta < 2; ++eta) {
    const u32x4 v4 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(hb[eta].vc, ln.v_off, 0, kNonTemporal));
#pragma unroll
    for (int j = 0; j < 4; ++j) L.vd[2 * j + eta] = v4[j];
    L.vs[eta] = __builtin_amdgcn_raw_buffer_load_b32(hb[eta].vs, ln.vs_off, 0, 0);
  }
}

// V operands of PV instructions 2K (dims 8c + 2K, from ev) and 2K + 1 (from od).
template <int K>
__device__ __forceinline__ void pf_v_operands(const uint32_t (&ev)[4], const uint32_t (&od)[4], const half2v (&sig)[4],
                                              u32x4& be, u32x4& bo) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    be[p] = as_u32(fp4_pair_x256<K>(ev[p]) * sig[p]);
    bo[p] = as_u32(fp4_pair_x256<K>(od[p]) * sig[p]);
  }
}

template <int K>
__device__ __forceinline__ void pf_pv(const uint32_t (&ev)[4], const uint32_t (&od)[4], const half2v (&sig)[4],
                                      const half8 (&ap)[2][2], PfState& st) {
  u32x4 be, bo;
  pf_v_operands<K>(ev, od, sig, be, bo);
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      st.acc[rb][2 * K] =
          __builtin_amdgcn_mfma_f32_16x16x32_f16(ap[rb][t], __builtin_bit_cast(half8, be), st.acc[rb][2 * K], 0, 0, 0);
      st.acc[rb][2 * K + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ap[rb][t], __builtin_bit_cast(half8, bo),
                                                                     st.acc[rb][2 * K + 1], 0, 0, 0);
    }
}

// One 32-token iteration (tokens t0..t0+31) of a wavefront for its 32 rows.  L is the
// wavefront's single load buffer: after_k() runs once QK has consumed L.k and may refill it
// (the next iteration's key loads), after_v() once the V operands have been taken from L.vd
// and L.vs and may refill those; so the loads of the next iteration are in flight during the
// softmax and PV of this one.  ok[eta]: the page of half eta is in range.
template <bool KBF16, int NT, class AfterK, class AfterV>
__device__ __forceinline__ void pf_iter(const IterLoads<KBF16>& L, const bool (&ok)[2], int t0, int t_end,
                                        const u32x4 (&qa)[2][NT][4][64], const float (&desc)[2][4], const int (&pos)[2],
                                        const Lane& ln, uint32_t* p_w, PfState& st, bool full, AfterK&& after_k,
                                        AfterV&& after_v) {
  const int c = ln.c, g = ln.g;
  // ---- QK ----
  // The MFMA phases (QK, PV) run at raised issue priority: the wavefront in such a phase
  // keeps the matrix pipe fed while the other wavefront of the SIMD fills the issue slots
  // in between with its softmax and operand work.
  __builtin_amdgcn_s_setprio(1);
  floatx4 sacc[2][2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int eta = 0; eta < 2; ++eta) sacc[rb][eta] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int eta = 0; eta < 2; ++eta) {
    half2v s0, s1;
    if constexpr (!KBF16) {
      s0 = scale_pair_same(L.k.ks[eta][0] >> ln.ks_shift);
      s1 = scale_pair_same(L.k.ks[eta][1] >> ln.ks_shift);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if constexpr (!KBF16) {
        const half8 bk = dequant_dword(L.k.kc[eta][u], u < 2 ? s0 : s1);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int t = 0; t < NT; ++t)
            sacc[rb][eta] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, qa[rb][t][u][ln.c + 16 * ln.g]), bk,
                                                                   sacc[rb][eta], 0, 0, 0);
      } else {
        const bf16x8 bk = __builtin_bit_cast(bf16x8, L.k.kr[eta][u]);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int t = 0; t < NT; ++t)
            sacc[rb][eta] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qa[rb][t][u][ln.c + 16 * ln.g]), bk,
                                                                    sacc[rb][eta], 0, 0, 0);
      }
    }
  }
  __builtin_amdgcn_s_setprio(0);
  after_k();
  // ---- scores (masked to -inf where needed) and the lazy running max.  The row descale
  // (a power of two) is folded into the exponent's FMA and into each row's raw threshold, so
  // the common case needs no cross-lane reduction: only when some raw score passes its row's
  // threshold is the row max taken and the reference moved. ----
  // full (wave-uniform): every key of the iteration is visible to every row of the tile, so
  // the causal and range masks are skipped (all iterations below the diagonal)
  float x[2][2][4];
  if (full) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int eta = 0; eta < 2; ++eta)
#pragma unroll
        for (int j = 0; j < 4; ++j) x[rb][eta][j] = sacc[rb][eta][j];
  } else {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int eta = 0; eta < 2; ++eta) {
        const bool vis = ok[eta] && (t0 + 16 * eta + c < t_end) && (t0 + 16 * eta + c <= pos[rb]);
#pragma unroll
        for (int j = 0; j < 4; ++j) x[rb][eta][j] = vis ? sacc[rb][eta][j] : -INFINITY;
      }
  }
  bool need_any = false;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int j = 0; j < 4; ++j) need_any |= (x[rb][0][j] > st.thr[rb][j]) | (x[rb][1][j] > st.thr[rb][j]);
  if (__builtin_expect(__any(need_any), 0)) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // rows differ in their causal masks: a row that does not move (possibly still at
        // -inf) keeps alpha = 1 rather than evaluating 2^(-inf + inf)
        const float bmax = row16_max(fmaxf(x[rb][0][j], x[rb][1][j])) * desc[rb][j];
        const bool need = bmax > st.m_ref[rb][j] + kLazyMax;
        const float m_new = need ? bmax : st.m_ref[rb][j];
        const float alpha = need ? exp2f(st.m_ref[rb][j] - m_new) : 1.0f;   // 0 on a row's first keys
        st.m_ref[rb][j] = m_new;
        st.thr[rb][j] = (m_new + kLazyMax) / desc[rb][j];
        st.l_acc[rb][j] *= alpha;
#pragma unroll
        for (int v = 0; v < 8; ++v) st.acc[rb][v][j] *= alpha;
      }
  }
  // p split into hi + lo fp16 terms (|p - hi - lo| < 2^-20 p), written as P rows
  // (row 4g + j, token pair word c = tokens (c, 16 + c)) of the wavefront's buffers
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float neg_m = (st.m_ref[rb][j] == -INFINITY) ? 0.0f : -st.m_ref[rb][j];
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[rb][0][j], desc[rb][j], neg_m));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[rb][1][j], desc[rb][j], neg_m));
      st.l_acc[rb][j] += p0 + p1;
      const half2v hi = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(p0, p1));
      const half2v lo = __builtin_bit_cast(
          half2v, __builtin_amdgcn_cvt_pkrtz(p0 - static_cast<float>(hi[0]), p1 - static_cast<float>(hi[1])));
      p_w[(2 * rb + 0) * kPfPWords + (4 * g + j) * kPfStride + c] = as_u32(hi);
      p_w[(2 * rb + 1) * kPfPWords + (4 * g + j) * kPfStride + c] = as_u32(lo);
    }
  // (LDS operations of one wavefront complete in issue order, and the compiler keeps the
  // reads after the possibly aliasing writes.)
  half8 ap[2][2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int t = 0; t < 2; ++t)
      ap[rb][t] = __builtin_bit_cast(half8, *reinterpret_cast<const u32x4*>(
                                                p_w + (2 * rb + t) * kPfPWords + c * kPfStride + 4 * g));
  // ---- PV: B operand column c <-> dim 8c + v, k = 8g + e <-> token 16 (e & 1) + 4g + (e >> 1) ----
  const uint32_t w0 = L.vs[0] & 0x7F7F7F7Fu, w1 = L.vs[1] & 0x7F7F7F7Fu;
  half2v sig[4];
  uint32_t ev[4], od[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t sel = 0x0Cu | (uint32_t(p) << 8) | (0x0Cu << 16) | (uint32_t(4 + p) << 24);
    sig[p] = as_half2(__builtin_amdgcn_perm(w1, w0, sel) >> 1);
    ev[p] = nib_even(L.vd[2 * p], L.vd[2 * p + 1]);
    od[p] = nib_odd(L.vd[2 * p], L.vd[2 * p + 1]);
  }
  after_v();
  __builtin_amdgcn_s_setprio(1);
  pf_pv<0>(ev, od, sig, ap, st);
  pf_pv<1>(ev, od, sig, ap, st);
  pf_pv<2>(ev, od, sig, ap, st);
  pf_pv<3>(ev, od, sig, ap, st);
  __builtin_amdgcn_s_setprio(0);
}

// Two workgroups per CU, so two wavefronts per SIMD: registers are capped at 256 (launch
// bounds), which the single load buffer fits without spills.
template <bool KBF16>
__global__ void __launch_bounds__(256, 2) k_prefill_attn(PrefillArgs a) {
  constexpr int NT = KBF16 ? 3 : 2;           // query operand terms
  const int n_tiles = static_cast<int>(gridDim.x);
  const int tile = n_tiles - 1 - static_cast<int>(blockIdx.x);   // latest positions first
  const int h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, g = lane >> 4;
  Lane ln;
  ln.c = c;
  ln.g = g;
  ln.k_off = KBF16 ? static_cast<uint32_t>(c * kHeadDim * 2 + 64 * g) : static_cast<uint32_t>(c * 64 + 16 * g);
  ln.ks_off = static_cast<uint32_t>((c >> 2) * 32 + 8 * g);
  ln.ks_shift = static_cast<uint32_t>(8 * (c & 3));
  ln.v_off = static_cast<uint32_t>(16 * (16 * g + c));
  ln.vs_off = static_cast<uint32_t>(32 * g + 4 * (c >> 1));

  __shared__ __attribute__((aligned(16))) PfSmem<NT> sm;
  __shared__ __attribute__((aligned(16))) float q_rot[KBF16 ? 1 : kPfWaves][KBF16 ? 4 : kHeadDim];   // KLT rows

  int n = a.seq_lens[b];
  n = n < 0 ? 0 : (n > a.seq_cap ? a.seq_cap : n);
  const int i0 = tile * kPfPos;                       // first query index of the tile
  const int pos0 = n - a.tq + i0;                     // its position (may be negative)
  const int t_end = min(pos0 + kPfPos, n);            // keys [0, t_end) are needed
  const const_i32_ptr ptab = __builtin_bit_cast(const_i32_ptr, a.page_table) + static_cast<int64_t>(b) * a.max_pages_per_seq;

  // ---- query prologue: wavefront w prepares rows 8w..8w+7 (row R = 4 * position + head) ----
  const bool klt = !KBF16 && (a.k_flags & NVKV_K_KLT);
  if (klt) {                                 // the KLT basis shares the bytes of the loop buffers
    load_basis_lds(a.basis + static_cast<int64_t>(h) * kBasisFloats, sm.basis, threadIdx.x, 64 * kPfWaves);
    __syncthreads();
  }
  {
    float2 sv = make_float2(1.0f, 1.0f);
    if (!KBF16 && (a.k_flags & NVKV_K_SMOOTH)) sv = reinterpret_cast<const float2*>(a.smooth + h * kHeadDim)[lane];
    const float gk = KBF16 ? 1.0f : a.gscale[0];
    uint32_t qw[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int R = 8 * wave + k;
      const int i = i0 + (R >> 2);
      qw[k] = 0u;
      if (i < a.tq)
        qw[k] = reinterpret_cast<const uint32_t*>(
            a.q + ((static_cast<int64_t>(b) * a.tq + i) * a.hq + 4 * h + (R & 3)) * kHeadDim)[lane];
    }
    uint32_t w[8][3];
    float descale[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      descale[k] = query_terms<KBF16>(qw[k], sv, a.k_flags, a.sm_scale, gk, lane, w[k][0], w[k][1], w[k][2],
                                      sm.basis, q_rot[KBF16 ? 0 : wave]);
    if (klt) __syncthreads();               // every wavefront is done with the basis
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int R = 8 * wave + k;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int d = 2 * lane;                                  // dims d, d + 1
        const int gg = d >> 5, uu = (d & 31) >> 3, ww = (d & 7) >> 1;
        reinterpret_cast<uint32_t*>(&sm.loop.qa[R >> 4][t][uu][(R & 15) + 16 * gg])[ww] = w[k][t];
      }
      if (lane == 0) sm.loop.desc[R] = descale[k];
    }
  }
  __syncthreads();

  PfState st;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      st.m_ref[rb][j] = -INFINITY;
      st.thr[rb][j] = -INFINITY;
      st.l_acc[rb][j] = 0.0f;
    }
#pragma unroll
    for (int v = 0; v < 8; ++v) st.acc[rb][v] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  }

  if (t_end > 0) {
    // A operands of QK come from LDS at each use (sm.loop.qa): in registers they would take
    // 64-96 of the 256
    float desc[2][4];
    int pos[2];                                       // position of the lane's score rows
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
      for (int j = 0; j < 4; ++j) desc[rb][j] = sm.loop.desc[16 * rb + 4 * g + j];
      pos[rb] = pos0 + 4 * rb + g;
    }
    uint32_t* p_w = sm.loop.p[wave][0][0];

    // iterations it = wave, wave + 4, ...
    const int n_it = (t_end + kIterTok - 1) / kIterTok;
    // One register buffer: the next iteration's key loads are issued as soon as QK has
    // consumed this one's keys, its value loads once the V operands are extracted (pf_iter's
    // callbacks).  Two buffers would push the kernel past 256 registers (one wavefront per
    // SIMD instead of two) and cost 1.6x (measured).
    IterLoads<KBF16> buf;
    HalfBase hb[2];
    int it = wave;
    if (it < n_it) {
      half_bases<KBF16>(a, load_pages(a, ptab, kIterTok * it, t_end), h, hb);
      issue_loads<KBF16>(hb, ln, buf);
    }
    for (; it < n_it; it += kPfWaves) {
      // (a separate unmasked instance for the iterations below the diagonal spills registers
      // and runs 4x slower: measured)
      const int t_last = kIterTok * it + kIterTok - 1;
      const bool full = __all(hb[0].ok && hb[1].ok && t_last < t_end && t_last <= pos0);
      const bool ok[2] = {hb[0].ok, hb[1].ok};
      const bool has_next = it + kPfWaves < n_it;
      // page entries of the next iteration (scalar loads), needed once QK is done
      IterPages pn{};
      if (has_next) pn = load_pages(a, ptab, kIterTok * (it + kPfWaves), t_end);
      pf_iter<KBF16, NT>(
          buf, ok, kIterTok * it, t_end, sm.loop.qa, desc, pos, ln, p_w, st, full,
          [&] {
            if (has_next) {
              half_bases<KBF16>(a, pn, h, hb);
              issue_k_loads<KBF16>(hb, ln, buf.k);
            }
          },
          [&] {
            if (has_next) issue_v_loads<KBF16>(hb, ln, buf);
          });
    }
  }
  __syncthreads();     // every wavefront is done with the query terms and P buffers

  // ---- workgroup merge: waves 2, 3 -> 0, 1; then 1 -> 0, which writes the output ----
  if (wave >= 2) pf_merge_to(sm.merge, wave - 2, lane, st);
  __syncthreads();
  if (wave < 2) pf_merge_from(sm.merge, wave, lane, st);
  __syncthreads();
  if (wave == 1) pf_merge_to(sm.merge, 0, lane, st);
  __syncthreads();
  if (wave != 0) return;
  pf_merge_from(sm.merge, 0, lane, st);
  const float gv = a.gscale[1];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float L = row16_sum(st.l_acc[rb][j]);
      const int R = 16 * rb + 4 * g + j;                  // row (position 4rb + g, head j)
      const int i = i0 + (R >> 2);
      if (i < a.tq) {
        const float f = L > 0.0f ? gv / L : 0.0f;
        float4* dst = reinterpret_cast<float4*>(
            a.out + ((static_cast<int64_t>(b) * a.tq + i) * a.hq + 4 * h + j) * kHeadDim + 8 * c);
        dst[0] = make_float4(st.acc[rb][0][j] * f, st.acc[rb][1][j] * f, st.acc[rb][2][j] * f, st.acc[rb][3][j] * f);
        dst[1] = make_float4(st.acc[rb][4][j] * f, st.acc[rb][5][j] * f, st.acc[rb][6][j] * f, st.acc[rb][7][j] * f);
      }
    }
}

hipError_t launch_prefill_attention(const nvkv_layer& L, const uint16_t* q, int32_t B, int32_t Tq, int32_t Hq,
                                    const int32_t* page_table, int32_t max_pages_per_seq, const int32_t* seq_lens,
                                    int32_t max_seq_len, float sm_scale, float* out, hipStream_t stream) {
  PrefillArgs a{};
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
  a.hkv = L.num_kv_heads;
  a.hq = Hq;
  a.page_size = L.page_size;
  a.page_shift = (L.page_size & (L.page_size - 1)) == 0 ? __builtin_ctz(static_cast<unsigned>(L.page_size)) : -1;
  a.num_pages = L.num_pages;
  a.max_pages_per_seq = max_pages_per_seq;
  const int64_t cap_pages = static_cast<int64_t>(max_pages_per_seq) * L.page_size;
  a.seq_cap = static_cast<int32_t>(cap_pages < max_seq_len ? cap_pages : max_seq_len);
  a.tq = Tq;
  a.k_flags = L.k_flags;
  a.sm_scale = sm_scale;
  a.basis = L.k_basis;
  const dim3 grid((Tq + kPfPos - 1) / kPfPos, L.num_kv_heads, B);
  const dim3 block(64 * kPfWaves);
  if (L.k_fmt == NVKV_FMT_BF16)
    hipLaunchKernelGGL((k_prefill_attn<true>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((k_prefill_attn<false>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace nvkv
