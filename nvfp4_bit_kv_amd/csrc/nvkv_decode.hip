// Split-K GQA decode attention over the packed NVFP4 cache (gfx950, MFMA).
//
// [cache post] = rstation.ai post "NVFP4 attention cache on W4A4 Qwen3-8B: static key
// smoothing is near-lossless, key rotations hurt": attention over the NVFP4 post-RoPE cache,
// keys smoothed per channel (queries carry the factor) and optionally in a Hadamard-128 basis.
// [QServe rec] = inference-research record "QServe SmoothAttention (4-bit KV cache ...)":
// the smoothing factor is folded into the query; attention is kept memory-bound so the 4-bit
// cache pays off.
//
// Work decomposition: one workgroup (4..16 wavefronts) per (split, KV head, sequence); the
// split's tokens are cut into 32-token iterations dealt round-robin to the wavefronts; the
// plan aims at about one workgroup per CU.  Per iteration a wavefront does:
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
// V codes are stored quad-interleaved (the four tokens of a quad side by side per 8-dim
// word), so lane (c, g) fetches word c of its four tokens of each half with one 16-byte load
// and serves column c of PV instruction v as dim 8c + v.
// Dequantisation: nibble -> fp16 (value * 2^8) with the gfx950 scaled FP4 convert (it
// applies only the exponent of its scale operand, so the scale is 2^8), E4M3 scale -> fp16
// (sigma * 2^-8) by a bit shift, one v_pk_mul_f16 per element pair; the product is the exact
// code * sigma.
// Partials (unnormalised O, running max m, sum l) are merged across wavefronts in LDS and,
// when a sequence has several splits, across workgroups by the last workgroup of the
// (sequence, KV head) to finish: partials travel through device-coherent stores and loads
// and one arrival counter per (sequence, KV head) in the workspace (reset by that
// workgroup), so a single launch produces the output without any cache writeback.
// Latency: the query row, page-table entries and the first two iterations' cache loads are
// issued at kernel start, before the sequence length is known; later iterations are
// software-pipelined two deep.
#include <mutex>
#include <unordered_map>

#include "nvkv_device.hpp"
#include "nvkv_encode.hpp"
#include "nvkv_internal.hpp"
#include "nvkv_klt.hpp"
#include "nvkv_tiles.hpp"

namespace nvkv {

constexpr int kMaxWaves = 16;   // wavefronts per workgroup: 4..16 (runtime, blockDim.x / 64)

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
  unsigned* counters;         // [B][Hkv] arrival counters (kCounterStride apart), zero between calls
  int32_t hkv, hq, page_size, num_pages, max_pages_per_seq, seq_cap;
  int32_t page_shift;         // log2(page_size) when it is a power of two, else -1
  int32_t split_tokens, n_splits;
  uint32_t k_flags;
  float sm_scale;
  // fused append (k_decode<.., .., true>): the new token of sequence b, at position
  // seq_len - 1, is quantised into the cache and attended from registers
  const uint16_t* k_new;      // bf16 [B][Hkv][128]
  const uint16_t* v_new;      // bf16 [B][Hkv][128]
  const float* inv_smooth;    // r [Hkv][128] (key smoothing)
  uint8_t* k_codes_w;         // writable views of the cache arrays
  uint8_t* k_scales_w;
  uint8_t* v_codes_w;
  uint8_t* v_scales_w;
  const float* basis;         // KLT basis [Hkv][128][128] (NVKV_K_KLT), staged in dynamic LDS
  uint64_t* trace;            // phase stamps of the measurement instance (TRACE), else unused
};

// Phase stamps of the measurement instance k_decode<..., TRACE = true>: s_memrealtime values
// (a 100 MHz counter common to the whole chip) per workgroup, kTraceSlots apart, in the
// linear workgroup order split + n_splits * (h + Hkv * b).  Slots:
//   0 entry; 1 query prologue barrier passed; 2 first workgroup (LDS) merge barrier passed;
//   3 split partials acknowledged (after the workgroup barrier); 4 arrival counter returned;
//   5 merging workgroup: splits loaded and folded, output stores issued; 6 output stores
//   complete; 7 identity: bit 0 = merging workgroup, bits 8..39 = HW_ID, bits 40..47 =
//   XCC_ID, bits 48..63 = split index; 8 split partial stores issued; 9 merging workgroup:
//   split partials in registers; with the KLT basis (wavefront 0): 10 its quarter of the
//   basis staged, 11 the basis barrier passed, 12 its query head transformed;
//   16 + w: wavefront w's first cache data in registers; 32 + w: wavefront w's loop done
//   (w < 16).  Slots a workgroup never reaches stay 0.
constexpr int kTraceSlots = 48;
struct TraceStamps {
  uint64_t entry = 0, prologue = 0, lds_merge = 0, acked = 0, counted = 0, folded = 0, stored = 0, ident = 0;
  uint64_t issue = 0, loaded = 0;
  uint64_t basis = 0, basis_bar = 0, query = 0;
  uint64_t data = 0, done = 0;     // this wavefront's
};
// the scheduling barriers keep the stamp where it is written relative to the code around it
__device__ __forceinline__ uint64_t stamp_now() {
  __builtin_amdgcn_sched_barrier(0);
  const uint64_t t = __builtin_amdgcn_s_memrealtime();
  __builtin_amdgcn_sched_barrier(0);
  return t;
}
__device__ __forceinline__ uint64_t hw_identity() {
  uint32_t hw, xcc;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
  return (static_cast<uint64_t>(hw) << 8) | (static_cast<uint64_t>(xcc & 0xFFu) << 40);
}
__device__ __forceinline__ void trace_write(const DecodeArgs& a, const TraceStamps& t, int wave, int tid) {
  const int64_t wg = blockIdx.x + static_cast<int64_t>(gridDim.x) * (blockIdx.y + static_cast<int64_t>(gridDim.y) * blockIdx.z);
  uint64_t* r = a.trace + wg * kTraceSlots;
  if ((tid & 63) == 0 && wave < 16) {
    r[16 + wave] = t.data;
    r[32 + wave] = t.done;
  }
  if (tid == 0) {
    r[0] = t.entry;
    r[1] = t.prologue;
    r[2] = t.lds_merge;
    r[3] = t.acked;
    r[4] = t.counted;
    r[5] = t.folded;
    r[6] = t.stored;
    r[7] = t.ident;
    r[8] = t.issue;
    r[9] = t.loaded;
    r[10] = t.basis;
    r[11] = t.basis_bar;
    r[12] = t.query;
  }
}

// Online-softmax state of one wavefront.  Lane (c, g) serves query head g: its running max,
// its share of the denominator and the PV accumulator rows 4g..4g+3 = (head g, term 0..3).
struct SoftmaxState {
  float m_ref;          // lazy running max of head g (base-2 units)
  float l_acc;          // lane's share of head g's denominator
  floatx4 acc[8];       // PV accumulators: column c <-> dim 8c + v
};

// P transpose buffer of a wavefront in LDS: 16 rows (head i, term t) of 32 fp16 in the PV
// token order k, row stride kPStride dwords (padded against bank conflicts).
constexpr int kPStride = 20;
constexpr int kPWords = 16 * kPStride;

// PV for dims 8c + 2K (from ev) and 8c + 2K + 1 (from od): instructions v = 2K, 2K + 1.
template <int K>
__device__ __forceinline__ void pv_pair(const uint32_t (&ev)[4], const uint32_t (&od)[4], const half2v (&sig)[4],
                                        const half8& ap, SoftmaxState& st) {
  u32x4 be, bo;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    be[p] = as_u32(fp4_pair_x256<K>(ev[p]) * sig[p]);
    bo[p] = as_u32(fp4_pair_x256<K>(od[p]) * sig[p]);
  }
  st.acc[2 * K] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ap, __builtin_bit_cast(half8, be), st.acc[2 * K], 0, 0, 0);
  st.acc[2 * K + 1] =
      __builtin_amdgcn_mfma_f32_16x16x32_f16(ap, __builtin_bit_cast(half8, bo), st.acc[2 * K + 1], 0, 0, 0);
}

// One 32-token iteration of a wavefront.  valid[eta]: token c of half eta is inside the split
// and its page index is in range.
template <bool KBF16>
__device__ __forceinline__ void compute_iter(const IterLoads<KBF16>& L, const bool (&valid)[2], const u32x4 (&qa)[4],
                                             float descale, const Lane& ln, SoftmaxState& st, uint32_t* p_w) {
  // ---- QK: S = Q' Khat^T.  A = Q' (row = (head, term)), B = Khat^T (column = token c of the
  // half); lane (c, g) receives rows 4g..4g+3 = the query terms of head g for token c ----
  floatx4 sacc[2];
#pragma unroll
  for (int eta = 0; eta < 2; ++eta) {
    sacc[eta] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (!KBF16) {
      const half2v s0 = scale_pair_same(L.k.ks[eta][0] >> ln.ks_shift);
      const half2v s1 = scale_pair_same(L.k.ks[eta][1] >> ln.ks_shift);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const half8 bk = dequant_dword(L.k.kc[eta][u], u < 2 ? s0 : s1);
        sacc[eta] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, qa[u]), bk, sacc[eta], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        sacc[eta] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qa[u]),
                                                             __builtin_bit_cast(bf16x8, L.k.kr[eta][u]), sacc[eta],
                                                             0, 0, 0);
    }
  }
  float s[2];
#pragma unroll
  for (int eta = 0; eta < 2; ++eta) {
    float x = sacc[eta][0] + sacc[eta][1];       // fp16 queries: terms 2, 3 are zero
    if constexpr (KBF16) x += sacc[eta][2];      // bf16 queries: three terms
    s[eta] = valid[eta] ? x : -INFINITY;
  }
  const float bmax = row16_max(fmaxf(s[0], s[1])) * descale;   // descale > 0: max commutes with it
  // ---- lazy running max: it moves only when a block max exceeds it by more than 8 ----
  const bool need = bmax > st.m_ref + kLazyMax;
  if (__builtin_expect(__any(need), 0)) {
    const float m_new = need ? bmax : st.m_ref;
    const float alpha = exp2f(st.m_ref - m_new);           // 0 on the first block
    st.m_ref = m_new;
    st.l_acc *= alpha;
#pragma unroll
    for (int v = 0; v < 8; ++v) st.acc[v] *= alpha;
  }
  const float neg_m = (st.m_ref == -INFINITY) ? 0.0f : -st.m_ref;   // a fully masked block keeps p = 0
  // p = 2^(s*descale - m) <= 256, split into hi + lo fp16 terms by round-toward-zero packed
  // converts (|p - hi - lo| < 2^-20 p); PV rows (head, 0) take hi, (head, 1) lo.
  const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[0], descale, neg_m));
  const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[1], descale, neg_m));
  st.l_acc += p0 + p1;
  const half2v hi = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(p0, p1));
  const half2v lo = __builtin_bit_cast(
      half2v, __builtin_amdgcn_cvt_pkrtz(p0 - static_cast<float>(hi[0]), p1 - static_cast<float>(hi[1])));
  // ---- P: scores layout (lane = token) -> PV A-operand layout (lane = row, 8 tokens) through
  // the wavefront's LDS rows.  PV token order k = 2c + eta, i.e. k = 8g' + e is token
  // 16 (e & 1) + 4 g' + (e >> 1). ----
  // (LDS operations of one wavefront complete in issue order, and the compiler keeps the
  // read after the possibly aliasing writes.)
  p_w[(4 * ln.g + 0) * kPStride + ln.c] = as_u32(hi);
  p_w[(4 * ln.g + 1) * kPStride + ln.c] = as_u32(lo);
  const half8 ap = __builtin_bit_cast(half8, *reinterpret_cast<const u32x4*>(p_w + ln.c * kPStride + 4 * ln.g));
  // ---- V: B operand column c <-> dim 8c + v, k = 8g + e <-> token T(g, e) as above.  The
  // scale pair of (k = 8g+2p, 8g+2p+1) is (half 0, half 1) token 4g+p, block c >> 1.
  // Masked tokens need no zeroing: p = 0 there and every code and scale decodes finite. ----
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
  pv_pair<0>(ev, od, sig, ap, st);
  pv_pair<1>(ev, od, sig, ap, st);
  pv_pair<2>(ev, od, sig, ap, st);
  pv_pair<3>(ev, od, sig, ap, st);
}

// Device-coherent 64-bit store / load (relaxed, device scope): they bypass the
// non-coherent per-die L2 state, which is what the cross-workgroup merge needs.
__device__ __forceinline__ void store_coherent_f2(float* p, float x, float y) {
  const unsigned long long v = (static_cast<unsigned long long>(__float_as_uint(y)) << 32) | __float_as_uint(x);
  __hip_atomic_store(reinterpret_cast<unsigned long long*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 load_coherent_f2(const float* p) {
  const unsigned long long v = __hip_atomic_load(reinterpret_cast<const unsigned long long*>(p), __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float(static_cast<uint32_t>(v)), __uint_as_float(static_cast<uint32_t>(v >> 32)));
}
// s_waitcnt vmcnt(0) expcnt(7) lgkmcnt(15): wait for this wave's vector memory operations
// (stores included) to complete.
constexpr int kWaitVmcnt0 = 0x0F70;

// Cross-split log-sum-exp merge run by the last workgroup of (b, h): wavefront w owns query
// head 4h + w, lane l its dims 2l, 2l+1.  Splits are read G at a time with device-coherent
// loads, all loads of a group independent (one memory round trip per group), and folded in
// with a running max.
constexpr int kMaxSplits = 1024;
// Arrival counters sit 256 bytes apart: the device-scope atomics of all workgroups would
// otherwise queue on one or two cache lines (measured: 0.8 us per launch at 4 x 2304).
constexpr int kCounterStride = 64;

template <int G, bool TRACE = false>
__device__ __forceinline__ void merge_splits(const DecodeArgs& a, int64_t unit, int i, int d0, float gv,
                                             uint64_t* loaded = nullptr) {
  const int n = a.n_splits;
  float M = -INFINITY, L = 0.0f, o0 = 0.0f, o1 = 0.0f;
  for (int s0 = 0; s0 < n; s0 += G) {
    float2 ml[G], o[G];
#pragma unroll
    for (int k = 0; k < G; ++k) {
      const int sp = s0 + k < n ? s0 + k : n - 1;
      const int64_t slot = (unit * n + sp) * 4 + i;
      ml[k] = load_coherent_f2(a.ws_ml + slot * 2);
      o[k] = load_coherent_f2(a.ws_o + slot * kHeadDim + d0);
      if (s0 + k >= n) ml[k] = make_float2(-INFINITY, 0.0f);   // padding entry: no weight
    }
    if constexpr (TRACE) {
      if (s0 == 0) {
        __builtin_amdgcn_s_waitcnt(0x0F70);
        *loaded = __builtin_amdgcn_s_memrealtime();
      }
    }
    // a split without tokens carries m = -inf and l = 0; raw exp2 gives exp2(-inf) = 0 and
    // weights in (0, 1]
    float mx = M;
#pragma unroll
    for (int k = 0; k < G; ++k) mx = fmaxf(mx, ml[k].x);
    const float mr = mx == -INFINITY ? 0.0f : mx;
    const float sc = __builtin_amdgcn_exp2f(M - mr);   // 0 while M is still -inf
    L *= sc;
    o0 *= sc;
    o1 *= sc;
#pragma unroll
    for (int k = 0; k < G; ++k) {
      const float w = __builtin_amdgcn_exp2f(ml[k].x - mr);
      L = __builtin_fmaf(w, ml[k].y, L);
      o0 = __builtin_fmaf(w, o[k].x, o0);
      o1 = __builtin_fmaf(w, o[k].y, o1);
    }
    M = mx;
  }
  const float f = L > 0.0f ? gv / L : 0.0f;
  const int b = static_cast<int>(unit / a.hkv), h = static_cast<int>(unit % a.hkv);
  *reinterpret_cast<float2*>(a.out + (static_cast<int64_t>(b) * a.hq + 4 * h + i) * kHeadDim + d0) =
      make_float2(o0 * f, o1 * f);
}

// ---------------------------------------------------------------------------------------
// Fused append of the new token
// ---------------------------------------------------------------------------------------
// The new token as token 0 of a (page, head) block in the cache layouts (only the bytes of
// token 0), in LDS.
struct NewTokenStage {
  uint8_t kc[kHeadDim * 2];        // key row (64 B NVFP4 or 256 B bf16)
  uint8_t ks[32];                  // key scales: block b at byte 4b (token 0 of its quad)
  uint8_t vc[256];                 // value words: word w at byte 16w (quad-interleaved)
  uint8_t vs[32];                  // value scales: block b at byte 4b
  float ky[kHeadDim];              // transformed key row (MSE-searched key scales only)
};

// Registers of the encoding wavefront: the whole wavefront encodes the new token, lane L
// holding elements 4(L & 31) .. 4(L & 31) + 3 of the key row (L < 32) or the value row
// (L >= 32), i.e. quarter L & 3 of block (L >> 2) & 7.  Loaded at kernel start.
struct NewTokenRegs {
  uint2 raw;            // 4 bf16 elements
  float4 r;             // key smoothing factors of those elements (key lanes, smoothing on)
  float g;              // tensor scale of the lane's row
};

template <bool KBF16>
__device__ __forceinline__ void new_token_load(const DecodeArgs& a, int b, int h, int lane, NewTokenRegs& R) {
  const bool is_v = lane >= 32;
  const int64_t row = (static_cast<int64_t>(b) * a.hkv + h) * kHeadDim;
  R.raw = reinterpret_cast<const uint2*>((is_v ? a.v_new : a.k_new) + row)[lane & 31];
  R.g = a.gscale[is_v ? 1 : 0];
  R.r = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
  if (!KBF16 && !is_v && (a.k_flags & NVKV_K_SMOOTH))
    R.r = reinterpret_cast<const float4*>(a.inv_smooth + h * kHeadDim)[lane & 31];
}

// One Hadamard stage across lanes: element i of this lane pairs with element i of lane
// (lane ^ m), the lower lane keeping the sum, the upper the difference (lower - upper).
__device__ __forceinline__ void had_cross(float (&y)[4], int lane, int m) {
#pragma clang fp contract(off)   // part of the bit-exact key transform
  const bool upper = (lane & m) != 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float p = __shfl_xor(y[i], m, 64);
    y[i] = upper ? (p - y[i]) : (y[i] + p);
  }
}

// Transform of the new token's key row (the key transform of quantize_append_kv, four
// elements per lane): lane L < 32 leaves elements 4L .. 4L + 3 of the transformed key in y;
// lanes >= 32 leave their value elements untouched.  The whole wavefront takes part (the
// Hadamard butterfly and the KLT rotation are cross-lane).
template <bool KBF16>
__device__ __forceinline__ void new_token_transform(const DecodeArgs& a, int lane, const NewTokenRegs& R,
                                                    NewTokenStage& st, const float* basis_lds, float (&y)[4]) {
#pragma clang fp contract(off)   // part of the bit-exact key transform
  const bool is_v = lane >= 32;
  y[0] = bf16_to_f32(R.raw.x & 0xFFFFu);
  y[1] = bf16_to_f32(R.raw.x >> 16);
  y[2] = bf16_to_f32(R.raw.y & 0xFFFFu);
  y[3] = bf16_to_f32(R.raw.y >> 16);
  if (KBF16) return;
  if (!is_v && (a.k_flags & NVKV_K_SMOOTH)) {             // y_j = fl32(x_j * r_j)
    y[0] = y[0] * R.r.x;
    y[1] = y[1] * R.r.y;
    y[2] = y[2] * R.r.z;
    y[3] = y[3] * R.r.w;
  }
  if (!is_v && (a.k_flags & NVKV_K_HADAMARD)) {           // stages h = 1, 2, ..., 64 in order
    float t0 = y[0] + y[1], t1 = y[0] - y[1], t2 = y[2] + y[3], t3 = y[2] - y[3];
    y[0] = t0 + t2;
    y[2] = t0 - t2;
    y[1] = t1 + t3;
    y[3] = t1 - t3;
    had_cross(y, lane, 1);                                // h = 4
    had_cross(y, lane, 2);                                // h = 8
    had_cross(y, lane, 4);                                // h = 16
    had_cross(y, lane, 8);                                // h = 32
    had_cross(y, lane, 16);                               // h = 64
  }
  if (a.k_flags & NVKV_K_KLT) {
    // z = B^T y in the fixed rounding order of the append kernel (each output a chain of
    // fused multiply-adds over j), on the whole wavefront: the key row goes through LDS,
    // lane l forms z[2l] and z[2l + 1], and key lane L then reads back z[4L .. 4L + 3]
    if (!is_v) *reinterpret_cast<float4*>(&st.ky[4 * (lane & 31)]) = make_float4(y[0], y[1], y[2], y[3]);
    float z0 = 0.0f, z1 = 0.0f;
    // the reads of step j4 + 1 go out before the multiply-adds of step j4 (the two chains
    // are latency-bound otherwise)
    float4 y4 = *reinterpret_cast<const float4*>(&st.ky[0]);
    float2 bj[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) bj[u] = *reinterpret_cast<const float2*>(basis_lds + u * kHeadDim + 2 * lane);
#pragma unroll
    for (int j4 = 0; j4 < kHeadDim / 4; ++j4) {
      float4 y4n = y4;
      float2 bn[4] = {bj[0], bj[1], bj[2], bj[3]};
      if (j4 + 1 < kHeadDim / 4) {
        y4n = *reinterpret_cast<const float4*>(&st.ky[4 * (j4 + 1)]);
#pragma unroll
        for (int u = 0; u < 4; ++u)
          bn[u] = *reinterpret_cast<const float2*>(basis_lds + (4 * (j4 + 1) + u) * kHeadDim + 2 * lane);
      }
      const float yv[4] = {y4.x, y4.y, y4.z, y4.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        z0 = __builtin_fmaf(bj[u].x, yv[u], z0);
        z1 = __builtin_fmaf(bj[u].y, yv[u], z1);
      }
      y4 = y4n;
#pragma unroll
      for (int u = 0; u < 4; ++u) bj[u] = bn[u];
    }
    *reinterpret_cast<float2*>(&st.ky[2 * lane]) = make_float2(z0, z1);
    const float4 zk = *reinterpret_cast<const float4*>(&st.ky[4 * (lane & 31)]);
    if (!is_v) {
      y[0] = zk.x;
      y[1] = zk.y;
      y[2] = zk.z;
      y[3] = zk.w;
    }
  }
}

// Encode the new token from its transformed rows y (new_token_transform): the LDS stage
// receives it as token 0 of a 16-token block in the cache layouts, and the cache slot too
// when its page is in range (page pg, offset off).
template <bool KBF16>
__device__ __forceinline__ void new_token_encode(const DecodeArgs& a, int h, int lane, const NewTokenRegs& R,
                                                 const float (&y)[4], int32_t pg, int off, bool ok,
                                                 NewTokenStage& st) {
#pragma clang fp contract(off)
  const bool is_v = lane >= 32;
  const int blk = (lane >> 2) & 7, qtr = lane & 3;
  const int64_t ph = static_cast<int64_t>(ok ? pg : 0) * a.hkv + h;
  const int64_t row_index = ph * a.page_size + off;
  if (KBF16 && !is_v) {                                   // bf16 keys: plain copy of the row
    *reinterpret_cast<uint2*>(st.kc + 8 * (lane & 31)) = R.raw;
    if (ok) *reinterpret_cast<uint2*>(a.k_codes_w + row_index * (kHeadDim * 2) + 8 * (lane & 31)) = R.raw;
    return;
  }
  // block absmax over the block's four lanes, scale code, E2M1 nibbles
  float A = fmaxf(fmaxf(fabsf(y[0]), fabsf(y[1])), fmaxf(fabsf(y[2]), fabsf(y[3])));
  A = fmaxf(A, __shfl_xor(A, 1, 64));
  A = fmaxf(A, __shfl_xor(A, 2, 64));
  uint32_t S = e4m3_scale_code(A, R.g);
  if (!KBF16 && (a.k_flags & NVKV_K_MSE_SCALE)) {
    // MSE-searched key scales: the key row goes through LDS and the whole wavefront
    // searches its 8 blocks (8 lanes per block); key lane L then takes block (L >> 2) & 7's code
    if (!is_v) *reinterpret_cast<float4*>(&st.ky[4 * (lane & 31)]) = make_float4(y[0], y[1], y[2], y[3]);
    const uint32_t s_row = mse_scale_code_row(st.ky, a.gscale[0], lane);
    const uint32_t s_blk = static_cast<uint32_t>(__shfl(static_cast<int>(s_row), 8 * blk, 64));
    if (!is_v) S = s_blk;
  }
  const float sigma = e4m3_value(S);
  uint32_t bits = 0u;
  if (sigma > 0.0f) {
    const E2m1Thresholds t(sigma, R.g);
#pragma unroll
    for (int i = 0; i < 4; ++i) bits |= e2m1_nibble(y[i], t) << (4 * i);
  }
  // word w = 2 blk + (qtr >> 1) holds elements 8w..8w+7: even quarters take the odd
  // neighbour's 16 bits as their high half
  const uint32_t hi16 = static_cast<uint32_t>(__shfl_xor(static_cast<int>(bits), 1, 64));
  const uint32_t word = bits | (hi16 << 16);
  const int w = 2 * blk + (qtr >> 1);
  const int64_t sc = ph * a.page_size * 8 + ((off >> 2) * 8 + blk) * 4 + (off & 3);
  if ((qtr & 1) == 0) {
    if (!is_v) {
      *reinterpret_cast<uint32_t*>(st.kc + 4 * w) = word;
      if (ok) *reinterpret_cast<uint32_t*>(a.k_codes_w + row_index * 64 + 4 * w) = word;
    } else {
      *reinterpret_cast<uint32_t*>(st.vc + 16 * w) = word;
      if (ok) *reinterpret_cast<uint32_t*>(a.v_codes_w + (row_index - (off & 3)) * 64 + 16 * w + 4 * (off & 3)) = word;
    }
  }
  if (qtr == 0) {
    (is_v ? st.vs : st.ks)[4 * blk] = static_cast<uint8_t>(S);
    if (ok) (is_v ? a.v_scales_w : a.k_scales_w)[sc] = static_cast<uint8_t>(S);
  }
}

// Add the staged new token to a wavefront's softmax state (a single-token update instead of
// an MFMA iteration).  Scores: lane L takes dims 2L, 2L+1 of the four query heads (terms hi +
// lo from the query LDS image, exact in fp32) against the staged key (code * sigma, exact in
// fp16) and the sums are reduced over the wavefront.  Lane (c, g) then updates head g: the
// lazy max, the denominator (one lane per head) and row (g, term 0) of the accumulators with
// p * value(dims 8c..8c+7) in fp32.
template <bool KBF16>
__device__ __forceinline__ void new_token_update(const NewTokenStage& st, const uint16_t (*q_lds)[4][kHeadDim],
                                                 const float* q_descale, int lane, const Lane& ln,
                                                 SoftmaxState& sm) {
  float kx, ky;
  if constexpr (!KBF16) {
    const uint32_t kw = *reinterpret_cast<const uint32_t*>(st.kc + 4 * (lane >> 2));
    const uint32_t byte_sel = static_cast<uint32_t>(lane & 3);
    const uint32_t kb = (kw >> (8 * byte_sel)) & 0xFFu;
    const half2v kv = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(kb, 256.0f, 0)) *
                      scale_pair_same(st.ks[4 * (lane >> 3)]);
    kx = static_cast<float>(kv[0]);
    ky = static_cast<float>(kv[1]);
  } else {
    const uint32_t kb = *reinterpret_cast<const uint32_t*>(st.kc + 4 * lane);
    kx = bf16_to_f32(kb & 0xFFFFu);
    ky = bf16_to_f32(kb >> 16);
  }
  float sc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t hi = reinterpret_cast<const uint32_t*>(q_lds[i][0])[lane];
    const uint32_t lo = reinterpret_cast<const uint32_t*>(q_lds[i][1])[lane];
    float q0, q1;
    if constexpr (!KBF16) {
      const half2v h2 = as_half2(hi), l2 = as_half2(lo);
      q0 = static_cast<float>(h2[0]) + static_cast<float>(l2[0]);
      q1 = static_cast<float>(h2[1]) + static_cast<float>(l2[1]);
    } else {
      const uint32_t t2 = reinterpret_cast<const uint32_t*>(q_lds[i][2])[lane];
      q0 = (bf16_to_f32(hi & 0xFFFFu) + bf16_to_f32(lo & 0xFFFFu)) + bf16_to_f32(t2 & 0xFFFFu);
      q1 = (bf16_to_f32(hi >> 16) + bf16_to_f32(lo >> 16)) + bf16_to_f32(t2 >> 16);
    }
    float x = q0 * kx + q1 * ky;
    x = row16_sum(x);
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    sc[i] = (__uint_as_float(t[0]) + __uint_as_float(t[1])) * q_descale[i];
  }
  const float s = ln.g == 0 ? sc[0] : (ln.g == 1 ? sc[1] : (ln.g == 2 ? sc[2] : sc[3]));
  if (s > sm.m_ref + kLazyMax) {                   // per row of lanes, as in the iterations
    const float alpha = exp2f(sm.m_ref - s);
    sm.m_ref = s;
    sm.l_acc *= alpha;
#pragma unroll
    for (int v = 0; v < 8; ++v) sm.acc[v] *= alpha;
  }
  const float p = __builtin_amdgcn_exp2f(s - sm.m_ref);
  if (ln.c == 0) sm.l_acc += p;
  const uint32_t vw = *reinterpret_cast<const uint32_t*>(st.vc + 16 * ln.c);
  const half8 vv = dequant_dword(vw, scale_pair_same(st.vs[4 * (ln.c >> 1)]));
#pragma unroll
  for (int v = 0; v < 8; ++v) sm.acc[v][0] = __builtin_fmaf(p, static_cast<float>(vv[v]), sm.acc[v][0]);
}

// PIPE2: two register buffers and up to 8 wavefronts per workgroup (long splits, several
// iterations per wavefront); otherwise one buffer and few enough registers for 16
// wavefronts per workgroup (short splits, about one iteration per wavefront).
// APPEND: one extra wavefront per workgroup reads no cache.  In the workgroup whose split
// holds position seq_len - 1 it quantises the new token into its cache slot and an LDS stage
// once the query prologue is done and adds the token to its own softmax state; the cache
// wavefronts read the split without that position.
// KLT: compiled with the KLT key basis (basis staging and both rotations); the other
// instances carry none of that code.
// TRACE: the measurement instance, which also records the phase stamps above (and waits for
// its first cache data explicitly before the first iteration, to stamp its arrival).
template <bool KBF16, bool PIPE2, bool APPEND, bool KLT, bool TRACE = false>
__global__ void __launch_bounds__(PIPE2 ? 512 : 1024) k_decode(DecodeArgs a) {
  TraceStamps ts;
  if constexpr (TRACE) ts.entry = stamp_now();
  // Workgroups are dealt to the 8 dies (XCDs) round robin by linear id, so with several
  // splits the ids are remapped to give the splits of one (sequence, KV head) consecutive ids
  // within one die's share: their merge traffic then stays on one die where possible.  A
  // bijection for any grid; correctness does not depend on where workgroups run.
  int split, h, b;
  {
    const uint32_t n_split = gridDim.x, n_head = gridDim.y;
    const uint32_t total = n_split * n_head * gridDim.z;
    const uint32_t L = blockIdx.x + n_split * (blockIdx.y + n_head * blockIdx.z);
    const uint32_t q8 = total >> 3, r8 = total & 7u, x = L & 7u;
    const uint32_t G = n_split > 1 ? x * q8 + (x < r8 ? x : r8) + (L >> 3) : L;
    const uint32_t unit_g = G / n_split;
    split = static_cast<int>(G - unit_g * n_split);
    h = static_cast<int>(unit_g % n_head);
    b = static_cast<int>(unit_g / n_head);
  }
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

  __shared__ __attribute__((aligned(16))) uint16_t q_lds[4][4][kHeadDim];   // [head][term][dim]
  __shared__ __attribute__((aligned(16))) uint32_t p_lds[kMaxWaves][kPWords];
  __shared__ float q_descale[4];
  __shared__ float red_m[kMaxWaves][4], red_l[kMaxWaves][4];
  __shared__ __attribute__((aligned(16))) float red_o[kMaxWaves][4][kHeadDim];
  const int nw = static_cast<int>(blockDim.x) >> 6;
  const int nwc = APPEND ? nw - 1 : nw;                     // wavefronts that read the cache
  const bool app_wave = APPEND && wave == nw - 1;
  __shared__ int mrg_last;
  __shared__ __attribute__((aligned(16))) NewTokenStage nt_stage;

  const int64_t unit = static_cast<int64_t>(b) * a.hkv + h;
  const const_i32_ptr ptab = __builtin_bit_cast(const_i32_ptr, a.page_table) + static_cast<int64_t>(b) * a.max_pages_per_seq;

  // KLT key basis of this head into dynamic LDS (followed by a 128-float slot per query
  // wavefront for the rotation) by the four query wavefronts, a quarter each (below);
  // their loads go out before their cache loads, so waiting for them does not wait for the
  // cache, and the other wavefronts issue their cache loads at once
  extern __shared__ __attribute__((aligned(16))) float basis_dyn[];
  const bool klt = KLT && !KBF16 && (a.k_flags & NVKV_K_KLT);
  // ---- start every independent memory access first: query row, sequence length, pages ----
  const bool q_wave = wave < 4;                 // wavefronts 0..3 prepare query heads 4h..4h+3
  const int hq_w = 4 * h + (q_wave ? wave : 0);
  const uint32_t qw = reinterpret_cast<const uint32_t*>(a.q + (static_cast<int64_t>(b) * a.hq + hq_w) * kHeadDim)[lane];
  float2 sv = make_float2(1.0f, 1.0f);
  if (!KBF16 && (a.k_flags & NVKV_K_SMOOTH)) sv = reinterpret_cast<const float2*>(a.smooth + h * kHeadDim)[lane];
  const float gk = KBF16 ? 1.0f : a.gscale[0];
  const float gv = a.gscale[1];                // value tensor scale, applied to the output
  NewTokenRegs nreg;
  if (app_wave) new_token_load<KBF16>(a, b, h, lane, nreg);
  // the value is first needed after the loads of the first iterations have been issued
  const int seq_len_in = a.seq_lens[b];
  const int t_begin = split * a.split_tokens;
  // the basis quarter after the query row, so the query's latency hides under the basis copy
  if (klt && wave < 4) load_basis_quarter(a.basis + static_cast<int64_t>(h) * kBasisFloats, basis_dyn, wave, lane);
  if constexpr (TRACE) {
    if (klt) ts.basis = stamp_now();
  }

  // First two iterations of this wavefront: addresses and loads are issued before the
  // sequence length arrives, bounded by the kernel arguments only (t_lim >= t_end), so the
  // cache traffic overlaps the query prologue; tokens in [t_end, t_lim) are masked later.
  const int t_lim = min(t_begin + a.split_tokens, a.seq_cap);
  const int step = kIterTok * nwc;
  int t0 = app_wave ? INT_MAX / 2 : t_begin + kIterTok * wave;   // the append wavefront reads no cache
  IterLoads<KBF16> buf0, buf1;
  HalfBase hb0[2], hb1[2];
  if (t0 < t_lim) {
    half_bases<KBF16>(a, load_pages(a, ptab, t0, t_lim), h, hb0);
    issue_loads<KBF16>(hb0, ln, buf0);
  }
  if (PIPE2 && t0 + step < t_lim) {
    half_bases<KBF16>(a, load_pages(a, ptab, t0 + step, t_lim), h, hb1);
    issue_loads<KBF16>(hb1, ln, buf1);
  }
  IterPages pnext = load_pages(a, ptab, t0 + (PIPE2 ? 2 : 1) * step, t_lim > 0 ? t_lim : 1);

  const int seq_len = seq_len_in < 0 ? 0 : (seq_len_in > a.seq_cap ? a.seq_cap : seq_len_in);
  const int t_end = min(t_begin + a.split_tokens, seq_len);
  const bool empty = t_begin >= t_end;                      // uniform across the workgroup
  // APPEND: the new token is position t_new = seq_len - 1
  const int t_new = seq_len - 1;
  const bool owns_new = APPEND && !empty && t_new >= t_begin && t_new < t_begin + a.split_tokens;
  const int t_read = APPEND ? min(t_end, t_new) : t_end;  // the cache wavefronts skip t_new
  int32_t new_pg = 0;
  int new_off = 0;
  if (owns_new && app_wave) {
    if (a.page_shift >= 0) {
      new_pg = ptab[t_new >> a.page_shift];
      new_off = t_new & (a.page_size - 1);
    } else {
      new_pg = ptab[t_new / a.page_size];
      new_off = t_new % a.page_size;
    }
  }

  // ---------------- query prologue: wavefront w < 4 prepares query head 4h + w ----------------
  if (klt) __syncthreads();                    // the basis is in LDS
  if constexpr (TRACE) {
    if (klt) ts.basis_bar = stamp_now();
  }
  // the new token's key transform: with the KLT rotation the idle extra wavefront does it
  // during the query prologue, otherwise after it
  float ny[4];
  const bool nt_early = klt && owns_new && app_wave;
  if (nt_early) new_token_transform<KBF16>(a, lane, nreg, nt_stage, basis_dyn, ny);
  if (!empty && q_wave) {
    uint32_t w0, w1, w2;
    const float descale = query_terms<KBF16>(qw, sv, a.k_flags, a.sm_scale, gk, lane, w0, w1, w2, basis_dyn,
                                                  basis_dyn + kBasisFloats + (wave & 3) * kHeadDim);
    reinterpret_cast<uint32_t*>(q_lds[wave][0])[lane] = w0;
    reinterpret_cast<uint32_t*>(q_lds[wave][1])[lane] = w1;
    reinterpret_cast<uint32_t*>(q_lds[wave][2])[lane] = w2;
    reinterpret_cast<uint32_t*>(q_lds[wave][3])[lane] = 0u;
    if (lane == 0) q_descale[wave] = descale;
    if constexpr (TRACE) ts.query = stamp_now();
  }
  __syncthreads();
  if constexpr (TRACE) ts.prologue = stamp_now();

  SoftmaxState st;
  st.m_ref = -INFINITY;
  st.l_acc = 0.0f;
#pragma unroll
  for (int v = 0; v < 8; ++v) st.acc[v] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

  // The new token first, right after the query barrier: the extra wavefront needs none of the
  // cache wavefronts' set-up below, and its encode (with MSE-searched key scales, the search)
  // is what the split's partials wait for.
  if (owns_new && app_wave) {
    // the extra wavefront is the youngest on its SIMD: raised issue priority keeps it from
    // waiting behind the cache wavefronts there, whose workgroup merge waits for it
    __builtin_amdgcn_s_setprio(2);
    uint64_t nt_begin = 0, nt_encoded = 0;
    if constexpr (TRACE) nt_begin = stamp_now();
    const bool ok = static_cast<uint32_t>(new_pg) < static_cast<uint32_t>(a.num_pages);
    if (!nt_early) new_token_transform<KBF16>(a, lane, nreg, nt_stage, basis_dyn, ny);
    new_token_encode<KBF16>(a, h, lane, nreg, ny, new_pg, new_off, ok, nt_stage);
    if constexpr (TRACE) nt_encoded = stamp_now();
    if (ok) new_token_update<KBF16>(nt_stage, q_lds, q_descale, lane, ln, st);
    __builtin_amdgcn_s_setprio(0);
    if constexpr (TRACE) {
      // the new-token wavefront's own stamps, slots 13-15 of its workgroup's record
      const uint64_t nt_done = stamp_now();
      if (lane == 0) {
        uint64_t* r = a.trace + (blockIdx.x + static_cast<int64_t>(gridDim.x) *
                                                 (blockIdx.y + static_cast<int64_t>(gridDim.y) * blockIdx.z)) * kTraceSlots;
        r[13] = nt_begin;
        r[14] = nt_encoded;
        r[15] = nt_done;
      }
    }
  }

  if (!empty) {
    // A operand of QK (Q'): lane (c, g) = row c = (head c>>2, term c&3); instruction u, item
    // e <-> dim 32g + 8u + e (the same dim order as the key codes a lane loads).
    u32x4 qa[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      qa[u] = *reinterpret_cast<const u32x4*>(&q_lds[c >> 2][c & 3][32 * g + 8 * u]);
    const float descale = q_descale[g];        // the lane's scores belong to head g
    // P rows (head, term 2 or 3) stay zero
    uint32_t* p_w = p_lds[wave];
    for (int i = lane; i < kPWords; i += 64) p_w[i] = 0u;
    bool vm[2];

    // Software pipeline: two register buffers hold the next two iterations' cache data and
    // the page entries of the iteration after them are already loaded, so neither the
    // vector loads nor the page lookups sit on the critical path.
    if constexpr (TRACE) {
      if (t0 < t_read) {
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        ts.data = stamp_now();
      }
    }
    if constexpr (!PIPE2) {
      while (t0 < t_read) {
        valid_tokens(hb0, t0, t_read, c, vm);
        compute_iter<KBF16>(buf0, vm, qa, descale, ln, st, p_w);
        t0 += step;
        if (t0 >= t_read) break;
        half_bases<KBF16>(a, pnext, h, hb0);
        issue_loads<KBF16>(hb0, ln, buf0);
        pnext = load_pages(a, ptab, t0 + step, t_read);
      }
    }
    while (PIPE2 && t0 < t_read) {
      valid_tokens(hb0, t0, t_read, c, vm);
      compute_iter<KBF16>(buf0, vm, qa, descale, ln, st, p_w);
      t0 += step;
      if (t0 >= t_read) break;
      if (t0 + step < t_read) {
        half_bases<KBF16>(a, pnext, h, hb0);
        issue_loads<KBF16>(hb0, ln, buf0);
        pnext = load_pages(a, ptab, t0 + 2 * step, t_read);
      }
      valid_tokens(hb1, t0, t_read, c, vm);
      compute_iter<KBF16>(buf1, vm, qa, descale, ln, st, p_w);
      t0 += step;
      if (t0 + step < t_read) {
        half_bases<KBF16>(a, pnext, h, hb1);
        issue_loads<KBF16>(hb1, ln, buf1);
        pnext = load_pages(a, ptab, t0 + 2 * step, t_read);
      }
    }
    if constexpr (TRACE) ts.done = stamp_now();
  }

  // ---------------- wavefront partials -> LDS -> workgroup partial ----------------
  // Every wavefront publishes (m, l, o) per head; the slots of wavefronts that do not exist
  // are filled with empty entries (m = -inf, l = 0, o = 0) by the existing ones, so the owner
  // threads combine a fixed number of slots without selects, in a fixed order (the result is
  // the same on every run).  The combination is VALU work on the owner wavefronts only (one
  // per SIMD), so it is kept short: raw exp2 (exp2(-inf) = 0; weights lie in (0, 1]).
  {
    constexpr int kRed = PIPE2 ? 8 : kMaxWaves;
    const float l_tot = row16_sum(st.l_acc);
    if (c == 0) {
      red_m[wave][g] = st.m_ref;
      red_l[wave][g] = l_tot;
    }
    float4* dst = reinterpret_cast<float4*>(&red_o[wave][g][8 * c]);
    dst[0] = make_float4(st.acc[0][0] + st.acc[0][1], st.acc[1][0] + st.acc[1][1],
                         st.acc[2][0] + st.acc[2][1], st.acc[3][0] + st.acc[3][1]);
    dst[1] = make_float4(st.acc[4][0] + st.acc[4][1], st.acc[5][0] + st.acc[5][1],
                         st.acc[6][0] + st.acc[6][1], st.acc[7][0] + st.acc[7][1]);
    // empty entries in slots nw .. kRed-1: wavefront w fills slots nw + w, 2 nw + w, ...
    for (int zs = nw + wave; zs < kRed; zs += nw) {
      float4* z = reinterpret_cast<float4*>(&red_o[zs][g][8 * c]);
      z[0] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      z[1] = z[0];
      if (c == 0) {
        red_m[zs][g] = -INFINITY;
        red_l[zs][g] = 0.0f;
      }
    }
  }
  __syncthreads();
  if constexpr (TRACE) ts.lds_merge = stamp_now();

  // threads 0..255 own (head i, dims d0, d0+1) in the merges; the others only take part in
  // the barriers
  const bool owner = tid < 256;
  const int i = (tid >> 6) & 3;
  const int d0 = 2 * (tid & 63);
  float M = -INFINITY, Lw = 0.0f, o0 = 0.0f, o1 = 0.0f;
  if (owner) {
    constexpr int kRed = PIPE2 ? 8 : kMaxWaves;
    float mw[kRed], lw[kRed];
    float2 ow[kRed];
#pragma unroll
    for (int w = 0; w < kRed; ++w) {
      mw[w] = red_m[w][i];
      lw[w] = red_l[w][i];
      ow[w] = *reinterpret_cast<const float2*>(&red_o[w][i][d0]);
    }
#pragma unroll
    for (int w = 0; w < kRed; ++w) M = fmaxf(M, mw[w]);
    const float Mr = M == -INFINITY ? 0.0f : M;          // all empty: every weight is 0
#pragma unroll
    for (int w = 0; w < kRed; ++w) {
      const float wt = __builtin_amdgcn_exp2f(mw[w] - Mr);
      Lw = __builtin_fmaf(wt, lw[w], Lw);
      o0 = __builtin_fmaf(wt, ow[w].x, o0);
      o1 = __builtin_fmaf(wt, ow[w].y, o1);
    }
  }
  if (a.n_splits == 1) {
    if (owner) {
      const float f = Lw > 0.0f ? gv / Lw : 0.0f;
      float* out_row = a.out + (static_cast<int64_t>(b) * a.hq + 4 * h + i) * kHeadDim + d0;
      *reinterpret_cast<float2*>(out_row) = make_float2(o0 * f, o1 * f);
    }
    if constexpr (TRACE) {
      ts.ident = hw_identity() | 1u | (static_cast<uint64_t>(split) << 48);
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      ts.stored = stamp_now();
      trace_write(a, ts, wave, tid);
    }
    return;
  }
  // ---- cross-workgroup merge: the last workgroup of (b, h) to arrive combines the splits ----
  // Partials are written with device-coherent stores and read with device-coherent loads, so
  // no cache writeback or invalidate is needed (a device-scope fence would write back and
  // invalidate the whole L2 of the die).  Each wavefront waits until its stores have
  // completed before the workgroup barrier; only then does one thread count the arrival.
  //
  // Why this is ordered without release/acquire (all accesses involved are relaxed atomics at
  // agent scope, which the language model alone would not order across locations):
  //  1. The partial stores are agent-scope atomic stores: on gfx950 a store with sc1 set.  It
  //     is written through the die's L2 to the device coherence point, and its completion is
  //     reported only once it is performed there.
  //  2. s_waitcnt vmcnt(0) waits for every vector memory operation of the wavefront, stores
  //     included (gfx9-family parts count stores in vmcnt; there is no separate store counter).
  //     After it, this wavefront's partials are visible to any agent-scope load on any die.
  //  3. The workgroup barrier (with its workgroup-scope fences, which also stop the compiler
  //     from moving memory operations across it) puts every wavefront's wait before the
  //     arrival RMW of thread 0.  The RMW is an agent-scope atomic performed at the coherence
  //     point, so the arrivals of one (b, h) are totally ordered: the workgroup that reads
  //     n_splits - 1 arrived after every other workgroup's stores had completed.
  //  4. The merging workgroup's loads are issued after the barrier that publishes mrg_last, and
  //     are agent-scope atomic loads (sc1): they are served from the coherence point, not from
  //     a line its own die's L2 may hold from earlier, so they return the partials.
  //  5. The counter is reset by the merging workgroup; the next launch reads it after the
  //     kernel boundary, which orders all of this launch's memory operations before it.
  // What would break it: plain stores or loads for the partials (they stay in, or are served
  // from, one die's write-back L2); a part whose store completion does not mean device
  // visibility, or that counts stores separately from vmcnt; an RMW issued before the barrier
  // or from a wavefront that has not waited.  The portable form, a release RMW and an acquire
  // load, costs a write-back and invalidate of the whole L2 per workgroup.
  if constexpr (TRACE) ts.issue = stamp_now();
  if (owner) {
    const int64_t slot = (unit * a.n_splits + split) * 4 + i;
    store_coherent_f2(a.ws_o + slot * kHeadDim + d0, o0, o1);
    if ((tid & 63) == 0) store_coherent_f2(a.ws_ml + slot * 2, M, Lw);
  }
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  if constexpr (TRACE) ts.acked = stamp_now();
  if (tid == 0) {
    const unsigned prev =
        __hip_atomic_fetch_add(a.counters + unit * kCounterStride, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    mrg_last = (prev == static_cast<unsigned>(a.n_splits - 1)) ? 1 : 0;
    if constexpr (TRACE) ts.counted = stamp_now();
  }
  __syncthreads();
  if (!mrg_last || !owner) {
    if constexpr (TRACE) {
      ts.ident = hw_identity() | (mrg_last ? 1u : 0u) | (static_cast<uint64_t>(split) << 48);
      trace_write(a, ts, wave, tid);
    }
    return;
  }
  // groups of 8 splits when that covers them all (16-entry groups would be half padding)
  if (a.n_splits <= 8)
    merge_splits<8, TRACE>(a, unit, i, d0, gv, &ts.loaded);
  else
    merge_splits<16, TRACE>(a, unit, i, d0, gv, &ts.loaded);
  if constexpr (TRACE) ts.folded = stamp_now();
  if (tid == 0) __hip_atomic_store(a.counters + unit * kCounterStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if constexpr (TRACE) {
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    ts.stored = stamp_now();
    ts.ident = hw_identity() | 1u | (static_cast<uint64_t>(split) << 48);
    trace_write(a, ts, wave, tid);
  }
}

// ---------------------------------------------------------------------------------------
// Split plan and launcher
// ---------------------------------------------------------------------------------------
DecodePlan plan_decode(int32_t B, int32_t Hkv, int32_t max_seq_len, int32_t split_tokens, bool append) {
  DecodePlan p{};
  p.append = append;
  const int32_t len = max_seq_len > 0 ? max_seq_len : 1;
  const int64_t iters = (len + kIterTok - 1) / kIterTok;          // 32-token iterations
  int64_t per;                                                    // iterations per split
  if (split_tokens <= 0) {
    // About one workgroup per CU (256): splits per (sequence, KV head) = 256 / units, at
    // least one; the wavefronts of a workgroup take one iteration each when that fits in 16
    // wavefronts, otherwise 8 wavefronts share the split's iterations.
    const int64_t units = static_cast<int64_t>(B) * Hkv;
    int64_t ns = (256 + units / 2) / units;
    if (ns < 1) ns = 1;
    if (ns > iters) ns = iters;
    per = (iters + ns - 1) / ns;
  } else {
    per = split_tokens / kIterTok;
  }
  // the merge of a sequence visits splits in groups; bound their number
  const int64_t min_per = (iters + kMaxSplits - 1) / kMaxSplits;
  if (per < min_per) per = min_per;
  if (per < 1) per = 1;
  p.split_tokens = static_cast<int32_t>(per * kIterTok);
  p.n_splits = static_cast<int32_t>((len + p.split_tokens - 1) / p.split_tokens);
  // the fused append adds one wavefront (the append wavefront) to every workgroup
  const int64_t max_cache_waves = append ? kMaxWaves - 1 : kMaxWaves;
  if (per <= max_cache_waves) {
    p.pipe2 = false;
    p.waves = static_cast<int32_t>((per < 4 ? 4 : per) + (append ? 1 : 0));
  } else {
    p.pipe2 = true;
    p.waves = 8;                 // with the append wavefront: 7 cache wavefronts + 1
  }
  return p;
}

namespace {
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
size_t counter_bytes(int32_t B, int32_t Hkv) {
  return align256(static_cast<size_t>(B) * Hkv * kCounterStride * sizeof(unsigned));
}
size_t ml_bytes(int32_t B, int32_t Hkv, const DecodePlan& plan) {
  return align256(static_cast<size_t>(B) * Hkv * plan.n_splits * 4 * 2 * sizeof(float));
}
}  // namespace

// Workspace layout: [arrival counters: B*Hkv, 256 bytes apart][(m, l) per split and head]
// [O per split and head].  The counters come first so that their place does not depend on the split
// count: calls with different split counts may share a workspace.
size_t decode_partial_bytes(int32_t B, int32_t Hkv, const DecodePlan& plan) {
  if (plan.n_splits <= 1) return 0;
  const size_t slots = static_cast<size_t>(B) * Hkv * plan.n_splits * 4;
  return ml_bytes(B, Hkv, plan) + align256(slots * kHeadDim * sizeof(float));
}

size_t decode_workspace_bytes(int32_t B, int32_t Hkv, const DecodePlan& plan) {
  return counter_bytes(B, Hkv) + decode_partial_bytes(B, Hkv, plan);
}

DecodeWs carve_decode_workspace(void* workspace, int32_t B, int32_t Hkv, const DecodePlan& plan) {
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  DecodeWs w;
  w.counters = reinterpret_cast<unsigned*>(ws);
  w.ml = reinterpret_cast<float*>(ws + counter_bytes(B, Hkv));
  w.o = reinterpret_cast<float*>(ws + counter_bytes(B, Hkv) + ml_bytes(B, Hkv, plan));
  return w;
}

// ---------------------------------------------------------------------------------------
// Static scratch of the allocation-free entry point (for callers that cannot allocate).
// One array per GPU (each device that loads the library holds its own copy until the process
// ends).  Layout: [arrival counters: kScratchUnits, 256 bytes apart][partials].  The counter
// region has a fixed size, so partials of one call never land on counters of another.  Every
// call on a device shares its array: calls that overlap on one GPU race.
// ---------------------------------------------------------------------------------------
constexpr size_t kScratchCounterBytes = kScratchUnits * kCounterStride * sizeof(unsigned);
static __device__ __attribute__((aligned(256))) uint8_t scratch[kScratchCounterBytes + kScratchPartialBytes];

__global__ void k_clear_words(uint32_t* p, uint32_t n) {
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

namespace {
std::mutex g_scratch_mu;
std::unordered_map<int, uint8_t*> g_scratch_addr;   // device -> device address of `scratch`
}  // namespace

hipError_t scratch_decode_workspace(int32_t B, int32_t Hkv, const DecodePlan& plan, hipStream_t stream,
                                    DecodeWs* ws) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  uint8_t* base = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    auto it = g_scratch_addr.find(dev);
    if (it != g_scratch_addr.end()) {
      base = it->second;
    } else {
      // the array's name is a host-side stand-in: its device address comes from the runtime,
      // once per device, with that device current
      void* ptr = nullptr;
      e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      base = static_cast<uint8_t*>(ptr);
      // the counters must start at zero (every completed call leaves them at zero); cleared by a
      // kernel on the caller's stream, which a graph capture may record
      const uint32_t words = static_cast<uint32_t>(kScratchCounterBytes / sizeof(uint32_t));
      hipLaunchKernelGGL(k_clear_words, dim3(64), dim3(256), 0, stream, reinterpret_cast<uint32_t*>(base), words);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      g_scratch_addr.emplace(dev, base);
    }
  }
  ws->counters = reinterpret_cast<unsigned*>(base);
  ws->ml = reinterpret_cast<float*>(base + kScratchCounterBytes);
  ws->o = reinterpret_cast<float*>(base + kScratchCounterBytes + ml_bytes(B, Hkv, plan));
  return hipSuccess;
}

hipError_t launch_decode(const nvkv_layer& L, const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                         int32_t B, int32_t Hq, const int32_t* page_table, int32_t max_pages_per_seq,
                         const int32_t* seq_lens, int32_t max_seq_len, float sm_scale, float* out,
                         const DecodeWs& ws, const DecodePlan& plan, hipStream_t stream, uint64_t* trace) {
  DecodeArgs a{};
  a.k_new = k_new;
  a.v_new = v_new;
  a.inv_smooth = L.k_inv_smooth;
  a.k_codes_w = static_cast<uint8_t*>(L.k_data);
  a.k_scales_w = L.k_scales;
  a.v_codes_w = static_cast<uint8_t*>(L.v_data);
  a.v_scales_w = L.v_scales;
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
  a.counters = ws.counters;
  a.ws_ml = ws.ml;
  a.ws_o = ws.o;
  a.hkv = L.num_kv_heads;
  a.hq = Hq;
  a.page_size = L.page_size;
  a.page_shift = (L.page_size & (L.page_size - 1)) == 0 ? __builtin_ctz(static_cast<unsigned>(L.page_size)) : -1;
  a.num_pages = L.num_pages;
  a.max_pages_per_seq = max_pages_per_seq;
  const int64_t cap_pages = static_cast<int64_t>(max_pages_per_seq) * L.page_size;
  a.seq_cap = static_cast<int32_t>(cap_pages < max_seq_len ? cap_pages : max_seq_len);
  a.split_tokens = plan.split_tokens;
  a.n_splits = plan.n_splits;
  a.k_flags = L.k_flags;
  a.sm_scale = sm_scale;
  a.basis = L.k_basis;
  a.trace = trace;
  const dim3 grid(plan.n_splits, L.num_kv_heads, B);
  const dim3 block(64 * plan.waves);
  const bool bf = L.k_fmt == NVKV_FMT_BF16;
  using Kernel = void (*)(DecodeArgs);
  const bool klt = !bf && (L.k_flags & NVKV_K_KLT);
  Kernel kern;
  if (trace) {
    // the measurement instances: NVFP4 keys; with the KLT basis the fused short-split form only
    if (bf || (klt && (!plan.append || plan.pipe2))) return hipErrorNotSupported;
    if (klt) kern = k_decode<false, false, true, true, true>;
    else if (plan.append) kern = plan.pipe2 ? k_decode<false, true, true, false, true> : k_decode<false, false, true, false, true>;
    else kern = plan.pipe2 ? k_decode<false, true, false, false, true> : k_decode<false, false, false, false, true>;
  } else if (klt) {
    if (plan.append) kern = plan.pipe2 ? k_decode<false, true, true, true> : k_decode<false, false, true, true>;
    else kern = plan.pipe2 ? k_decode<false, true, false, true> : k_decode<false, false, false, true>;
  } else if (plan.append) {
    kern = bf ? (plan.pipe2 ? k_decode<true, true, true, false> : k_decode<true, false, true, false>)
              : (plan.pipe2 ? k_decode<false, true, true, false> : k_decode<false, false, true, false>);
  } else {
    kern = bf ? (plan.pipe2 ? k_decode<true, true, false, false> : k_decode<true, false, false, false>)
              : (plan.pipe2 ? k_decode<false, true, false, false> : k_decode<false, false, false, false>);
  }
  // the KLT key basis of the workgroup's head is staged in dynamic LDS
  const size_t dyn_lds = klt ? (kBasisFloats + 4 * kHeadDim) * sizeof(float) : 0;
  if (dyn_lds) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(dyn_lds));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, grid, block, dyn_lds, stream, a);
  return hipGetLastError();
}

}  // namespace nvkv
