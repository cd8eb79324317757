/*
 * nvfp4kv.h -- C ABI of the NVFP4 attention-KV-cache library for AMD MI355X (gfx950).
 *
 * The operations (sources named by page title and section):
 *   [cache post] rstation.ai post "NVFP4 attention cache on W4A4 Qwen3-8B: static key
 *                smoothing is near-lossless, key rotations hurt": post-RoPE cached keys and
 *                values quantised to NVFP4 in 16-element blocks along head_dim (opening
 *                paragraph); static per-channel key smoothing sqrt(absmax) from 4 calibration
 *                windows with position 0 excluded, optional Hadamard-128 key basis
 *                (cache-config table); attention runs over the quantised cache.
 *   [OSFP4]      paperlayer.ai summary of arXiv 2610.08231v1 "OSFP4: Joint Optimization of
 *                Diagonal Smoothing and Block Scales for NVFP4 Quantization": E2M1 values,
 *                E4M3 scale per 16 entries, FP32 tensor scale (appendix D.1); block scale
 *                set so the block absmax maps to 6 (section 1); a static calibration-based
 *                global scale for online quantisation (section 3).
 *   [QServe rec] inference-research record "QServe SmoothAttention (4-bit KV cache ...)":
 *                smoothing keys by a per-channel factor and folding it into the query.
 *
 * Numerics (fixed here where the pages leave them open):
 *   block scale S_b = E4M3FN round-to-nearest-even of the exact A_b/(6 g), saturating at 448;
 *   element code  = E2M1 round-to-nearest-even (ties to the even code) of the exact
 *                   |y|/(sigma_b g), saturating at 6; a zero magnitude is stored as code 0;
 *   g = amax/2688 from calibration (1 when amax = 0); keys are multiplied by r = fl32(1/s)
 *   before quantisation, queries by s; the Hadamard key basis is the unnormalised Sylvester
 *   butterfly in fp32, stages h = 1,2,..,64, applied after smoothing; the query side carries
 *   the exact 1/128.  V is never transformed.
 *
 * Conventions for every entry point:
 *   - All buffers are DEVICE memory owned by the caller.  The library allocates nothing,
 *     keeps no mutable global state except a thread-local last-error string, never
 *     synchronises, and enqueues its kernels on `stream` (a hipStream_t passed as void*;
 *     NULL = the legacy default stream).
 *   - Argument errors are detected on the host and returned BEFORE any HIP call, so they can
 *     be exercised on a machine without a GPU.  HIP failures return NVKV_ERR_HIP; the text is
 *     in nvkv_last_error().
 *   - Device-side data the host cannot see (slot numbers, page-table entries, sequence
 *     lengths) is range-checked by the kernels: out-of-range rows are skipped, never written.
 *   - head_dim is fixed at 128.  Non-finite K/V/Q inputs give unspecified results.
 *
 * Cache layout of one layer (page_size tokens per page, multiple of 16; a contiguous cache is
 * num_pages = batch with one page of max-context tokens per sequence):
 *   NVFP4 codes   64 bytes per (token, head): byte k = element 2k in the low nibble |
 *                 element 2k+1 in the high nibble; nibble = sign<<3 | E2M1 magnitude code.
 *                 Word w (4 bytes, elements 8w..8w+7) of token t of a page:
 *                   keys   u8 [num_pages][Hkv][page_size][64]: byte 64t + 4w of the
 *                          (page, head) block (row-major);
 *                   values u8 [num_pages][Hkv][page_size/4][16][4][4]: byte
 *                          ((t/4)*16 + w)*16 + (t%4)*4 of the block (quad-interleaved: the
 *                          four tokens of a quad side by side per word, so a decode lane
 *                          reads one word of four tokens with one 16-byte load).
 *   NVFP4 scales  u8  [num_pages][Hkv][page_size/4][8][4] (K and V alike)
 *                 the E4M3FN scale of block b (elements 16b..16b+15) of token t of a page is
 *                 byte ((t/4)*8 + b)*4 + t%4 of that (page, head).
 *   BF16 rows     u16 [num_pages][Hkv][page_size][128]   (keys only)
 */
#ifndef NVFP4KV_H
#define NVFP4KV_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define NVKV_API __attribute__((visibility("default")))
#else
#define NVKV_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum nvkv_status {
  NVKV_OK = 0,
  NVKV_ERR_NULL = 1,        /* a required pointer is NULL                                  */
  NVKV_ERR_SHAPE = 2,       /* a count or size is out of range (<= 0, head_dim != 128, ...) */
  NVKV_ERR_UNSUPPORTED = 3, /* a valid but unimplemented combination of formats/flags      */
  NVKV_ERR_WORKSPACE = 4,   /* workspace missing, too small or not 256-byte aligned        */
  NVKV_ERR_HIP = 5          /* a HIP runtime call failed (see nvkv_last_error)             */
} nvkv_status;

enum { NVKV_FMT_BF16 = 0, NVKV_FMT_NVFP4 = 1 };
/* Key options.  NVKV_K_SMOOTH: static per-channel smoothing ([cache post] cache-config table;
 * [QServe rec] SmoothAttention).  NVKV_K_HADAMARD: Hadamard-128 basis on head_dim ([cache post]
 * table).  NVKV_K_MSE_SCALE: each key block's E4M3 scale is searched for the smallest squared
 * FP4 error instead of mapping the block maximum to 6 ([OSFP4] sections 1 and 3, appendices C
 * and H; candidates are the absmax-to-6 code and every code that puts the block maximum
 * between 7/4 and 7 scale units, the flat interval of section 2.1 and appendix A; ties keep
 * the absmax-to-6 code, then the smaller code).  It changes only how keys are encoded: the
 * cache format, the calibration (g_K) and the attention calls are unchanged. */
enum { NVKV_K_SMOOTH = 1u, NVKV_K_HADAMARD = 2u, NVKV_K_MSE_SCALE = 4u, NVKV_K_KLT = 8u };
/* NVKV_K_KLT: static per-head KLT key basis ([cache post] cache-config table rows "K: static
 * per-head KLT" and "K: static KLT + smoothing"): keys are rotated z = B^T y after the optional
 * smoothing, queries q' = B^T (q * s), with B = layer->k_basis from nvkv_calibrate_key_basis.
 * Each z_i is the chain of fp32 fused multiply-adds z <- fl32(B[j][i] * y_j + z) over
 * j = 0..127 from z = 0 (one rounding per step), so codes are reproducible bit for bit.
 * Not combined with NVKV_K_HADAMARD. */
enum { NVKV_PART_CODES = 0, NVKV_PART_SCALES = 1 };

#define NVKV_HEAD_DIM 128
#define NVKV_TENSOR_SCALE_DIVISOR 2688.0f /* 6 * 448: calibrated amax maps to 6 * E4M3 max */

/* One layer of cache plus its static calibration state.  Pointers are device memory. */
typedef struct nvkv_layer {
  int32_t num_kv_heads;       /* Hkv >= 1                                                  */
  int32_t head_dim;           /* must be 128                                               */
  int32_t page_size;          /* tokens per page, a positive multiple of 16                */
  int32_t num_pages;          /* pages in k_data / v_data                                  */
  int32_t k_fmt;              /* NVKV_FMT_NVFP4 or NVKV_FMT_BF16                           */
  int32_t v_fmt;              /* NVKV_FMT_NVFP4                                            */
  uint32_t k_flags;           /* NVKV_K_SMOOTH | NVKV_K_HADAMARD | NVKV_K_MSE_SCALE | NVKV_K_KLT
                                 (not HADAMARD with KLT); 0 for BF16 keys                  */
  int32_t reserved;           /* must be 0                                                 */
  void *k_data;               /* NVFP4 codes or BF16 rows, layout above                    */
  void *v_data;               /* NVFP4 codes                                               */
  uint8_t *k_scales;          /* NVFP4 scales (NULL for BF16 keys)                         */
  uint8_t *v_scales;          /* NVFP4 scales                                              */
  const float *k_smooth;      /* s [Hkv][128]: query side; required when NVKV_K_SMOOTH     */
  const float *k_inv_smooth;  /* r [Hkv][128] = fl32(1/s): key side; required with SMOOTH  */
  const float *global_scale;  /* [2] = {g_K, g_V}; g_K unused for BF16 keys                */
  const float *k_basis;       /* B [Hkv][128][128] fp32, element (j, i) of head h at
                                 (h*128 + j)*128 + i, column i = basis vector i; required
                                 with NVKV_K_KLT, ignored otherwise                        */
} nvkv_layer;

/*
 * Static calibration ([cache post] cache-config table, smoothing rows; [OSFP4] section 3).
 *   k_win, v_win: bf16 [W][T][Hkv][128] calibration windows (either may be NULL, not both).
 *   From k_win:  s[h][j] = fl32(sqrt(a)), a = max |k| over all windows and positions t >= 1
 *                (t >= 0 when exclude_pos0 == 0); s = 1 where a = 0.  r = fl32(1/s).
 *                g_out[0] = fl32(A_K / 2688), A_K = max |y| over every window, position
 *                (including 0) and head of the keys transformed as selected by k_flags
 *                (smoothing by r, then the Hadamard butterfly); 1 when A_K = 0.
 *                NVKV_K_MSE_SCALE in k_flags is accepted and does not change the result.
 *                With NVKV_K_KLT in k_flags, g_out[0] is not written: the basis comes first
 *                (nvkv_calibrate_key_basis, which then writes g_K).
 *   From v_win:  g_out[1] = fl32(A_V / 2688), A_V = max |v|; 1 when A_V = 0.
 *   s_out, r_out: fp32 [Hkv][128] (needed when k_win != NULL); g_out: fp32 [2].  Entries whose
 *   input is NULL are left untouched.  s_out and g_out double as the reduction buffers, so
 *   they must not alias the inputs.  W >= 1, T >= 1, Hkv >= 1.
 */
NVKV_API nvkv_status nvkv_calibrate_key_smoothing(const uint16_t *k_win, const uint16_t *v_win,
                                         int32_t W, int32_t T, int32_t Hkv,
                                         int32_t exclude_pos0, uint32_t k_flags,
                                         float *s_out, float *r_out, float *g_out,
                                         void *stream);

/*
 * Static per-head KLT key basis and its tensor scale ([cache post] cache-config table rows
 * "K: static per-head KLT" and "K: static KLT + smoothing").  Run after
 * nvkv_calibrate_key_smoothing on the same windows.
 *   k_win:     bf16 [W][T][Hkv][128] calibration windows.
 *   r:         fp32 [Hkv][128] key smoothing factors (1/s); used when k_flags has
 *              NVKV_K_SMOOTH (the basis is then computed from the smoothed keys), else ignored.
 *   k_flags:   must contain NVKV_K_KLT and not NVKV_K_HADAMARD.
 *   basis_out: fp32 [Hkv][128][128], layout of nvkv_layer.k_basis.  Column i of head h is the
 *              eigenvector of the i-th largest eigenvalue of the covariance (mean removed) of
 *              head h's keys over all windows and positions t >= 1 (t >= 0 when exclude_pos0
 *              == 0), computed in fp64 (cyclic Jacobi), signed so that its largest-magnitude
 *              entry is positive (entries within a relative 1e-6 of the largest count as ties;
 *              the first decides), rounded to fp32.
 *   g_out:     fp32 [2]; g_out[0] = fl32(A_K / 2688), A_K = max |z| over every window,
 *              position and head of the keys smoothed and rotated by basis_out (1 when A_K = 0).
 *              g_out[1] is not touched.
 *   workspace: device scratch of nvkv_calibrate_key_basis_workspace_bytes(Hkv) bytes,
 *              256-byte aligned; no initial contents needed.
 * W >= 1, T >= 2, Hkv >= 1.  Errors: NVKV_ERR_NULL, NVKV_ERR_SHAPE, NVKV_ERR_UNSUPPORTED
 * (flags), NVKV_ERR_WORKSPACE, NVKV_ERR_HIP.
 */
NVKV_API size_t nvkv_calibrate_key_basis_workspace_bytes(int32_t Hkv);
NVKV_API nvkv_status nvkv_calibrate_key_basis(const uint16_t *k_win, int32_t W, int32_t T, int32_t Hkv,
                                     int32_t exclude_pos0, uint32_t k_flags, const float *r,
                                     float *basis_out, float *g_out,
                                     void *workspace, size_t workspace_bytes, void *stream);

/*
 * Quantise-and-append ([cache post] opening paragraph and table; [OSFP4] sections 1, 3 and
 * appendix D.1).  k_new, v_new: bf16 [N][Hkv][128] post-RoPE rows of N new tokens.
 * slot_mapping: int32 [N], device; slot = page * page_size + offset.  Rows whose slot is
 * negative or >= num_pages * page_size are skipped.  Keys are transformed per
 * layer->k_flags (NVFP4 keys) and encoded with g_K; values with g_V; BF16 keys are copied.
 * Each written row replaces the previous contents of its slot.  N >= 0 (N = 0 is a no-op).
 */
NVKV_API nvkv_status nvkv_quantize_append_kv(const nvkv_layer *layer,
                                    const uint16_t *k_new, const uint16_t *v_new,
                                    const int32_t *slot_mapping, int32_t N, void *stream);

/*
 * Workspace needed by nvkv_decode_attention_nvfp4 (and by
 * nvkv_decode_append_attention_nvfp4) for the same (B, Hq, Hkv, max_seq_len,
 * split_tokens).  split_tokens = 0 selects the library's own split size; otherwise it must
 * be a positive multiple of 32 (tokens handled by one workgroup).  Returns 0 for invalid arguments.
 */
NVKV_API size_t nvkv_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t max_seq_len,
                                   int32_t split_tokens);

/*
 * Fused GQA decode attention over the packed cache ([cache post]: attention over the
 * quantised post-RoPE cache; [QServe rec]: the smoothing factor folded into the query).
 *   q:          bf16 [B][Hq][128], post-RoPE, untransformed (the library applies q*s and
 *               the 1/128-normalised Hadamard as layer->k_flags select).
 *   page_table: int32 [B][max_pages_per_seq], device; token t of sequence b lives in page
 *               page_table[b][t / page_size] at offset t % page_size.
 *   seq_lens:   int32 [B], device; tokens already in the cache (the current token is
 *               appended before this call).  Attention covers tokens [0, seq_lens[b]) with
 *               no mask; seq_lens[b] = 0 gives a zero output row.  Lengths above
 *               min(max_seq_len, max_pages_per_seq * page_size) are clamped to it.
 *   Query head hq reads KV head hq / (Hq / Hkv); Hq must be 4 * Hkv.
 *   out:        fp32 [B][Hq][128] = softmax(sm_scale * q' . k_hat) v_hat.
 *   workspace:  device scratch of at least nvkv_decode_workspace_bytes(...) bytes, 256-byte
 *               aligned (NULL allowed when that size is 0).  Its first 256*B*Hkv bytes hold
 *               one arrival counter per (sequence, KV head), 256 bytes apart; the rest holds
 *               the per-split partials.  Zero-fill it before its first use (and again if a
 *               later call has a larger B*Hkv); every completed
 *               call leaves the counters at zero, so the workspace can be reused by calls with
 *               other split counts or lengths without clearing.  Calls that may run
 *               concurrently must not share a workspace.
 */
NVKV_API nvkv_status nvkv_decode_attention_nvfp4(const nvkv_layer *layer,
                                        const uint16_t *q, int32_t B, int32_t Hq,
                                        const int32_t *page_table, int32_t max_pages_per_seq,
                                        const int32_t *seq_lens, int32_t max_seq_len,
                                        float sm_scale, float *out,
                                        void *workspace, size_t workspace_bytes,
                                        int32_t split_tokens, void *stream);

/*
 * One decode step with the new token appended in the same launch: exactly the effect of
 * nvkv_quantize_append_kv of k_new/v_new at position n-1, followed by
 * nvkv_decode_attention_nvfp4 over [0, n), where n = min(seq_lens[b], max_seq_len,
 * max_pages_per_seq * page_size) is the length INCLUDING the new token.  The quantisation
 * is the one of nvkv_quantize_append_kv ([cache post] opening paragraph and cache-config
 * table; [OSFP4] sections 1 and 3), the attention the one of nvkv_decode_attention_nvfp4.
 *   k_new, v_new: bf16 [B][Hkv][128], device: the new token's post-RoPE key and value.
 *   The slot is taken from the page table (page page_table[b][(n-1) / page_size], offset
 *   (n-1) % page_size); an out-of-range page index writes nothing and leaves the new token
 *   out of the attention, as the two separate calls would.  Sequences with n = 0 append
 *   nothing and get a zero output row.
 *   Other arguments, the workspace rules and the output are those of
 *   nvkv_decode_attention_nvfp4 (same nvkv_decode_workspace_bytes).  The workgroup that
 *   owns position n-1 encodes the row while the others stream the cache, which saves the
 *   separate append launch of a decode step.
 */
NVKV_API nvkv_status nvkv_decode_append_attention_nvfp4(const nvkv_layer *layer,
                                        const uint16_t *q, const uint16_t *k_new,
                                        const uint16_t *v_new, int32_t B, int32_t Hq,
                                        const int32_t *page_table, int32_t max_pages_per_seq,
                                        const int32_t *seq_lens, int32_t max_seq_len,
                                        float sm_scale, float *out,
                                        void *workspace, size_t workspace_bytes,
                                        int32_t split_tokens, void *stream);

/*
 * Allocation-free form of nvkv_decode_append_attention_nvfp4, for callers that cannot
 * allocate device memory or pass a workspace (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  Same arguments, semantics and output, minus the
 * workspace: the cross-split state (arrival counters and split partials) lives in a static
 * device array of the library, 512 KiB of counters + 7 MiB of partials, one per GPU, held
 * until the process ends.  Nothing is allocated, by the library or by any routine it calls.
 *   Limits: B * Hkv <= 2048, and the split partials of the call (8 + 512 bytes per (split,
 *   query head), each array rounded up to 256 bytes) within 7 MiB: about 14,000 (split, query
 *   head) pairs.  A call beyond them returns
 *   NVKV_ERR_WORKSPACE before any HIP call.  Calls with one split per sequence use no scratch.
 *   The first call on a device looks up the array's device address and clears its counters
 *   with a kernel on `stream`; every completed call leaves them at zero again.
 *   Every call on a GPU shares that GPU's array, which keeps the last call's contents: calls
 *   that may overlap on one GPU (other streams, other threads) race and must be serialised by
 *   the caller.
 */
NVKV_API nvkv_status nvkv_decode_append_attention_nvfp4_noalloc(const nvkv_layer *layer,
                                        const uint16_t *q, const uint16_t *k_new,
                                        const uint16_t *v_new, int32_t B, int32_t Hq,
                                        const int32_t *page_table, int32_t max_pages_per_seq,
                                        const int32_t *seq_lens, int32_t max_seq_len,
                                        float sm_scale, float *out,
                                        int32_t split_tokens, void *stream);

/*
 * Causal multi-query attention over the packed cache: the last Tq positions of each sequence
 * attend to the cached keys up to and including their own position ([cache post] opening
 * paragraph: models are scored teacher-forced over full windows while attention reads the
 * quantised post-RoPE cache; the same call serves a prefill chunk whose keys and values were
 * appended with nvkv_quantize_append_kv just before).
 *   q:          bf16 [B][Tq][Hq][128], post-RoPE, untransformed (the library applies q*s and
 *               the 1/128-normalised Hadamard as layer->k_flags select, as in decode).
 *   seq_lens:   int32 [B], device; n_b = tokens in the cache INCLUDING the Tq query positions,
 *               clamped to min(max_seq_len, max_pages_per_seq * page_size).  Query i of
 *               sequence b sits at position p = n_b - Tq + i and attends to tokens [0, p];
 *               rows with p < 0 (a sequence shorter than Tq) are zero.
 *   page_table: as for decode.  Hq must be 4 * Hkv.
 *   out:        fp32 [B][Tq][Hq][128] = softmax(sm_scale * q' . k_hat, causal) v_hat.
 *   No workspace: the split of a tile's keys over its workgroup is merged in LDS.
 *   Tq = 0 returns NVKV_OK without a launch.  Errors as for decode (NVKV_ERR_NULL,
 *   NVKV_ERR_SHAPE, NVKV_ERR_UNSUPPORTED for Hq != 4 Hkv, NVKV_ERR_HIP for a failed launch).
 */
NVKV_API nvkv_status nvkv_prefill_attention_nvfp4(const nvkv_layer *layer,
                                        const uint16_t *q, int32_t B, int32_t Tq, int32_t Hq,
                                        const int32_t *page_table, int32_t max_pages_per_seq,
                                        const int32_t *seq_lens, int32_t max_seq_len,
                                        float sm_scale, float *out, void *stream);

/* Bytes of one cache array of one layer: fmt NVKV_FMT_*, part NVKV_PART_*; 0 if invalid
 * (including a BF16 scales array, which does not exist). */
NVKV_API size_t nvkv_cache_array_bytes(int32_t fmt, int32_t part, int32_t num_pages, int32_t Hkv,
                              int32_t page_size);

/* Bytes per cached token across `layers` layers ([cache post] closing paragraph gives the
 * BF16 figure 144 KiB/token for 36 layers x 8 KV heads x 128). */
NVKV_API size_t nvkv_cache_bytes_per_token(int32_t k_fmt, int32_t v_fmt, int32_t Hkv, int32_t layers);

NVKV_API const char *nvkv_status_string(nvkv_status status);
NVKV_API const char *nvkv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4KV_H */
