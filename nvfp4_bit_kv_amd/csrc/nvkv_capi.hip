// C ABI entry points: argument validation on the host (before any HIP call), kernel launch,
// error reporting.  The operations themselves are documented in include/nvfp4kv.h.
#include <cmath>
#include <string>

#include "nvkv_internal.hpp"

namespace {

thread_local std::string g_last_error;

nvkv_status fail(nvkv_status st, const char* what) {
  g_last_error = what;
  return st;
}

nvkv_status hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) {
    g_last_error.clear();
    return NVKV_OK;
  }
  g_last_error = std::string(where) + ": " + hipGetErrorString(e);
  return NVKV_ERR_HIP;
}

constexpr int kMaxGridYZ = 65535;

nvkv_status check_layer(const nvkv_layer* L) {
  if (!L) return fail(NVKV_ERR_NULL, "layer is NULL");
  if (L->head_dim != NVKV_HEAD_DIM) return fail(NVKV_ERR_SHAPE, "head_dim must be 128");
  if (L->num_kv_heads < 1 || L->num_kv_heads > kMaxGridYZ) return fail(NVKV_ERR_SHAPE, "num_kv_heads out of range");
  if (L->page_size < 16 || L->page_size % 16 != 0) return fail(NVKV_ERR_SHAPE, "page_size must be a positive multiple of 16");
  if (L->num_pages < 1) return fail(NVKV_ERR_SHAPE, "num_pages must be >= 1");
  if (L->reserved != 0) return fail(NVKV_ERR_SHAPE, "reserved field must be 0");
  if (static_cast<int64_t>(L->num_pages) * L->page_size > INT32_MAX) return fail(NVKV_ERR_SHAPE, "num_pages * page_size exceeds int32");
  if (L->k_fmt != NVKV_FMT_NVFP4 && L->k_fmt != NVKV_FMT_BF16) return fail(NVKV_ERR_UNSUPPORTED, "unknown k_fmt");
  if (L->v_fmt != NVKV_FMT_NVFP4) return fail(NVKV_ERR_UNSUPPORTED, "v_fmt must be NVKV_FMT_NVFP4");
  if (L->k_flags & ~(NVKV_K_SMOOTH | NVKV_K_HADAMARD | NVKV_K_MSE_SCALE | NVKV_K_KLT))
    return fail(NVKV_ERR_UNSUPPORTED, "unknown k_flags bits");
  if ((L->k_flags & NVKV_K_HADAMARD) && (L->k_flags & NVKV_K_KLT))
    return fail(NVKV_ERR_UNSUPPORTED, "the Hadamard and KLT key bases exclude each other");
  if (L->k_fmt == NVKV_FMT_BF16 && L->k_flags != 0) return fail(NVKV_ERR_UNSUPPORTED, "key transforms need NVFP4 keys");
  if ((L->k_flags & NVKV_K_KLT) && !L->k_basis) return fail(NVKV_ERR_NULL, "k_basis is NULL");
  if (!L->k_data || !L->v_data || !L->v_scales || !L->global_scale) return fail(NVKV_ERR_NULL, "cache pointer is NULL");
  if (L->k_fmt == NVKV_FMT_NVFP4 && !L->k_scales) return fail(NVKV_ERR_NULL, "k_scales is NULL");
  if ((L->k_flags & NVKV_K_SMOOTH) && (!L->k_smooth || !L->k_inv_smooth))
    return fail(NVKV_ERR_NULL, "smoothing vectors are NULL");
  return NVKV_OK;
}

size_t row_bytes(int32_t fmt) { return fmt == NVKV_FMT_BF16 ? 256 : (fmt == NVKV_FMT_NVFP4 ? 72 : 0); }

}  // namespace

extern "C" {

const char* nvkv_status_string(nvkv_status s) {
  switch (s) {
    case NVKV_OK: return "ok";
    case NVKV_ERR_NULL: return "null pointer";
    case NVKV_ERR_SHAPE: return "invalid shape or count";
    case NVKV_ERR_UNSUPPORTED: return "unsupported combination";
    case NVKV_ERR_WORKSPACE: return "workspace too small or misaligned";
    case NVKV_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* nvkv_last_error(void) { return g_last_error.c_str(); }

size_t nvkv_cache_array_bytes(int32_t fmt, int32_t part, int32_t num_pages, int32_t Hkv, int32_t page_size) {
  if (num_pages < 1 || Hkv < 1 || page_size < 16 || page_size % 16 != 0) return 0;
  const size_t rows = static_cast<size_t>(num_pages) * Hkv * page_size;
  if (fmt == NVKV_FMT_NVFP4) return part == NVKV_PART_CODES ? rows * 64 : (part == NVKV_PART_SCALES ? rows * 8 : 0);
  if (fmt == NVKV_FMT_BF16) return part == NVKV_PART_CODES ? rows * 256 : 0;
  return 0;
}

size_t nvkv_cache_bytes_per_token(int32_t k_fmt, int32_t v_fmt, int32_t Hkv, int32_t layers) {
  const size_t rk = row_bytes(k_fmt), rv = row_bytes(v_fmt);
  if (!rk || !rv || Hkv < 1 || layers < 1) return 0;
  return static_cast<size_t>(layers) * Hkv * (rk + rv);
}

nvkv_status nvkv_calibrate_key_smoothing(const uint16_t* k_win, const uint16_t* v_win, int32_t W, int32_t T,
                                         int32_t Hkv, int32_t exclude_pos0, uint32_t k_flags, float* s_out,
                                         float* r_out, float* g_out, void* stream) {
  if (!k_win && !v_win) return fail(NVKV_ERR_NULL, "both window pointers are NULL");
  if (!g_out) return fail(NVKV_ERR_NULL, "g_out is NULL");
  if (k_win && (!s_out || !r_out)) return fail(NVKV_ERR_NULL, "s_out / r_out is NULL");
  if (W < 1 || W > kMaxGridYZ || T < 1 || Hkv < 1) return fail(NVKV_ERR_SHAPE, "W, T, Hkv must be >= 1 (W <= 65535)");
  if (static_cast<int64_t>(W) * T * Hkv * NVKV_HEAD_DIM > INT32_MAX)
    return fail(NVKV_ERR_SHAPE, "calibration windows exceed 2^31 elements");
  if (k_flags & ~(NVKV_K_SMOOTH | NVKV_K_HADAMARD | NVKV_K_MSE_SCALE | NVKV_K_KLT))
    return fail(NVKV_ERR_UNSUPPORTED, "unknown k_flags bits");
  if ((k_flags & NVKV_K_HADAMARD) && (k_flags & NVKV_K_KLT))
    return fail(NVKV_ERR_UNSUPPORTED, "the Hadamard and KLT key bases exclude each other");
  (void)hipGetLastError();
  return hip_status(nvkv::launch_calibrate(k_win, v_win, W, T, Hkv, exclude_pos0, k_flags, s_out, r_out, g_out,
                                           static_cast<hipStream_t>(stream)),
                    "calibrate launch");
}

size_t nvkv_calibrate_key_basis_workspace_bytes(int32_t Hkv) {
  if (Hkv < 1 || Hkv > kMaxGridYZ) return 0;
  return nvkv::klt_workspace_bytes(Hkv);
}

nvkv_status nvkv_calibrate_key_basis(const uint16_t* k_win, int32_t W, int32_t T, int32_t Hkv, int32_t exclude_pos0,
                                     uint32_t k_flags, const float* r, float* basis_out, float* g_out,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  if (!k_win || !basis_out || !g_out) return fail(NVKV_ERR_NULL, "k_win / basis_out / g_out is NULL");
  if (W < 1 || T < 2 || Hkv < 1 || Hkv > kMaxGridYZ) return fail(NVKV_ERR_SHAPE, "W >= 1, T >= 2, 1 <= Hkv <= 65535");
  if (static_cast<int64_t>(W) * T * Hkv * NVKV_HEAD_DIM > INT32_MAX)
    return fail(NVKV_ERR_SHAPE, "calibration windows exceed 2^31 elements");
  if (k_flags & ~(NVKV_K_SMOOTH | NVKV_K_HADAMARD | NVKV_K_MSE_SCALE | NVKV_K_KLT))
    return fail(NVKV_ERR_UNSUPPORTED, "unknown k_flags bits");
  if (!(k_flags & NVKV_K_KLT) || (k_flags & NVKV_K_HADAMARD))
    return fail(NVKV_ERR_UNSUPPORTED, "k_flags must select the KLT basis and not the Hadamard basis");
  if ((k_flags & NVKV_K_SMOOTH) && !r) return fail(NVKV_ERR_NULL, "r is NULL with NVKV_K_SMOOTH");
  if (!workspace || workspace_bytes < nvkv::klt_workspace_bytes(Hkv) ||
      (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(NVKV_ERR_WORKSPACE, "workspace missing, too small or not 256-byte aligned");
  (void)hipGetLastError();
  return hip_status(nvkv::launch_calibrate_basis(k_win, W, T, Hkv, exclude_pos0, k_flags, r, basis_out, g_out,
                                                 workspace, static_cast<hipStream_t>(stream)),
                    "calibrate_key_basis launch");
}

nvkv_status nvkv_quantize_append_kv(const nvkv_layer* layer, const uint16_t* k_new, const uint16_t* v_new,
                                    const int32_t* slot_mapping, int32_t N, void* stream) {
  const nvkv_status st = check_layer(layer);
  if (st != NVKV_OK) return st;
  if (N < 0) return fail(NVKV_ERR_SHAPE, "N must be >= 0");
  if (N == 0) return NVKV_OK;
  if (!k_new || !v_new || !slot_mapping) return fail(NVKV_ERR_NULL, "input pointer is NULL");
  if (static_cast<int64_t>(N) * layer->num_kv_heads * 2 > INT32_MAX / 2)
    return fail(NVKV_ERR_SHAPE, "N * Hkv too large for one call");
  (void)hipGetLastError();
  return hip_status(nvkv::launch_quantize_append(*layer, k_new, v_new, slot_mapping, N,
                                                 static_cast<hipStream_t>(stream)),
                    "quantize_append launch");
}

size_t nvkv_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t max_seq_len, int32_t split_tokens) {
  if (B < 1 || Hkv < 1 || Hq != 4 * Hkv || max_seq_len < 0 || split_tokens < 0 || split_tokens % 32 != 0) return 0;
  const nvkv::DecodePlan plan = nvkv::plan_decode(B, Hkv, max_seq_len, split_tokens, false);
  if (plan.n_splits <= 1) return 0;
  return nvkv::decode_workspace_bytes(B, Hkv, plan);
}

namespace {
// use_scratch: the allocation-free variant (the library's static per-device scratch instead of
// a caller workspace).
nvkv_status decode_common(const nvkv_layer* layer, const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                          bool append, int32_t B, int32_t Hq, const int32_t* page_table, int32_t max_pages_per_seq,
                          const int32_t* seq_lens, int32_t max_seq_len, float sm_scale, float* out, void* workspace,
                          size_t workspace_bytes, int32_t split_tokens, void* stream, bool use_scratch = false) {
  const nvkv_status st = check_layer(layer);
  if (st != NVKV_OK) return st;
  if (!q || !page_table || !seq_lens || !out) return fail(NVKV_ERR_NULL, "input/output pointer is NULL");
  if (append && (!k_new || !v_new)) return fail(NVKV_ERR_NULL, "k_new / v_new is NULL");
  if (B < 1 || B > kMaxGridYZ) return fail(NVKV_ERR_SHAPE, "B must be in [1, 65535]");
  if (Hq < 1 || Hq % layer->num_kv_heads != 0) return fail(NVKV_ERR_SHAPE, "Hq must be a multiple of Hkv");
  if (Hq != 4 * layer->num_kv_heads) return fail(NVKV_ERR_UNSUPPORTED, "only 4 query heads per KV head");
  if (max_pages_per_seq < 1 || max_seq_len < 0) return fail(NVKV_ERR_SHAPE, "max_pages_per_seq >= 1, max_seq_len >= 0");
  if (split_tokens < 0 || split_tokens % 32 != 0) return fail(NVKV_ERR_SHAPE, "split_tokens must be a multiple of 32");
  if (!std::isfinite(sm_scale)) return fail(NVKV_ERR_SHAPE, "sm_scale must be finite");
  const nvkv::DecodePlan plan = nvkv::plan_decode(B, layer->num_kv_heads, max_seq_len, split_tokens, append);
  if (plan.n_splits > 1 && use_scratch) {
    if (static_cast<int64_t>(B) * layer->num_kv_heads > static_cast<int64_t>(nvkv::kScratchUnits) ||
        nvkv::decode_partial_bytes(B, layer->num_kv_heads, plan) > nvkv::kScratchPartialBytes)
      return fail(NVKV_ERR_WORKSPACE, "the call needs more split state than the static scratch holds "
                                      "(B * Hkv <= 2048 and at most 7 MiB of split partials)");
  } else if (plan.n_splits > 1) {
    const size_t need = nvkv::decode_workspace_bytes(B, layer->num_kv_heads, plan);
    if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255u))
      return fail(NVKV_ERR_WORKSPACE, "workspace missing, too small or not 256-byte aligned");
  }
  (void)hipGetLastError();
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  nvkv::DecodeWs ws{nullptr, nullptr, nullptr};
  if (plan.n_splits > 1) {
    if (use_scratch) {
      const nvkv_status s0 = hip_status(nvkv::scratch_decode_workspace(B, layer->num_kv_heads, plan, hs, &ws),
                                        "static scratch set-up");
      if (s0 != NVKV_OK) return s0;
    } else {
      ws = nvkv::carve_decode_workspace(workspace, B, layer->num_kv_heads, plan);
    }
  }
  if (append && plan.pipe2) {
    // Long splits: the decode dominates and the fused kernel would give up a cache
    // wavefront, so the new tokens go in with the append kernel first (same effect).
    const int64_t cap_pages = static_cast<int64_t>(max_pages_per_seq) * layer->page_size;
    const int32_t seq_cap = static_cast<int32_t>(cap_pages < max_seq_len ? cap_pages : max_seq_len);
    const nvkv_status s1 = hip_status(nvkv::launch_quantize_append_rows(*layer, k_new, v_new, nullptr, B, page_table,
                                                                        seq_lens, max_pages_per_seq, seq_cap, hs),
                                      "decode-append: append launch");
    if (s1 != NVKV_OK) return s1;
    nvkv::DecodePlan dplan = nvkv::plan_decode(B, layer->num_kv_heads, max_seq_len, split_tokens, false);
    return hip_status(nvkv::launch_decode(*layer, q, nullptr, nullptr, B, Hq, page_table, max_pages_per_seq,
                                          seq_lens, max_seq_len, sm_scale, out, ws, dplan, hs),
                      "decode-append: decode launch");
  }
  return hip_status(nvkv::launch_decode(*layer, q, append ? k_new : nullptr, append ? v_new : nullptr, B, Hq,
                                        page_table, max_pages_per_seq, seq_lens, max_seq_len, sm_scale, out,
                                        ws, plan, hs),
                    append ? "decode-append launch" : "decode launch");
}
}  // namespace

nvkv_status nvkv_decode_attention_nvfp4(const nvkv_layer* layer, const uint16_t* q, int32_t B, int32_t Hq,
                                        const int32_t* page_table, int32_t max_pages_per_seq,
                                        const int32_t* seq_lens, int32_t max_seq_len, float sm_scale, float* out,
                                        void* workspace, size_t workspace_bytes, int32_t split_tokens,
                                        void* stream) {
  return decode_common(layer, q, nullptr, nullptr, false, B, Hq, page_table, max_pages_per_seq, seq_lens,
                       max_seq_len, sm_scale, out, workspace, workspace_bytes, split_tokens, stream);
}

nvkv_status nvkv_decode_append_attention_nvfp4(const nvkv_layer* layer, const uint16_t* q, const uint16_t* k_new,
                                               const uint16_t* v_new, int32_t B, int32_t Hq,
                                               const int32_t* page_table, int32_t max_pages_per_seq,
                                               const int32_t* seq_lens, int32_t max_seq_len, float sm_scale,
                                               float* out, void* workspace, size_t workspace_bytes,
                                               int32_t split_tokens, void* stream) {
  return decode_common(layer, q, k_new, v_new, true, B, Hq, page_table, max_pages_per_seq, seq_lens, max_seq_len,
                       sm_scale, out, workspace, workspace_bytes, split_tokens, stream);
}

nvkv_status nvkv_decode_append_attention_nvfp4_noalloc(const nvkv_layer* layer, const uint16_t* q,
                                                       const uint16_t* k_new, const uint16_t* v_new, int32_t B,
                                                       int32_t Hq, const int32_t* page_table,
                                                       int32_t max_pages_per_seq, const int32_t* seq_lens,
                                                       int32_t max_seq_len, float sm_scale, float* out,
                                                       int32_t split_tokens, void* stream) {
  return decode_common(layer, q, k_new, v_new, true, B, Hq, page_table, max_pages_per_seq, seq_lens, max_seq_len,
                       sm_scale, out, nullptr, 0, split_tokens, stream, true);
}

nvkv_status nvkv_prefill_attention_nvfp4(const nvkv_layer* layer, const uint16_t* q, int32_t B, int32_t Tq,
                                         int32_t Hq, const int32_t* page_table, int32_t max_pages_per_seq,
                                         const int32_t* seq_lens, int32_t max_seq_len, float sm_scale, float* out,
                                         void* stream) {
  const nvkv_status st = check_layer(layer);
  if (st != NVKV_OK) return st;
  if (B < 1 || B > kMaxGridYZ) return fail(NVKV_ERR_SHAPE, "B must be in [1, 65535]");
  if (Tq < 0) return fail(NVKV_ERR_SHAPE, "Tq must be >= 0");
  if (Tq == 0) return NVKV_OK;
  if (!q || !page_table || !seq_lens || !out) return fail(NVKV_ERR_NULL, "input/output pointer is NULL");
  if (Hq < 1 || Hq % layer->num_kv_heads != 0) return fail(NVKV_ERR_SHAPE, "Hq must be a multiple of Hkv");
  if (Hq != 4 * layer->num_kv_heads) return fail(NVKV_ERR_UNSUPPORTED, "only 4 query heads per KV head");
  if (max_pages_per_seq < 1 || max_seq_len < 0) return fail(NVKV_ERR_SHAPE, "max_pages_per_seq >= 1, max_seq_len >= 0");
  if (!std::isfinite(sm_scale)) return fail(NVKV_ERR_SHAPE, "sm_scale must be finite");
  if (static_cast<int64_t>(B) * Tq * Hq * NVKV_HEAD_DIM > INT64_C(1) << 40)
    return fail(NVKV_ERR_SHAPE, "B * Tq * Hq too large");
  (void)hipGetLastError();
  return hip_status(nvkv::launch_prefill_attention(*layer, q, B, Tq, Hq, page_table, max_pages_per_seq, seq_lens,
                                                   max_seq_len, sm_scale, out, static_cast<hipStream_t>(stream)),
                    "prefill attention launch");
}

}  // extern "C"
