// Internal declarations shared by the C ABI layer and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/nvfp4kv.h"

namespace nvkv {

hipError_t launch_quantize_append(const nvkv_layer& L, const uint16_t* k_new, const uint16_t* v_new,
                                  const int32_t* slots, int32_t N, hipStream_t stream);
// slots == nullptr: row n is the new token of sequence n, at position
// min(seq_lens[n], seq_cap) - 1 taken through the page table.
hipError_t launch_quantize_append_rows(const nvkv_layer& L, const uint16_t* k_new, const uint16_t* v_new,
                                       const int32_t* slots, int32_t N, const int32_t* page_table,
                                       const int32_t* seq_lens, int32_t max_pages_per_seq, int32_t seq_cap,
                                       hipStream_t stream);

hipError_t launch_calibrate(const uint16_t* k_win, const uint16_t* v_win, int32_t W, int32_t T, int32_t hkv,
                            int32_t exclude_pos0, uint32_t k_flags, float* s_out, float* r_out, float* g_out,
                            hipStream_t stream);

// Static per-head KLT basis and g_K (workspace: fp64 covariance and eigenvectors per head).
size_t klt_workspace_bytes(int32_t hkv);
hipError_t launch_calibrate_basis(const uint16_t* k_win, int32_t W, int32_t T, int32_t hkv, int32_t exclude_pos0,
                                  uint32_t k_flags, const float* r, float* basis_out, float* g_out, void* workspace,
                                  hipStream_t stream);

// Decode split plan: number of splits and tokens per split for a call.
struct DecodePlan {
  int32_t split_tokens;   // tokens handled by one workgroup (multiple of 32)
  int32_t n_splits;       // workgroups per (sequence, KV head)
  int32_t waves;          // wavefronts per workgroup (4..16)
  bool pipe2;             // two-deep software pipeline (several iterations per wavefront)
  bool append;            // fused append of the new token (one extra wavefront)
};
DecodePlan plan_decode(int32_t B, int32_t Hkv, int32_t max_seq_len, int32_t split_tokens, bool append);
size_t decode_workspace_bytes(int32_t B, int32_t Hkv, const DecodePlan& plan);

// Where a decode call keeps its cross-split state: one arrival counter per (sequence, KV head),
// 256 bytes apart (zero between calls), and the per-split partials (m, l) and O.
struct DecodeWs {
  unsigned* counters;
  float* ml;
  float* o;
};
// The layout inside a caller's workspace of decode_workspace_bytes(B, Hkv, plan) bytes.
DecodeWs carve_decode_workspace(void* workspace, int32_t B, int32_t Hkv, const DecodePlan& plan);

// The allocation-free variant keeps its cross-split state in a static device array of fixed
// size, one per GPU: arrival counters for up to kScratchUnits (sequence, KV head) units, then
// kScratchPartialBytes of partials.
constexpr size_t kScratchUnits = 2048;
constexpr size_t kScratchPartialBytes = size_t(7) << 20;
// Bytes of partials a plan needs (0 with one split).
size_t decode_partial_bytes(int32_t B, int32_t Hkv, const DecodePlan& plan);
// The static scratch of the current device, carved for a call (B * Hkv <= kScratchUnits and
// decode_partial_bytes <= kScratchPartialBytes, checked by the caller).  The first call on a
// device looks up the array's device address and clears its counters on `stream`.
hipError_t scratch_decode_workspace(int32_t B, int32_t Hkv, const DecodePlan& plan, hipStream_t stream,
                                    DecodeWs* ws);

// k_new / v_new non-null: fused append of the new token of each sequence (plan.append).
// trace non-null: the measurement instance, which also writes phase stamps (kTraceSlots per
// workgroup, see nvkv_decode.hip); NVFP4 keys without the KLT basis only.
hipError_t launch_decode(const nvkv_layer& L, const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                         int32_t B, int32_t Hq, const int32_t* page_table, int32_t max_pages_per_seq,
                         const int32_t* seq_lens, int32_t max_seq_len, float sm_scale, float* out,
                         const DecodeWs& ws, const DecodePlan& plan, hipStream_t stream, uint64_t* trace = nullptr);

// Causal attention of the last Tq positions of each sequence over the cache (no workspace).
hipError_t launch_prefill_attention(const nvkv_layer& L, const uint16_t* q, int32_t B, int32_t Tq, int32_t Hq,
                                    const int32_t* page_table, int32_t max_pages_per_seq, const int32_t* seq_lens,
                                    int32_t max_seq_len, float sm_scale, float* out, hipStream_t stream);

}  // namespace nvkv
