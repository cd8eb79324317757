// Measurement helpers of the bench (libnvkv_bench.so; not part of the library's C ABI):
//   - a plain streaming read of given device arrays (the reference point for what one launch
//     can stream at the size of a decode launch's bytes);
//   - the phase-stamped instance of the decode kernels (the same kernel sources, compiled with
//     the stamps of k_decode<..., TRACE>), for a timeline of where a launch spends its time;
//   - quantize_append_kv in the layout of one wavefront per (token, KV head) row, the
//     comparison point for the library's layout of one lane per 16-element block.
// All return a hipError_t as int.
#include <hip/hip_runtime.h>

#include "nvkv_encode.hpp"
#include "nvkv_internal.hpp"

#define NVKVB_API extern "C" __attribute__((visibility("default")))

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kMaxSeg = 4;

struct StreamArgs {
  const uint8_t* base[kMaxSeg];
  uint32_t words[kMaxSeg];     // 16-byte words of each segment
  int nseg;
  uint32_t* sink;              // written only when the folded value has an impossible pattern
};

// Every 16-byte word of every segment is read once (non-temporal, as the decode kernel reads
// the cache), four loads in flight per lane; the loaded words are folded so the loads stay.
__global__ void __launch_bounds__(256) k_stream_read(StreamArgs a) {
  const uint32_t nthr = gridDim.x * blockDim.x;
  const uint32_t gid = blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0u;
  for (int sgi = 0; sgi < a.nseg; ++sgi) {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.base[sgi]), 0, a.words[sgi] * 16u, 0x00020000);
    const uint32_t n = a.words[sgi];
    uint32_t i = gid;
    for (; i + 3 * nthr < n; i += 4 * nthr) {
      u32x4_t v0 = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, i * 16u, 0, 2));
      u32x4_t v1 = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, (i + nthr) * 16u, 0, 2));
      u32x4_t v2 = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, (i + 2 * nthr) * 16u, 0, 2));
      u32x4_t v3 = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, (i + 3 * nthr) * 16u, 0, 2));
      acc ^= (v0[0] ^ v0[1] ^ v0[2] ^ v0[3]) + (v1[0] ^ v1[1] ^ v1[2] ^ v1[3]) +
             (v2[0] ^ v2[1] ^ v2[2] ^ v2[3]) + (v3[0] ^ v3[1] ^ v3[2] ^ v3[3]);
    }
    for (; i < n; i += nthr) {
      u32x4_t v = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, i * 16u, 0, 2));
      acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
  }
  if (acc == 0x9E3779B9u) a.sink[gid & 255u] = acc;
}

// quantize_append_kv with one wavefront per (token, KV head) row ([cache post] opening
// paragraph: 16-element blocks along head_dim with an E4M3 scale each; cache-config table:
// smoothing and the Hadamard-128 basis on keys).  Lane l holds elements 2l and 2l + 1, so a
// block is 8 consecutive lanes: the block maximum is a 3-step lane-xor reduction, the
// Hadamard stages 2..64 are lane-xor exchanges, and lane l's two E2M1 codes form byte l of
// the row.  Each lane decides its own two codes exactly (converter brackets, the bound-based
// encoder where they differ), so the bytes equal the library kernel's.  Four rows (one
// token's consecutive heads) per workgroup; grid y: 0 keys, 1 values.
struct RowWaveArgs {
  const uint16_t* src[2];     // k_new, v_new: bf16 [N][Hkv][128]
  uint8_t* codes[2];          // key codes (row-major), value codes (quad-interleaved words)
  uint8_t* scales[2];
  const float* inv_smooth;    // r [Hkv][128] (keys with smoothing)
  const float* gscale;        // [2] = {g_K, g_V}
  const int32_t* slots;       // [N]
  uint32_t kflags;            // key transform: 1 smoothing, 2 Hadamard
  int32_t n_rows;             // N * Hkv
  int32_t hkv;
  int32_t page_size;
  int64_t max_slot;
};

__global__ void __launch_bounds__(256) k_append_rowwave(RowWaveArgs a) {
#pragma clang fp contract(off)
  const int which = static_cast<int>(blockIdx.y);
  const int lane = threadIdx.x & 63;
  const int row = static_cast<int>(blockIdx.x) * 4 + static_cast<int>(threadIdx.x >> 6);
  if (row >= a.n_rows) return;                                   // uniform per wavefront
  const int n = row / a.hkv, h = row - n * a.hkv;
  const uint16_t* src = which ? a.src[1] : a.src[0];
  const uint32_t pair = reinterpret_cast<const uint32_t*>(src + static_cast<int64_t>(row) * nvkv::kHeadDim)[lane];
  float y0 = __uint_as_float(pair << 16), y1 = __uint_as_float(pair & 0xFFFF0000u);
  const uint32_t fl = which ? 0u : a.kflags;
  if (fl & 1u) {
    const float2 r = reinterpret_cast<const float2*>(a.inv_smooth + h * nvkv::kHeadDim)[lane];
    y0 = y0 * r.x;
    y1 = y1 * r.y;
  }
  if (fl & 2u) {                       // (y_i, y_i+s) <- (y_i + y_i+s, y_i - y_i+s), s = 1 .. 64
    const float t0 = y0 + y1, t1 = y0 - y1;
    y0 = t0;
    y1 = t1;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const float p0 = __shfl_xor(y0, m, 64), p1 = __shfl_xor(y1, m, 64);
      const bool upper = (lane & m) != 0;
      y0 = upper ? p0 - y0 : y0 + p0;
      y1 = upper ? p1 - y1 : y1 + p1;
    }
  }
  float A = fmaxf(fabsf(y0), fabsf(y1));
  A = fmaxf(A, __shfl_xor(A, 1, 64));
  A = fmaxf(A, __shfl_xor(A, 2, 64));
  A = fmaxf(A, __shfl_xor(A, 4, 64));
  const float g = a.gscale[which];
  const uint32_t S = nvkv::e4m3_scale_code(A, g);
  const float sigma = nvkv::e4m3_value(S);
  const float u = sigma * g;
  const float R = __builtin_amdgcn_rcpf(u);
  const float r1 = R * nvkv::kBracketDown, r2 = R * nvkv::kBracketUp;
  const uint32_t b1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y0 * r1, y1 * r1, 1.0f, 0) & 0xFFu;
  const uint32_t b2 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y0 * r2, y1 * r2, 1.0f, 0) & 0xFFu;
  uint32_t byte = b1;
  if (__builtin_expect(sigma > 0.0f && !(b1 == b2 && u >= 0x1p-125f), 0)) {
    const nvkv::E2m1Thresholds t(sigma, g);
    byte = nvkv::e2m1_nibble(y0, t) | (nvkv::e2m1_nibble(y1, t) << 4);
  }
  byte = sigma > 0.0f ? (nvkv::clear_zero_signs(byte) & 0xFFu) : 0u;
  // four bytes to lanes 4k (dword k of the row: elements 8k .. 8k + 7)
  uint32_t w = byte | (static_cast<uint32_t>(__shfl_down(static_cast<int>(byte), 1, 64)) << 8);
  w = w | (static_cast<uint32_t>(__shfl_down(static_cast<int>(w), 2, 64)) << 16);
  const int32_t slot = a.slots[n];
  if (slot < 0 || static_cast<int64_t>(slot) >= a.max_slot) return;
  const int32_t page = slot / a.page_size, off = slot - page * a.page_size;
  const int64_t ri = (static_cast<int64_t>(page) * a.hkv + h) * a.page_size + off;
  if ((lane & 3) == 0) {
    const int k = lane >> 2;
    uint8_t* dst = which ? a.codes[1] + (ri - (off & 3)) * 64 + 16 * k + 4 * (off & 3) : a.codes[0] + ri * 64 + 4 * k;
    *reinterpret_cast<uint32_t*>(dst) = w;
  }
  if ((lane & 7) == 0) {
    const int64_t sbase = (static_cast<int64_t>(page) * a.hkv + h) * a.page_size * 8;
    (which ? a.scales[1] : a.scales[0])[sbase + ((off >> 2) * 8 + (lane >> 3)) * 4 + (off & 3)] =
        static_cast<uint8_t>(S);
  }
}

}  // namespace

// Stream-read nseg (<= 4) device arrays of bytes[i] bytes (multiples of 16) with `grid`
// workgroups of 256 threads.  sink: 1 KiB of device memory.
NVKVB_API int nvkvb_stream_read(const void* const* ptrs, const size_t* bytes, int nseg, void* sink, int grid,
                                void* stream) {
  if (nseg < 1 || nseg > kMaxSeg || grid < 1 || !sink) return static_cast<int>(hipErrorInvalidValue);
  StreamArgs a{};
  for (int i = 0; i < nseg; ++i) {
    if (!ptrs[i] || bytes[i] % 16 != 0 || bytes[i] / 16 > 0xFFFFFFFFull / 16) return static_cast<int>(hipErrorInvalidValue);
    a.base[i] = static_cast<const uint8_t*>(ptrs[i]);
    a.words[i] = static_cast<uint32_t>(bytes[i] / 16);
  }
  a.nseg = nseg;
  a.sink = static_cast<uint32_t*>(sink);
  hipLaunchKernelGGL(k_stream_read, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream), a);
  return static_cast<int>(hipGetLastError());
}

// The split plan the library picks for a decode call: {n_splits, waves per workgroup, pipe2}.
NVKVB_API void nvkvb_decode_plan(int32_t B, int32_t Hkv, int32_t max_seq_len, int32_t split_tokens, int32_t append,
                                 int32_t* out3) {
  const nvkv::DecodePlan p = nvkv::plan_decode(B, Hkv, max_seq_len, split_tokens, append != 0);
  out3[0] = p.n_splits;
  out3[1] = p.waves;
  out3[2] = p.pipe2 ? 1 : 0;
}

// The phase-stamped decode (append != 0: the fused step, one launch).  Arguments as for
// nvkv_decode_append_attention_nvfp4 / nvkv_decode_attention_nvfp4 (validated by the caller:
// the bench passes the same arguments it times), plus trace: uint64
// [n_splits * Hkv * B][48] device memory, zero-filled by the caller.  The fused form with
// long splits (pipe2) is not traced (the library issues two launches there).
NVKVB_API int nvkvb_decode_trace(const nvkv_layer* layer, const uint16_t* q, const uint16_t* k_new,
                                 const uint16_t* v_new, int32_t append, int32_t B, int32_t Hq,
                                 const int32_t* page_table, int32_t max_pages_per_seq, const int32_t* seq_lens,
                                 int32_t max_seq_len, float sm_scale, float* out, void* workspace,
                                 int32_t split_tokens, uint64_t* trace, void* stream) {
  if (!layer || !trace) return static_cast<int>(hipErrorInvalidValue);
  const nvkv::DecodePlan plan = nvkv::plan_decode(B, layer->num_kv_heads, max_seq_len, split_tokens, append != 0);
  if (append && plan.pipe2) return static_cast<int>(hipErrorNotSupported);
  nvkv::DecodeWs ws{nullptr, nullptr, nullptr};
  if (plan.n_splits > 1) ws = nvkv::carve_decode_workspace(workspace, B, layer->num_kv_heads, plan);
  return static_cast<int>(nvkv::launch_decode(*layer, q, append ? k_new : nullptr, append ? v_new : nullptr, B, Hq,
                                              page_table, max_pages_per_seq, seq_lens, max_seq_len, sm_scale, out,
                                              ws, plan, static_cast<hipStream_t>(stream), trace));
}

// quantize_append_kv of N tokens with one wavefront per (token, KV head) row (k_append_rowwave):
// NVFP4 keys and values, key flags within NVKV_K_SMOOTH | NVKV_K_HADAMARD, slots given; code
// arrays 4-byte aligned.  Bytes identical to nvkv_quantize_append_kv's.
NVKVB_API int nvkvb_quantize_append_rowwave(const nvkv_layer* layer, const uint16_t* k_new, const uint16_t* v_new,
                                            const int32_t* slots, int32_t N, void* stream) {
  if (!layer || !k_new || !v_new || !slots || N < 0) return static_cast<int>(hipErrorInvalidValue);
  if (layer->k_fmt != NVKV_FMT_NVFP4 || layer->v_fmt != NVKV_FMT_NVFP4 || layer->head_dim != nvkv::kHeadDim ||
      (layer->k_flags & ~(NVKV_K_SMOOTH | NVKV_K_HADAMARD)) != 0u || layer->page_size < 16 ||
      layer->page_size % 16 != 0 || layer->num_kv_heads < 1)
    return static_cast<int>(hipErrorNotSupported);
  if (((reinterpret_cast<uintptr_t>(layer->k_data) | reinterpret_cast<uintptr_t>(layer->v_data)) & 3u) != 0)
    return static_cast<int>(hipErrorInvalidValue);
  if (N == 0) return static_cast<int>(hipSuccess);
  const int64_t rows = static_cast<int64_t>(N) * layer->num_kv_heads;
  if (rows > (int64_t{1} << 30)) return static_cast<int>(hipErrorInvalidValue);
  RowWaveArgs a{};
  a.src[0] = k_new;
  a.src[1] = v_new;
  a.codes[0] = static_cast<uint8_t*>(layer->k_data);
  a.codes[1] = static_cast<uint8_t*>(layer->v_data);
  a.scales[0] = layer->k_scales;
  a.scales[1] = layer->v_scales;
  a.inv_smooth = layer->k_inv_smooth;
  a.gscale = layer->global_scale;
  a.slots = slots;
  a.kflags = layer->k_flags;
  a.n_rows = static_cast<int32_t>(rows);
  a.hkv = layer->num_kv_heads;
  a.page_size = layer->page_size;
  a.max_slot = static_cast<int64_t>(layer->num_pages) * layer->page_size;
  hipLaunchKernelGGL(k_append_rowwave, dim3(static_cast<uint32_t>((rows + 3) / 4), 2), dim3(256), 0,
                     static_cast<hipStream_t>(stream), a);
  return static_cast<int>(hipGetLastError());
}
