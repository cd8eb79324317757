// Measurement helpers of the bench (libnvkv_bench.so; not part of the library's C ABI):
//   - a plain streaming read of given device arrays (the reference point for what one launch
//     can stream at the size of a decode launch's bytes);
//   - the phase-stamped instance of the decode kernels (the same kernel sources, compiled with
//     the stamps of k_decode<..., TRACE>), for a timeline of where a launch spends its time.
// Both return a hipError_t as int.
#include <hip/hip_runtime.h>

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
