"""NVFP4 attention-KV-cache path for AMD MI355X (gfx950): Python binding of libnvfp4kv.so.

The three operations (calibrate_key_smoothing, quantize_append_kv, decode_attention_nvfp4),
the fused decode step decode_append_attention_nvfp4 (append the new token, then attend) and
the causal multi-query prefill_attention_nvfp4 (a block of positions over the cache),
run entirely in the HIP kernels of the native library; this package only marshals
arguments and allocates torch buffers.  Importing it does not need a GPU; calling the
operations needs the built library (`python -m nvfp4_bit_kv_amd.build`) and fails loudly
without it.
"""
from ._native import (FMT_BF16, FMT_NVFP4, HEAD_DIM, K_HADAMARD, K_KLT, K_MSE_SCALE, K_SMOOTH, PART_CODES,  # noqa: F401
                      PART_SCALES, EXPORTED, LIB_PATH, Layer, NvkvError, cache_array_bytes,
                      cache_bytes_per_token, calibrate_key_basis, calibrate_key_basis_workspace_bytes,
                      calibrate_key_smoothing, decode_append_attention_nvfp4, decode_append_attention_nvfp4_noalloc,
                      decode_attention_nvfp4,
                      decode_workspace_bytes, last_error, load, prefill_attention_nvfp4, quantize_append_kv,
                      status_string)
from .cache import CacheLayer  # noqa: F401
