"""ctypes binding of libnvfp4kv.so: argument marshalling only.

Every function here forwards to the C entry point of the same name (include/nvfp4kv.h);
torch tensors are passed as device pointers and the current HIP stream.  There is no
fallback: if the shared library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libnvfp4kv.so")

NVKV_OK = 0
STATUS_NAMES = {0: "NVKV_OK", 1: "NVKV_ERR_NULL", 2: "NVKV_ERR_SHAPE", 3: "NVKV_ERR_UNSUPPORTED",
                4: "NVKV_ERR_WORKSPACE", 5: "NVKV_ERR_HIP"}
FMT_BF16, FMT_NVFP4 = 0, 1
K_SMOOTH, K_HADAMARD, K_MSE_SCALE, K_KLT = 1, 2, 4, 8
PART_CODES, PART_SCALES = 0, 1
HEAD_DIM = 128

EXPORTED = ["nvkv_calibrate_key_smoothing", "nvkv_quantize_append_kv", "nvkv_decode_workspace_bytes",
            "nvkv_decode_attention_nvfp4", "nvkv_decode_append_attention_nvfp4", "nvkv_cache_array_bytes", "nvkv_cache_bytes_per_token",
            "nvkv_status_string", "nvkv_last_error", "nvkv_prefill_attention_nvfp4",
            "nvkv_calibrate_key_basis_workspace_bytes", "nvkv_calibrate_key_basis",
            "nvkv_decode_append_attention_nvfp4_noalloc"]


class NvkvError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({detail})")


class Layer(ctypes.Structure):
    """Mirror of struct nvkv_layer."""
    _fields_ = [
        ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32),
        ("k_fmt", ctypes.c_int32), ("v_fmt", ctypes.c_int32),
        ("k_flags", ctypes.c_uint32), ("reserved", ctypes.c_int32),
        ("k_data", ctypes.c_void_p), ("v_data", ctypes.c_void_p),
        ("k_scales", ctypes.c_void_p), ("v_scales", ctypes.c_void_p),
        ("k_smooth", ctypes.c_void_p), ("k_inv_smooth", ctypes.c_void_p),
        ("global_scale", ctypes.c_void_p), ("k_basis", ctypes.c_void_p),
    ]


_lib = None


def load(path: str | None = None) -> ctypes.CDLL:
    """Load the native library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise ImportError(f"native library {path} is missing: build it with "
                          f"`python -m nvfp4_bit_kv_amd.build` (there is no fallback path)")
    lib = ctypes.CDLL(path)
    vp, i32, u32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_float, ctypes.c_size_t
    lib.nvkv_calibrate_key_smoothing.argtypes = [vp, vp, i32, i32, i32, i32, u32, vp, vp, vp, vp]
    lib.nvkv_calibrate_key_smoothing.restype = ctypes.c_int
    lib.nvkv_calibrate_key_basis_workspace_bytes.argtypes = [i32]
    lib.nvkv_calibrate_key_basis_workspace_bytes.restype = sz
    lib.nvkv_calibrate_key_basis.argtypes = [vp, i32, i32, i32, i32, u32, vp, vp, vp, vp, sz, vp]
    lib.nvkv_calibrate_key_basis.restype = ctypes.c_int
    lib.nvkv_quantize_append_kv.argtypes = [ctypes.POINTER(Layer), vp, vp, vp, i32, vp]
    lib.nvkv_quantize_append_kv.restype = ctypes.c_int
    lib.nvkv_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.nvkv_decode_workspace_bytes.restype = sz
    lib.nvkv_decode_attention_nvfp4.argtypes = [ctypes.POINTER(Layer), vp, i32, i32, vp, i32, vp, i32, f32, vp,
                                                vp, sz, i32, vp]
    lib.nvkv_decode_attention_nvfp4.restype = ctypes.c_int
    lib.nvkv_decode_append_attention_nvfp4.argtypes = [ctypes.POINTER(Layer), vp, vp, vp, i32, i32, vp, i32, vp, i32,
                                                       f32, vp, vp, sz, i32, vp]
    lib.nvkv_decode_append_attention_nvfp4.restype = ctypes.c_int
    lib.nvkv_decode_append_attention_nvfp4_noalloc.argtypes = [ctypes.POINTER(Layer), vp, vp, vp, i32, i32, vp, i32,
                                                               vp, i32, f32, vp, i32, vp]
    lib.nvkv_decode_append_attention_nvfp4_noalloc.restype = ctypes.c_int
    lib.nvkv_prefill_attention_nvfp4.argtypes = [ctypes.POINTER(Layer), vp, i32, i32, i32, vp, i32, vp, i32, f32,
                                                 vp, vp]
    lib.nvkv_prefill_attention_nvfp4.restype = ctypes.c_int
    lib.nvkv_cache_array_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.nvkv_cache_array_bytes.restype = sz
    lib.nvkv_cache_bytes_per_token.argtypes = [i32, i32, i32, i32]
    lib.nvkv_cache_bytes_per_token.restype = sz
    lib.nvkv_status_string.argtypes = [ctypes.c_int]
    lib.nvkv_status_string.restype = ctypes.c_char_p
    lib.nvkv_last_error.argtypes = []
    lib.nvkv_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    if not torch.cuda.is_available():
        return None          # NULL stream; argument errors are still reported before any HIP call
    return torch.cuda.current_stream().cuda_stream


def _check(status: int, where: str) -> None:
    if status != NVKV_OK:
        raise NvkvError(status, where, load().nvkv_last_error().decode())


def calibrate_key_smoothing(k_win, v_win, W: int, T: int, Hkv: int, exclude_pos0: bool, k_flags: int,
                            s_out, r_out, g_out, stream=None) -> None:
    _check(load().nvkv_calibrate_key_smoothing(_ptr(k_win), _ptr(v_win), W, T, Hkv, int(bool(exclude_pos0)),
                                               k_flags, _ptr(s_out), _ptr(r_out), _ptr(g_out), _stream(stream)),
           "nvkv_calibrate_key_smoothing")


def calibrate_key_basis_workspace_bytes(Hkv: int) -> int:
    return int(load().nvkv_calibrate_key_basis_workspace_bytes(Hkv))


def calibrate_key_basis(k_win, W: int, T: int, Hkv: int, exclude_pos0: bool, k_flags: int, r, basis_out, g_out,
                        workspace, workspace_bytes: int, stream=None) -> None:
    _check(load().nvkv_calibrate_key_basis(_ptr(k_win), W, T, Hkv, int(bool(exclude_pos0)), k_flags, _ptr(r),
                                           _ptr(basis_out), _ptr(g_out), _ptr(workspace), workspace_bytes,
                                           _stream(stream)), "nvkv_calibrate_key_basis")


def quantize_append_kv(layer: Layer, k_new, v_new, slot_mapping, N: int, stream=None) -> None:
    _check(load().nvkv_quantize_append_kv(ctypes.byref(layer), _ptr(k_new), _ptr(v_new), _ptr(slot_mapping), N,
                                          _stream(stream)), "nvkv_quantize_append_kv")


def decode_workspace_bytes(B: int, Hq: int, Hkv: int, max_seq_len: int, split_tokens: int = 0) -> int:
    return int(load().nvkv_decode_workspace_bytes(B, Hq, Hkv, max_seq_len, split_tokens))


def decode_attention_nvfp4(layer: Layer, q, B: int, Hq: int, page_table, max_pages_per_seq: int, seq_lens,
                           max_seq_len: int, sm_scale: float, out, workspace, workspace_bytes: int,
                           split_tokens: int = 0, stream=None) -> None:
    _check(load().nvkv_decode_attention_nvfp4(ctypes.byref(layer), _ptr(q), B, Hq, _ptr(page_table),
                                              max_pages_per_seq, _ptr(seq_lens), max_seq_len, sm_scale, _ptr(out),
                                              _ptr(workspace), workspace_bytes, split_tokens, _stream(stream)),
           "nvkv_decode_attention_nvfp4")


def decode_append_attention_nvfp4(layer: Layer, q, k_new, v_new, B: int, Hq: int, page_table,
                                  max_pages_per_seq: int, seq_lens, max_seq_len: int, sm_scale: float, out,
                                  workspace, workspace_bytes: int, split_tokens: int = 0, stream=None) -> None:
    _check(load().nvkv_decode_append_attention_nvfp4(ctypes.byref(layer), _ptr(q), _ptr(k_new), _ptr(v_new), B, Hq,
                                                     _ptr(page_table), max_pages_per_seq, _ptr(seq_lens),
                                                     max_seq_len, sm_scale, _ptr(out), _ptr(workspace),
                                                     workspace_bytes, split_tokens, _stream(stream)),
           "nvkv_decode_append_attention_nvfp4")


def decode_append_attention_nvfp4_noalloc(layer: Layer, q, k_new, v_new, B: int, Hq: int, page_table,
                                          max_pages_per_seq: int, seq_lens, max_seq_len: int, sm_scale: float,
                                          out, split_tokens: int = 0, stream=None) -> None:
    _check(load().nvkv_decode_append_attention_nvfp4_noalloc(ctypes.byref(layer), _ptr(q), _ptr(k_new), _ptr(v_new),
                                                             B, Hq, _ptr(page_table), max_pages_per_seq,
                                                             _ptr(seq_lens), max_seq_len, sm_scale, _ptr(out),
                                                             split_tokens, _stream(stream)),
           "nvkv_decode_append_attention_nvfp4_noalloc")


def prefill_attention_nvfp4(layer: Layer, q, B: int, Tq: int, Hq: int, page_table, max_pages_per_seq: int,
                            seq_lens, max_seq_len: int, sm_scale: float, out, stream=None) -> None:
    _check(load().nvkv_prefill_attention_nvfp4(ctypes.byref(layer), _ptr(q), B, Tq, Hq, _ptr(page_table),
                                               max_pages_per_seq, _ptr(seq_lens), max_seq_len, sm_scale, _ptr(out),
                                               _stream(stream)),
           "nvkv_prefill_attention_nvfp4")


def cache_array_bytes(fmt: int, part: int, num_pages: int, Hkv: int, page_size: int) -> int:
    return int(load().nvkv_cache_array_bytes(fmt, part, num_pages, Hkv, page_size))


def cache_bytes_per_token(k_fmt: int, v_fmt: int, Hkv: int, layers: int) -> int:
    return int(load().nvkv_cache_bytes_per_token(k_fmt, v_fmt, Hkv, layers))


def status_string(status: int) -> str:
    return load().nvkv_status_string(status).decode()


def last_error() -> str:
    return load().nvkv_last_error().decode()
