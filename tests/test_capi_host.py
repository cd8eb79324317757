"""Host-side checks of the C ABI that need no GPU: the library loads, exports every symbol
that include/nvfp4kv.h declares, reports argument errors as status codes before any HIP
call, and its size helpers agree with the oracle's sizes."""
import ctypes
import os
import re

import pytest

import nvfp4_bit_kv_amd as nk
from oracle import nvfp4_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    text = open(os.path.join(ROOT, "include", "nvfp4kv.h")).read()
    return sorted(set(re.findall(r"NVKV_API\s+[\w\s\*]+?\b(nvkv_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def clib():
    if not os.path.exists(nk.LIB_PATH):
        from nvfp4_bit_kv_amd import build
        build.build()
    return nk.load()


def test_every_declared_symbol_is_exported(clib):
    decl = _declared_symbols()
    assert len(decl) == 13, decl
    assert sorted(decl) == sorted(nk.EXPORTED)
    for name in decl:
        assert hasattr(clib, name), name
    out = os.popen(f"nm -D --defined-only {nk.LIB_PATH}").read()
    exported = set(re.findall(r" T (nvkv_\w+)", out))
    assert exported == set(decl)


def test_status_strings(clib):
    for code in range(6):
        assert nk.status_string(code)
    assert nk.status_string(0) == "ok"


def test_sizes_match_oracle(clib):
    for kf, vf, kn, vn in [(0, 0, "bf16", "bf16"), (1, 1, "nvfp4", "nvfp4"), (0, 1, "bf16", "nvfp4")]:
        assert nk.cache_bytes_per_token(kf, vf, 8, 36) == O.cache_bytes_per_token(kn, vn, 8, 36)
    assert nk.cache_bytes_per_token(0, 0, 8, 36) == 147456
    assert nk.cache_array_bytes(1, 0, 10, 8, 16) == 10 * 8 * 16 * 64
    assert nk.cache_array_bytes(1, 1, 10, 8, 16) == 10 * 8 * 16 * 8
    assert nk.cache_array_bytes(0, 0, 10, 8, 16) == 10 * 8 * 16 * 256
    assert nk.cache_array_bytes(0, 1, 10, 8, 16) == 0
    assert nk.cache_array_bytes(1, 0, 10, 8, 20) == 0


def _layer(**kw):
    L = nk.Layer()
    L.num_kv_heads, L.head_dim, L.page_size, L.num_pages = 8, 128, 16, 4
    L.k_fmt, L.v_fmt, L.k_flags, L.reserved = 1, 1, 1, 0
    L.k_data = L.v_data = L.k_scales = L.v_scales = 0x1000
    L.k_smooth = L.k_inv_smooth = L.global_scale = 0x2000
    for k, v in kw.items():
        setattr(L, k, v)
    return L


BAD_LAYERS = [
    (dict(head_dim=64), 2), (dict(num_kv_heads=0), 2), (dict(page_size=24), 2), (dict(page_size=0), 2),
    (dict(num_pages=0), 2), (dict(reserved=1), 2), (dict(k_fmt=7), 3), (dict(v_fmt=0), 3),
    (dict(k_flags=16), 3), (dict(k_fmt=0, k_flags=1), 3), (dict(k_fmt=0, k_flags=4), 3), (dict(k_data=None), 1),
    (dict(k_flags=10, k_basis=0x3000), 3), (dict(k_flags=9), 1), (dict(k_fmt=0, k_flags=8, k_basis=0x3000), 3),
    (dict(v_scales=None), 1),
    (dict(k_scales=None), 1), (dict(k_smooth=None), 1), (dict(k_inv_smooth=None), 1),
    (dict(global_scale=None), 1),
]


@pytest.mark.parametrize("bad,code", BAD_LAYERS)
def test_append_rejects_bad_layer(clib, bad, code):
    st = clib.nvkv_quantize_append_kv(ctypes.byref(_layer(**bad)), 0x10, 0x10, 0x10, 4, None)
    assert st == code, nk.last_error()
    assert nk.last_error()


def test_append_argument_errors(clib):
    L = _layer()
    assert clib.nvkv_quantize_append_kv(None, 0x10, 0x10, 0x10, 4, None) == 1
    assert clib.nvkv_quantize_append_kv(ctypes.byref(L), None, 0x10, 0x10, 4, None) == 1
    assert clib.nvkv_quantize_append_kv(ctypes.byref(L), 0x10, 0x10, None, 4, None) == 1
    assert clib.nvkv_quantize_append_kv(ctypes.byref(L), 0x10, 0x10, 0x10, -1, None) == 2
    assert clib.nvkv_quantize_append_kv(ctypes.byref(L), None, None, None, 0, None) == 0   # N = 0: no-op


def test_decode_argument_errors(clib):
    L = _layer()
    f = clib.nvkv_decode_attention_nvfp4
    ok = dict(q=0x10, B=4, Hq=32, pt=0x10, mp=4, sl=0x10, msl=64, sm=0.1, out=0x10, ws=0x1000, wsb=1 << 30, sp=0)
    def call(**kw):
        a = dict(ok, **kw)
        return f(ctypes.byref(L), a["q"], a["B"], a["Hq"], a["pt"], a["mp"], a["sl"], a["msl"], a["sm"], a["out"],
                 a["ws"], a["wsb"], a["sp"], None)
    assert call(q=None) == 1 and call(pt=None) == 1 and call(sl=None) == 1 and call(out=None) == 1
    assert call(B=0) == 2 and call(B=70000) == 2
    assert call(Hq=30) == 2                     # not a multiple of Hkv
    assert call(Hq=16) == 3                     # group of 2: unsupported
    assert call(mp=0) == 2 and call(msl=-1) == 2
    assert call(sp=48) == 2 and call(sp=-32) == 2
    assert call(sm=float("inf")) == 2
    need = nk.decode_workspace_bytes(4, 32, 8, 4096, 32)
    assert need > 0
    assert call(msl=4096, sp=32, ws=None) == 4
    assert call(msl=4096, sp=32, wsb=need - 1) == 4
    assert call(msl=4096, sp=32, ws=0x1010) == 4      # misaligned
    assert nk.decode_workspace_bytes(4, 32, 8, 64, 64) == 0     # single split: none needed
    assert nk.decode_workspace_bytes(4, 30, 8, 64, 0) == 0      # invalid
    assert f(None, 0x10, 4, 32, 0x10, 4, 0x10, 64, 0.1, 0x10, None, 0, 0, None) == 1


def test_decode_append_argument_errors(clib):
    """The fused append+decode entry point validates like decode, plus k_new / v_new."""
    L = _layer()
    f = clib.nvkv_decode_append_attention_nvfp4
    ok = dict(q=0x10, kn=0x10, vn=0x10, B=4, Hq=32, pt=0x10, mp=4, sl=0x10, msl=64, sm=0.1, out=0x10, ws=0x1000,
              wsb=1 << 30, sp=0)
    def call(lay=L, **kw):
        a = dict(ok, **kw)
        return f(ctypes.byref(lay) if lay is not None else None, a["q"], a["kn"], a["vn"], a["B"], a["Hq"], a["pt"],
                 a["mp"], a["sl"], a["msl"], a["sm"], a["out"], a["ws"], a["wsb"], a["sp"], None)
    assert call(lay=None) == 1
    assert call(kn=None) == 1 and call(vn=None) == 1 and call(q=None) == 1 and call(out=None) == 1
    assert call(B=0) == 2 and call(Hq=16) == 3 and call(sp=48) == 2 and call(sm=float("nan")) == 2
    need = nk.decode_workspace_bytes(4, 32, 8, 4096, 32)
    assert call(msl=4096, sp=32, wsb=need - 1) == 4
    assert call(lay=_layer(k_fmt=7)) == 3


def test_decode_append_noalloc_argument_errors(clib):
    """The allocation-free fused step validates like the fused step, and rejects calls whose
    split state exceeds its static scratch (B * Hkv <= 2048, at most 7 MiB of partials)
    before any HIP call."""
    L = _layer()
    f = clib.nvkv_decode_append_attention_nvfp4_noalloc
    ok = dict(q=0x10, kn=0x10, vn=0x10, B=4, Hq=32, pt=0x10, mp=4, sl=0x10, msl=64, sm=0.1, out=0x10, sp=0)
    def call(lay=L, **kw):
        a = dict(ok, **kw)
        return f(ctypes.byref(lay) if lay is not None else None, a["q"], a["kn"], a["vn"], a["B"], a["Hq"], a["pt"],
                 a["mp"], a["sl"], a["msl"], a["sm"], a["out"], a["sp"], None)
    assert call(lay=None) == 1
    assert call(kn=None) == 1 and call(vn=None) == 1 and call(q=None) == 1 and call(out=None) == 1
    assert call(B=0) == 2 and call(Hq=16) == 3 and call(sp=48) == 2 and call(sm=float("nan")) == 2
    assert call(lay=_layer(k_fmt=7)) == 3
    # 257 x 8 = 2056 (sequence, KV head) units with two splits each: more counters than the scratch holds
    assert call(B=257, msl=64, sp=32, mp=4) == 4
    # 64 x 8 units x 1024 splits x 4 heads x 520 B of partials: far beyond 7 MiB
    assert call(B=64, msl=32768, sp=32, mp=2048) == 4
    assert "static scratch" in nk.last_error()


def test_prefill_attention_argument_errors(clib):
    """The causal prefill-attention entry point validates its arguments before any launch;
    Tq = 0 is a no-op."""
    L = _layer()
    f = clib.nvkv_prefill_attention_nvfp4
    ok = dict(q=0x10, B=4, Tq=64, Hq=32, pt=0x10, mp=4, sl=0x10, msl=64, sm=0.1, out=0x10)
    def call(lay=L, **kw):
        a = dict(ok, **kw)
        return f(ctypes.byref(lay) if lay is not None else None, a["q"], a["B"], a["Tq"], a["Hq"], a["pt"], a["mp"],
                 a["sl"], a["msl"], a["sm"], a["out"], None)
    assert call(lay=None) == 1
    assert call(q=None) == 1 and call(out=None) == 1 and call(pt=None) == 1 and call(sl=None) == 1
    assert call(B=0) == 2 and call(B=70000) == 2 and call(Tq=-1) == 2 and call(Hq=12) == 2
    assert call(Hq=16) == 3 and call(mp=0) == 2 and call(msl=-1) == 2 and call(sm=float("inf")) == 2
    assert call(lay=_layer(k_fmt=7)) == 3 and call(lay=_layer(page_size=24)) == 2
    assert call(Tq=0, q=None, out=None) == 0          # nothing to do, nothing launched


def test_calibrate_argument_errors(clib):
    f = clib.nvkv_calibrate_key_smoothing
    assert f(None, None, 4, 8, 2, 1, 1, 0x10, 0x10, 0x10, None) == 1
    assert f(0x10, None, 4, 8, 2, 1, 1, None, 0x10, 0x10, None) == 1
    assert f(0x10, None, 4, 8, 2, 1, 1, 0x10, 0x10, None, None) == 1
    assert f(0x10, None, 0, 8, 2, 1, 1, 0x10, 0x10, 0x10, None) == 2
    assert f(0x10, None, 4, 0, 2, 1, 1, 0x10, 0x10, 0x10, None) == 2
    assert f(0x10, None, 4, 8, 0, 1, 1, 0x10, 0x10, 0x10, None) == 2
    assert f(0x10, None, 4, 8, 2, 1, 16, 0x10, 0x10, 0x10, None) == 3
    assert f(0x10, None, 4, 8, 2, 1, 10, 0x10, 0x10, 0x10, None) == 3
    assert f(0x10, None, 4, 1 << 28, 8, 1, 1, 0x10, 0x10, 0x10, None) == 2


def test_calibrate_key_basis_argument_errors(clib):
    f = clib.nvkv_calibrate_key_basis
    wsb = clib.nvkv_calibrate_key_basis_workspace_bytes(2)
    assert wsb == 2 * 128 * 128 * 8 * 2
    assert clib.nvkv_calibrate_key_basis_workspace_bytes(0) == 0
    ws = 0x100000
    assert f(None, 4, 8, 2, 1, 9, 0x10, 0x10, 0x10, ws, wsb, None) == 1          # k_win
    assert f(0x10, 4, 8, 2, 1, 9, 0x10, None, 0x10, ws, wsb, None) == 1          # basis_out
    assert f(0x10, 4, 8, 2, 1, 9, 0x10, 0x10, None, ws, wsb, None) == 1          # g_out
    assert f(0x10, 4, 8, 2, 1, 9, None, 0x10, 0x10, ws, wsb, None) == 1          # r with smoothing
    assert f(0x10, 0, 8, 2, 1, 9, 0x10, 0x10, 0x10, ws, wsb, None) == 2
    assert f(0x10, 4, 1, 2, 1, 9, 0x10, 0x10, 0x10, ws, wsb, None) == 2          # T >= 2
    assert f(0x10, 4, 8, 0, 1, 9, 0x10, 0x10, 0x10, ws, wsb, None) == 2
    assert f(0x10, 4, 8, 2, 1, 1, 0x10, 0x10, 0x10, ws, wsb, None) == 3          # no KLT bit
    assert f(0x10, 4, 8, 2, 1, 10, 0x10, 0x10, 0x10, ws, wsb, None) == 3         # with Hadamard
    assert f(0x10, 4, 8, 2, 1, 24, 0x10, 0x10, 0x10, ws, wsb, None) == 3         # unknown bit
    assert f(0x10, 4, 8, 2, 1, 9, 0x10, 0x10, 0x10, None, wsb, None) == 4        # workspace
    assert f(0x10, 4, 8, 2, 1, 9, 0x10, 0x10, 0x10, ws, wsb - 1, None) == 4
    assert f(0x10, 4, 8, 2, 1, 9, 0x10, 0x10, 0x10, ws + 16, wsb, None) == 4     # alignment


def test_product_path_has_no_fallback(tmp_path):
    """Loading a missing library raises instead of falling back to anything else."""
    import importlib
    import nvfp4_bit_kv_amd._native as native
    saved = native._lib
    try:
        native._lib = None
        with pytest.raises(ImportError):
            native.load(str(tmp_path / "missing.so"))
    finally:
        native._lib = saved
