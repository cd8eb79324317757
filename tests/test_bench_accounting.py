"""Byte accounting of the decode-step bench line (CPU only: plain arithmetic).

The step's algorithmic bytes are, per layer, one pass over the cache (144 B per (token, KV
head) for K+V NVFP4: 64 B codes + 8 B scales each), the bf16 query in and the fp32 output out,
and the append of each sequence's new token (bf16 K and V rows in, their cache rows out).  The
fused launch carries both, so the step is exactly the layer count times one fused launch; the
two-call form moves the same bytes.  Sizes follow the rstation.ai cache post's closing "For
scale" paragraph (Qwen3-8B shape: 8 KV heads x 128, 36 layers).
"""
import bench


def test_fused_step_is_layers_times_launch():
    B, T, hkv, hq, L = 4, 2304, 8, 32, 36
    for k_fmt in (0, 1):
        launch = bench.decode_launch_bytes(B, T, hkv, hq, k_fmt, "fused")
        assert bench.decode_step_bytes(B, T, hkv, hq, k_fmt, L) == L * launch


def test_separate_calls_move_the_same_bytes():
    B, T, hkv, hq, L = 4, 2304, 8, 32, 36
    dec = bench.decode_launch_bytes(B, T, hkv, hq, 1, "decode")
    app = bench.append_bytes(B, hkv, 1)
    assert bench.decode_step_bytes(B, T, hkv, hq, 1, L) == L * (dec + app)
    assert dec == bench.decode_bytes(B, T, hkv, hq, 1)


def test_step36_figures():
    # cache: 4 x 8 x 2304 x 144 B; query + output: 4 x 32 x (256 + 512) B
    assert bench.decode_bytes(4, 2304, 8, 32, 1) == 10_616_832 + 98_304
    # append: 4 x 8 x (256 + 72 + 256 + 72) B
    assert bench.append_bytes(4, 8, 1) == 20_992
    assert bench.decode_launch_bytes(4, 2304, 8, 32, 1, "fused") == 10_736_128
    assert bench.decode_step_bytes(4, 2304, 8, 32, 1, 36) == 386_500_608
    # bf16 keys: 256 B key rows
    assert bench.decode_bytes(4, 2304, 8, 32, 0) == 4 * 8 * 2304 * (256 + 72) + 98_304


def test_measurement_library_exports_and_plan():
    """The bench's measurement helpers (libnvkv_bench.so: streaming read, phase-stamped decode)
    load without a GPU, export their three calls, and report the library's own split plan:
    batch 4 x 2304 over 8 KV heads -> 8 splits of 288 tokens, 9 cache wavefronts + 1 append."""
    import ctypes
    lib = bench.bench_lib()
    for name in ("nvkvb_stream_read", "nvkvb_decode_plan", "nvkvb_decode_trace"):
        assert hasattr(lib, name)
    out = (ctypes.c_int32 * 3)()
    lib.nvkvb_decode_plan(4, 8, 2304, 0, 1, out)
    assert list(out) == [8, 10, 0]
    lib.nvkvb_decode_plan(64, 8, 32768, 0, 1, out)
    assert list(out) == [1, 8, 1]
