#!/usr/bin/env python3
"""Benchmark of the NVFP4 KV-cache hot path on one MI355X.

Default workload ("step36"): one decode step of a Qwen3-8B-shaped attention cache.
  - shape: 36 layers x 8 KV heads x head_dim 128, 32 query heads, batch 4 x 2304 cached
    tokens, 16-token pages with a shuffled page table;
  - cache: keys and values NVFP4, static per-channel key smoothing;
  - a step runs, for every layer, one decode_append_attention_nvfp4 call: the new token of
    each sequence is quantised and packed into the cache and attention runs over all 2304
    tokens (quantise -> pack -> split-K decode -> merge) in one launch; --separate times the
    same step as quantize_append_kv + decode_attention_nvfp4 per layer (also reported);
  - steps replay HIP graphs over 4 rotating copies of the 36-layer cache (1.5 GB, beyond the
    256 MB last-level cache).
Other workloads (run by hand with --workload):
  - step36-vonly, step36-hadamard, step36-had-smooth, step36-mse, step36-klt: the same step
    with other cache formats (MSE-searched key block scales; the static per-head KLT basis);
  - long: decode step at batch 64 x 32768 context (87 GB packed cache);
  - prefill, prefill-hadamard, prefill-mse, prefill-klt: quantize_append_kv of 16 x 8192 new
    tokens into each of 36 paged layers;
  - prefill-attn: causal prefill attention of the 16 x 8192 positions over each of the 36
    layers' caches.

Printed: one JSON line with
  - the step throughput (algorithmic bytes / step time) and tokens/s;
  - the roofline of the dominant kernel: algorithmic bytes per launch / average launch time,
    from HIP events around graph replays on the launch stream;
  - the CPU oracle timed on a bounded sample of the same workload;
  - a sampled parity check of the timed configuration against the oracle.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "NVFP4-KV decode attention: achieved HBM GB/s (% of peak) and tokens/s"
HBM_PEAK_GBS = 8000.0
PAGE = 16
SM_SCALE = 1.0 / math.sqrt(128)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="step36",
                    help="step36 | step36-vonly | step36-hadamard | step36-had-smooth | step36-mse | step36-klt | "
                         "long | prefill | prefill-hadamard | prefill-mse | prefill-klt | prefill-attn")
    ap.add_argument("--copies", type=int, default=0, help="rotating cache copies (0: workload default)")
    ap.add_argument("--split-tokens", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-check", action="store_true")
    ap.add_argument("--sweep-splits", default="",
                    help="comma-separated split sizes: report the decode launch time of each")
    ap.add_argument("--profile-pass", action="store_true",
                    help="short run for rocprofv3: few steps, no CPU baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (5 times): the reference kernel for scaling "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE counts to bytes")
    ap.add_argument("--trace-phases", action="store_true",
                    help="decode workloads: also run the phase-stamped instance of the fused decode kernel "
                         "(libnvkv_bench.so) over one step and print its phase timeline")
    ap.add_argument("--trace-dump", default="",
                    help="with --trace-phases: also save the raw stamps (uint64 [layers][workgroups][48]) to this .npy file")
    ap.add_argument("--append-kernel", default="library", choices=("library", "rowwave"),
                    help="prefill workloads: time the library's quantize_append_kv (library) or the comparison "
                         "layout of one wavefront per (token, KV head) row (rowwave, libnvkv_bench.so; plain "
                         "and Hadamard key options only)")
    ap.add_argument("--no-stream-reference", action="store_true",
                    help="skip the plain streaming read of the same cache bytes (reference for stream_frac)")
    ap.add_argument("--separate", action="store_true",
                    help="decode step as two calls per layer (quantize_append_kv, then "
                         "decode_attention_nvfp4) instead of the fused decode_append_attention_nvfp4")
    return ap.parse_args()


VARIANTS = {
    "step36": dict(cfg="step36", k_fmt=1, flags=1, copies=4, label="K+V NVFP4, K smoothed"),
    "step36-vonly": dict(cfg="step36", k_fmt=0, flags=0, copies=4, label="K bf16, V NVFP4"),
    "step36-hadamard": dict(cfg="step36", k_fmt=1, flags=2, copies=4, label="K+V NVFP4, K Hadamard-128"),
    "step36-had-smooth": dict(cfg="step36", k_fmt=1, flags=3, copies=4,
                              label="K+V NVFP4, K smoothed + Hadamard-128"),
    "step36-mse": dict(cfg="step36", k_fmt=1, flags=5, copies=4,
                       label="K+V NVFP4, K smoothed, MSE-searched key scales"),
    "step36-klt": dict(cfg="step36", k_fmt=1, flags=9, copies=4,
                       label="K+V NVFP4, K smoothed + static per-head KLT basis"),
    "long": dict(cfg="long", k_fmt=1, flags=1, copies=1, label="K+V NVFP4, K smoothed"),
    "prefill": dict(cfg="prefill", k_fmt=1, flags=1, copies=1, label="K smoothed"),
    "prefill-hadamard": dict(cfg="prefill", k_fmt=1, flags=3, copies=1, label="K smoothed + Hadamard-128"),
    "prefill-mse": dict(cfg="prefill", k_fmt=1, flags=5, copies=1, label="K smoothed, MSE-searched key scales"),
    "prefill-klt": dict(cfg="prefill", k_fmt=1, flags=9, copies=1, label="K smoothed + static per-head KLT basis"),
    "prefill-attn": dict(cfg="prefill", k_fmt=1, flags=1, copies=1, label="K+V NVFP4, K smoothed",
                         attention=True),
}
MFMA_F16_PEAK_TFLOPS = 2500.0


def row_bytes(fmt):
    return 256 if fmt == 0 else 72


# Algorithmic bytes of the decode step (what the method must move at least once).
def decode_bytes(B, T, hkv, hq, k_fmt):
    """One decode over the cache: every cached K and V row with its scales once, the query
    (bf16) in and the output (fp32) out."""
    return B * hkv * T * (row_bytes(k_fmt) + 72) + B * hq * (256 + 512)


def append_bytes(B, hkv, k_fmt):
    """Appending the new token of each sequence: bf16 K and V rows in, their cache rows out."""
    return B * hkv * ((256 + row_bytes(k_fmt)) + (256 + 72))


def decode_launch_bytes(B, T, hkv, hq, k_fmt, mode):
    """One launch of the dominant kernel: the fused call (mode "fused") also appends the new
    token; otherwise the launch is the decode alone."""
    return decode_bytes(B, T, hkv, hq, k_fmt) + (append_bytes(B, hkv, k_fmt) if mode == "fused" else 0)


def decode_step_bytes(B, T, hkv, hq, k_fmt, layers):
    """One decode step: per layer the append of the new tokens and one decode, whether the
    two run as one fused launch or as two calls (the append is counted once)."""
    return layers * (decode_bytes(B, T, hkv, hq, k_fmt) + append_bytes(B, hkv, k_fmt))


def f32_of(torch, t):
    """bf16 torch tensor (host) -> fp32 numpy array of the same values."""
    from synth import kv_inputs as S
    return S.bf16_to_f32(t.contiguous().view(torch.int16).numpy().view(np.uint16))


def calib_windows_device(torch, S, c, l):
    kw = torch.cat([S.make_keys_device(c["kind"], c["cfg"], l, 1, c["Tw"], c["hkv"], role=S.ROLE_WIN0 + w)
                    for w in range(4)])
    vw = torch.cat([S.make_values_device(c["cfg"], l, 1, c["Tw"], c["hkv"], role=S.ROLE_WIN0 + 4 + w)
                    for w in range(4)])
    return kw, vw


def calibrate_device(torch, nk, kw, vw, Tw, hkv, flags):
    """The library's calibration of one layer on the device: s, r, g and, with the KLT flag,
    the key basis (which also sets g_K)."""
    s = torch.empty((hkv, 128), dtype=torch.float32, device="cuda")
    r = torch.empty_like(s)
    g = torch.empty(2, dtype=torch.float32, device="cuda")
    nk.calibrate_key_smoothing(kw, vw, 4, Tw, hkv, True, flags, s, r, g)
    basis = None
    if flags & nk.K_KLT:
        basis = torch.empty((hkv, 128, 128), dtype=torch.float32, device="cuda")
        wsb = nk.calibrate_key_basis_workspace_bytes(hkv)
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        nk.calibrate_key_basis(kw, 4, Tw, hkv, True, flags, r, basis, g, ws, wsb)
    return s, r, g, basis


def install_calibration(cache, s, r, g, basis):
    cache.smooth.copy_(s)
    cache.inv_smooth.copy_(r)
    cache.gscale.copy_(g)
    if basis is not None:
        cache.basis.copy_(basis)


class DecodeStep:
    """Decode-step workloads: per layer, append the new token of every sequence, then attend."""

    metric = METRIC

    def __init__(self, name, copies, split_tokens, fused=True):
        import torch
        import nvfp4_bit_kv_amd as nk
        from synth import kv_inputs as S
        self.torch, self.nk, self.S = torch, nk, S
        v = VARIANTS[name]
        c = S.CONFIGS[v["cfg"]]
        self.name, self.variant, self.c = name, v, c
        self.B, self.T, self.hkv, self.hq, self.L = c["B"], c["T"], c["hkv"], c["hq"], c["layers"]
        self.k_fmt, self.flags = v["k_fmt"], v["flags"]
        self.copies = copies or v["copies"]
        self.split_tokens = split_tokens
        self.mode = "fused" if fused else "separate"
        self.kernel_label = (
            "k_decode<append> (decode_append_attention_nvfp4: new-token quantise/append + split-K decode + "
            "in-kernel cross-split merge, one launch; for long splits the library issues k_quantize_append "
            "of the new tokens + k_decode), per layer" if fused else
            "k_decode (decode_attention_nvfp4: split-K decode + in-kernel cross-split merge), per layer")
        B, T, hkv = self.B, self.T, self.hkv
        self.pps = (T + PAGE - 1) // PAGE
        self.num_pages = B * self.pps
        rng = np.random.default_rng(1234)
        self.table_np = rng.permutation(self.num_pages).reshape(B, self.pps).astype(np.int32)
        dev = "cuda"
        self.table = torch.from_numpy(self.table_np).to(dev)
        t = np.arange(T)
        self.slots_np = (self.table_np[:, t // PAGE] * PAGE + t % PAGE).astype(np.int32)    # [B][T]
        self.seq_lens = torch.full((B,), T, dtype=torch.int32, device=dev)
        self.new_slots = torch.from_numpy(np.ascontiguousarray(self.slots_np[:, T - 1])).to(dev)
        self.caches = [[None] * self.L for _ in range(self.copies)]
        self.k_new, self.v_new, self.q = [], [], []
        self.out = torch.empty((self.L, B, self.hq, 128), dtype=torch.float32, device=dev)
        self.wsb = nk.decode_workspace_bytes(B, self.hq, hkv, T, split_tokens)
        self.ws = torch.zeros(max(self.wsb, 256), dtype=torch.uint8, device=dev)
        # sequences whose bf16 inputs are kept on the host for the oracle legs
        self.sample_b = list(range(B)) if B <= 4 else [0, B - 1]
        self._build()

    def _build(self):
        torch, nk, S = self.torch, self.nk, self.S
        c, B, T, hkv = self.c, self.B, self.T, self.hkv
        bc = max(1, min(B, (1 << 27) // (T * hkv * 128)))        # sequences per generation chunk
        for l in range(self.L):
            kw, vw = calib_windows_device(torch, S, c, l)
            s, r, g, basis = calibrate_device(torch, nk, kw, vw, c["Tw"], hkv, self.flags)
            layer_caches = []
            for cp in range(self.copies):
                cache = nk.CacheLayer(self.num_pages, PAGE, hkv, k_fmt=self.k_fmt, k_flags=self.flags)
                install_calibration(cache, s, r, g, basis)
                layer_caches.append((cache, cache.struct()))
            k_new = torch.empty((B, hkv, 128), dtype=torch.bfloat16, device="cuda")
            v_new = torch.empty_like(k_new)
            keep = {}
            for b0 in range(0, B, bc):
                b1 = min(B, b0 + bc)
                k = S.make_keys_device(c["kind"], c["cfg"], l, b1 - b0, T, hkv, seed_index=b0)
                v = S.make_values_device(c["cfg"], l, b1 - b0, T, hkv, seed_index=b0)
                n = (b1 - b0) * (T - 1)
                sl = torch.from_numpy(np.ascontiguousarray(self.slots_np[b0:b1, :T - 1]).reshape(-1)).cuda()
                kp, vp = k[:, :T - 1].contiguous(), v[:, :T - 1].contiguous()
                for cache, Ls in layer_caches:
                    nk.quantize_append_kv(Ls, kp, vp, sl, n)
                k_new[b0:b1] = k[:, T - 1]
                v_new[b0:b1] = v[:, T - 1]
                if l == 0:
                    for b in self.sample_b:
                        if b0 <= b < b1:
                            keep[b] = (k[b - b0].cpu(), v[b - b0].cpu())
                del k, v, kp, vp
            for cp in range(self.copies):
                self.caches[cp][l] = layer_caches[cp]
            self.k_new.append(k_new)
            self.v_new.append(v_new)
            self.q.append(S.make_queries_device(c["cfg"], l, B, self.hq))
            if l == 0:
                self.layer0 = (keep, kw.cpu(), vw.cpu())
            del kw, vw
            if self.L > 8 and (l + 1) % 6 == 0:
                torch.cuda.synchronize()
                print(f"[bench] built layer {l + 1}/{self.L}", file=sys.stderr, flush=True)
        torch.cuda.synchronize()

    # one layer of the hot path: append the new token, then attend over the whole cache
    # mode "fused": one decode_append_attention_nvfp4 call; "separate": quantize_append_kv of
    # the new token, then decode_attention_nvfp4; "decode": decode_attention_nvfp4 only
    def layer_step(self, cp, l, mode=None):
        nk = self.nk
        mode = mode or self.mode
        cache, Ls = self.caches[cp][l]
        if mode == "fused":
            nk.decode_append_attention_nvfp4(Ls, self.q[l], self.k_new[l], self.v_new[l], self.B, self.hq, self.table,
                                             self.pps, self.seq_lens, self.T, SM_SCALE, self.out[l], self.ws,
                                             self.wsb, self.split_tokens)
            return
        if mode == "separate":
            nk.quantize_append_kv(Ls, self.k_new[l], self.v_new[l], self.new_slots, self.B)
        nk.decode_attention_nvfp4(Ls, self.q[l], self.B, self.hq, self.table, self.pps, self.seq_lens, self.T,
                                  SM_SCALE, self.out[l], self.ws, self.wsb, self.split_tokens)

    def step(self, cp, mode=None):
        for l in range(self.L):
            self.layer_step(cp, l, mode)

    def snapshot(self):
        return self.out.clone()

    # algorithmic bytes (what the method must move)
    def decode_bytes(self):
        return decode_bytes(self.B, self.T, self.hkv, self.hq, self.k_fmt)

    def launch_bytes(self):
        return decode_launch_bytes(self.B, self.T, self.hkv, self.hq, self.k_fmt, self.mode)

    def append_bytes_per_layer(self):
        return append_bytes(self.B, self.hkv, self.k_fmt)

    def step_bytes(self):
        return decode_step_bytes(self.B, self.T, self.hkv, self.hq, self.k_fmt, self.L)

    def tokens_per_step(self):
        return self.B

    def launch_times(self, reps):
        return decode_launch_times(self.torch, self, reps, self.mode if self.mode == "fused" else "decode")

    def check(self):
        return decode_check_against_oracle(self)

    def cpu_baseline(self):
        return decode_cpu_baseline(self)

    def describe(self):
        c = self.c
        return (f"{self.name}: Qwen3-8B-shaped decode step, {c['layers']} layers x {c['hkv']} KV heads x 128, "
                f"{c['hq']} query heads, batch {c['B']} x {c['T']} context, 16-token paged cache, "
                f"{self.variant['label']}; per layer append 1 token + split-K decode")


class PrefillAppend:
    """Prefill workload: quantize_append_kv of B x T new tokens into each of the paged layers."""

    metric = "NVFP4-KV quantize/append: achieved HBM GB/s (% of peak) and tokens/s"
    kernel_label = "k_quantize_append (quantize_append_kv of batch 16 x 8192 new tokens), per layer"

    def __init__(self, name, append_kernel="library"):
        import torch
        import nvfp4_bit_kv_amd as nk
        from synth import kv_inputs as S
        self.torch, self.nk, self.S = torch, nk, S
        v = VARIANTS[name]
        c = S.CONFIGS[v["cfg"]]
        self.name, self.variant, self.c = name, v, c
        self.B, self.T, self.hkv, self.L = c["B"], c["T"], c["hkv"], c["layers"]
        self.flags = v["flags"]
        self.append_kernel = append_kernel
        if append_kernel == "rowwave":
            if self.flags & ~3:
                sys.exit("--append-kernel rowwave takes the plain and Hadamard key options only")
            self.kernel_label = ("k_append_rowwave (quantize_append_kv of batch 16 x 8192 new tokens, one "
                                 "wavefront per (token, KV head) row; comparison layout), per layer")
        self.copies = 1
        B, T, hkv = self.B, self.T, self.hkv
        self.pps = T // PAGE
        self.num_pages = B * self.pps
        rng = np.random.default_rng(4321)
        self.table_np = rng.permutation(self.num_pages).reshape(B, self.pps).astype(np.int32)
        t = np.arange(T)
        slots = (self.table_np[:, t // PAGE] * PAGE + t % PAGE).astype(np.int32)
        self.slots = torch.from_numpy(np.ascontiguousarray(slots.reshape(-1))).cuda()
        self.N = B * T
        self.caches, self.k, self.v = [], [], []
        for l in range(self.L):
            kw, vw = calib_windows_device(torch, S, c, l)
            cache = nk.CacheLayer(self.num_pages, PAGE, hkv, k_flags=self.flags)
            install_calibration(cache, *calibrate_device(torch, nk, kw, vw, c["Tw"], hkv, self.flags))
            self.caches.append((cache, cache.struct()))
            self.k.append(S.make_keys_device(c["kind"], c["cfg"], l, B, T, hkv).reshape(B * T, hkv, 128))
            self.v.append(S.make_values_device(c["cfg"], l, B, T, hkv).reshape(B * T, hkv, 128))
            if l == 0:
                self.layer0 = (kw.cpu(), vw.cpu())
        torch.cuda.synchronize()
        self._calib = None

    def step(self, cp):
        if self.append_kernel == "rowwave":
            lib, stream = bench_lib(), self.torch.cuda.current_stream().cuda_stream
            for l in range(self.L):
                cache, Ls = self.caches[l]
                st = lib.nvkvb_quantize_append_rowwave(Ls, self.k[l].data_ptr(), self.v[l].data_ptr(),
                                                       self.slots.data_ptr(), self.N, stream)
                if st != 0:
                    raise RuntimeError(f"row-wave append launch failed: {st}")
            return
        for l in range(self.L):
            cache, Ls = self.caches[l]
            self.nk.quantize_append_kv(Ls, self.k[l], self.v[l], self.slots, self.N)

    def snapshot(self):
        cache, _ = self.caches[0]
        return self.torch.cat([cache.k_data, cache.k_scales, cache.v_data, cache.v_scales])

    def launch_bytes(self):
        """One quantize_append_kv call: per (token, KV head) the bf16 K and V rows in
        (2 x 256 B) and their codes and scales out (2 x 72 B); the slot index per token."""
        return self.N * (self.hkv * 2 * (256 + 72) + 4)

    def step_bytes(self):
        return self.L * self.launch_bytes()

    def tokens_per_step(self):
        return self.N

    def launch_times(self, reps):
        """Average duration of one quantize_append_kv call: a HIP graph of the calls of all
        layers is replayed between HIP events on the launch stream, divided by the layer count."""
        torch = self.torch
        g = capture(torch, lambda: self.step(0))
        g.replay()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for r in range(reps):
            ev[r][0].record(stream)
            g.replay()
            ev[r][1].record(stream)
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in ev]) * 1e-3 / self.L

    def _oracle_calib(self):
        from oracle import nvfp4_oracle as O
        if self._calib is None:
            kw, vw = self.layer0
            kwf = f32_of(self.torch, kw)
            s, r, g = O.calibrate(kwf, f32_of(self.torch, vw), True, self.flags)
            basis = O.klt_basis(kwf, r, self.flags)[0] if self.flags & O.FLAG_KLT else None
            self._calib = (s, r, g, basis)
        return self._calib

    def _oracle_rows(self, rows):
        from oracle import nvfp4_oracle as O
        torch = self.torch
        s, r, g, basis = self._oracle_calib()
        k = f32_of(torch, self.k[0][rows].cpu())
        v = f32_of(torch, self.v[0][rows].cpu())
        kc, ks = O.quantize_keys(O.key_transform(k, r[None], self.flags, basis), g[0], self.flags)
        vc, vs = O.quantize_rows(v, g[1])
        return kc, ks, vc, vs

    def check(self):
        """Bit-exact comparison of sampled rows of layer 0 (first and last sequence, read back
        through the page table) and of the calibrated scales.  With the KLT basis the library's
        own basis (fp64 Jacobi) agrees with the oracle's (LAPACK) to rounding: g_K is compared
        to 1e-5 and at least 99 % of the key codes must be identical."""
        torch = self.torch
        cache, _ = self.caches[0]
        s, r, g, basis = self._oracle_calib()
        klt = basis is not None
        gg = cache.gscale.cpu().numpy()
        ok = bool(np.array_equal(cache.inv_smooth.cpu().numpy(), r) and gg[1] == g[1]
                  and (abs(float(gg[0]) - float(g[0])) <= 1e-5 * float(g[0]) if klt else gg[0] == g[0]))
        key_same = key_total = 0
        n_rows = 0
        # keys row-major; values quad-interleaved (word w of token t at ((t/4)*16 + w)*16 + (t%4)*4)
        vq = cache.v_data.view(self.num_pages, self.hkv, PAGE // 4, 16, 4, 4).permute(0, 1, 2, 4, 3, 5)
        views = (cache.k_data.view(self.num_pages, self.hkv, PAGE, 64),
                 cache.k_scales.view(self.num_pages, self.hkv, PAGE // 4, 8, 4),
                 vq.reshape(self.num_pages, self.hkv, PAGE, 64),
                 cache.v_scales.view(self.num_pages, self.hkv, PAGE // 4, 8, 4))
        t = np.arange(self.T)
        for b in (0, self.B - 1):
            want = self._oracle_rows(slice(b * self.T, (b + 1) * self.T))
            pg = torch.from_numpy(self.table_np[b][t // PAGE].astype(np.int64)).cuda()
            off = torch.from_numpy((t % PAGE).astype(np.int64)).cuda()
            got = (views[0][pg, :, off], views[1][pg, :, off // 4, :, off % 4],
                   views[2][pg, :, off], views[3][pg, :, off // 4, :, off % 4])
            for i, (gt, w) in enumerate(zip(got, want)):
                if klt and i < 2:                      # key codes and scales
                    key_same += int((gt.cpu().numpy() == w).sum())
                    key_total += w.size
                else:
                    ok &= bool(np.array_equal(gt.cpu().numpy(), w))
            n_rows += 2 * self.T * self.hkv
        out = dict(ok=ok, compared_rows=n_rows,
                   kind="bit-exact K/V codes and scales of layer 0, sequences 0 and last, and the calibration")
        if klt:
            frac = key_same / key_total
            out.update(ok=bool(ok and frac >= 0.99), key_bytes_identical=round(frac, 6),
                       kind="V codes/scales bit-exact; key bytes identical in >= 99 % (the library's own KLT "
                            "basis against the oracle's); g_K within 1e-5")
        return out

    def cpu_baseline(self, budget_s=12.0):
        """The oracle's key transform and NVFP4 quantisation of K and V on chunks of layer 0's
        new tokens (calibration done once beforehand, untimed), one BLAS thread, for a bounded
        time; the per-layer rate is divided by the layer count."""
        from threadpoolctl import threadpool_limits
        chunk = 1024
        with threadpool_limits(limits=1):
            self._oracle_calib()
            rows_done = 0
            t0 = time.perf_counter()
            while True:
                a = rows_done % (self.N - chunk)
                self._oracle_rows(slice(a, a + chunk))
                rows_done += chunk
                el = time.perf_counter() - t0
                if el >= budget_s:
                    break
        tok_s = rows_done / el
        return dict(value=round(tok_s / self.L, 2), unit="tokens/s", cores=1, kind="oracle",
                    sample=f"{rows_done} new tokens x {self.hkv} KV heads of layer 0 (key transform + NVFP4 "
                           f"quantisation of K and V) in {el:.1f} s on 1 core of "
                           f"{len(os.sched_getaffinity(0))}; per-layer rate divided by {self.L} layers",
                    oracle_effective_gbs=round(tok_s * self.launch_bytes() / self.N / 1e9, 6))

    def describe(self):
        c = self.c
        return (f"{self.name}: quantize_append_kv of batch {c['B']} x {c['T']} new tokens into each of "
                f"{c['layers']} layers x {c['hkv']} KV heads x 128, 16-token paged cache (shuffled pages), "
                f"{self.variant['label']}, K and V NVFP4")


class PrefillAttention:
    """Causal prefill attention: per layer, prefill_attention_nvfp4 of all B x T positions
    over the layer's cache of the same T tokens (a full teacher-forced window)."""

    metric = "NVFP4-KV causal prefill attention: achieved TFLOP/s (% of MFMA fp16 peak) and tokens/s"
    kernel_label = ("k_prefill_attn (prefill_attention_nvfp4: causal attention of batch 16 x 8192 positions over "
                    "the cache), per layer")
    roofline_bound = "mfma"
    protocol_runs = 3

    def __init__(self, name):
        import torch
        import nvfp4_bit_kv_amd as nk
        from synth import kv_inputs as S
        self.torch, self.nk, self.S = torch, nk, S
        v = VARIANTS[name]
        c = S.CONFIGS[v["cfg"]]
        self.name, self.variant, self.c = name, v, c
        self.B, self.T, self.hkv, self.hq, self.L = c["B"], c["T"], c["hkv"], c["hq"], c["layers"]
        self.flags = v["flags"]
        self.copies = 1
        B, T, hkv = self.B, self.T, self.hkv
        self.pps = T // PAGE
        self.num_pages = B * self.pps
        rng = np.random.default_rng(2468)
        self.table_np = rng.permutation(self.num_pages).reshape(B, self.pps).astype(np.int32)
        self.table = torch.from_numpy(self.table_np).cuda()
        t = np.arange(T)
        slots = (self.table_np[:, t // PAGE] * PAGE + t % PAGE).astype(np.int32)
        slots_dev = torch.from_numpy(np.ascontiguousarray(slots.reshape(-1))).cuda()
        self.seq_lens = torch.full((B,), T, dtype=torch.int32, device="cuda")
        self.caches, self.q = [], []
        self.sample_b = (0, B - 1)
        for l in range(self.L):
            kw, vw = calib_windows_device(torch, S, c, l)
            cache = nk.CacheLayer(self.num_pages, PAGE, hkv, k_flags=self.flags)
            install_calibration(cache, *calibrate_device(torch, nk, kw, vw, c["Tw"], hkv, self.flags))
            k = S.make_keys_device(c["kind"], c["cfg"], l, B, T, hkv)
            vv = S.make_values_device(c["cfg"], l, B, T, hkv)
            nk.quantize_append_kv(cache.struct(), k.reshape(B * T, hkv, 128), vv.reshape(B * T, hkv, 128),
                                  slots_dev, B * T)
            self.caches.append((cache, cache.struct()))
            self.q.append(S.make_query_block_device(c["cfg"], l, B, T, self.hq))
            if l == 0:
                self.layer0 = ({b: (k[b].cpu(), vv[b].cpu()) for b in self.sample_b}, kw.cpu(), vw.cpu())
            del k, vv
            if (l + 1) % 6 == 0:
                print(f"[bench] built layer {l + 1}/{self.L}", file=sys.stderr, flush=True)
        self.out = torch.empty((B, T, self.hq, 128), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        self._oracle = None

    def step(self, cp):
        for l in range(self.L):
            self.nk.prefill_attention_nvfp4(self.caches[l][1], self.q[l], self.B, self.T, self.hq, self.table,
                                            self.pps, self.seq_lens, self.T, SM_SCALE, self.out)

    def snapshot(self):
        return self.out.clone()

    def launch_flops(self):
        """Algorithmic flops of one call: QK and PV, 2 flops per multiply-add, over the causal
        (position, key) pairs: 4 * 128 * Hq * B * T (T + 1) / 2.  The exact-operand term splits
        (two fp16 query terms, two P terms) double the MFMA work actually issued; they are not
        counted."""
        return 4 * 128 * self.hq * self.B * self.T * (self.T + 1) // 2

    def step_flops(self):
        return self.L * self.launch_flops()

    def launch_bytes(self):
        """Cache bytes one call must read at least once (144 B per (token, KV head)) plus the
        queries in and the outputs out."""
        return self.B * self.T * (self.hkv * 144 + self.hq * 128 * (2 + 4))

    def step_bytes(self):
        return self.L * self.launch_bytes()

    def tokens_per_step(self):
        return self.B * self.T

    def launch_times(self, reps):
        """Average duration of one call: a HIP graph of the calls of all layers replayed
        between HIP events on the launch stream, divided by the layer count."""
        torch = self.torch
        g = capture(torch, lambda: self.step(0))
        g.replay()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for r in range(reps):
            ev[r][0].record(stream)
            g.replay()
            ev[r][1].record(stream)
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in ev]) * 1e-3 / self.L

    def _oracle_inputs(self):
        """Oracle calibration and dequantised cache of layer 0 for the sampled sequences, from
        the same bf16 inputs as the GPU path."""
        from oracle import nvfp4_oracle as O
        if self._oracle is None:
            torch = self.torch
            keep, kw, vw = self.layer0
            s, r, g = O.calibrate(f32_of(torch, kw), f32_of(torch, vw), True, self.flags)
            seqs = {}
            for b in self.sample_b:
                kf, vf = f32_of(torch, keep[b][0]), f32_of(torch, keep[b][1])
                kc, ks = O.quantize_keys(O.key_transform(kf, r[None], self.flags), g[0], self.flags)
                vc, vs = O.quantize_rows(vf, g[1])
                seqs[b] = (O.dequantize(kc, ks, g[0]), O.dequantize(vc, vs, g[1]))
            self._oracle = (O, s, g, seqs)
        return self._oracle

    def _oracle_rows(self, b, positions):
        """Oracle causal attention of the given positions of sequence b (layer 0), each as the
        last position of a block of one."""
        O, s, g, seqs = self._oracle_inputs()
        khat, vhat = seqs[b]
        qf = f32_of(self.torch, self.q[0][b, positions].cpu()).astype(np.float64)     # [P][Hq][128]
        qp = O.query_transform(qf, np.repeat(s, self.hq // self.hkv, 0)[None], self.flags)
        return np.stack([O.causal_attention(qp[j][None, None], [khat], [vhat], [int(p) + 1], SM_SCALE)[0, 0]
                         for j, p in enumerate(positions)])

    def check(self):
        """Sampled rows of layer 0 (first and last sequence; first, tile-boundary, last and
        random positions, all 32 heads) against the oracle: max |err| <= 1e-3 max|V_hat| and
        per-row relative L2 <= 1e-4."""
        torch = self.torch
        self.nk.prefill_attention_nvfp4(self.caches[0][1], self.q[0], self.B, self.T, self.hq, self.table,
                                        self.pps, self.seq_lens, self.T, SM_SCALE, self.out)
        torch.cuda.synchronize()
        rng = np.random.default_rng(77)
        positions = sorted(set([0, 1, 7, 8, 511, self.T // 2, self.T - 1] + list(rng.integers(0, self.T, 5))))
        O, s, g, seqs = self._oracle_inputs()
        ok, max_abs, max_rel = True, 0.0, 0.0
        for b in self.sample_b:
            got = self.out[b, positions].cpu().numpy().astype(np.float64)
            ref = self._oracle_rows(b, positions)
            vmax = float(np.abs(seqs[b][1]).max())
            err = float(np.abs(got - ref).max())
            rel = float((np.linalg.norm(got - ref, axis=-1) / np.maximum(np.linalg.norm(ref, axis=-1), 1e-30)).max())
            max_abs, max_rel = max(max_abs, err / vmax), max(max_rel, rel)
            ok &= bool(np.all(np.isfinite(got)) and err <= 1e-3 * vmax and rel <= 1e-4)
        return dict(ok=ok, sequences=list(self.sample_b), positions=[int(p) for p in positions],
                    max_abs_err_over_vmax=max_abs, max_rel_l2=max_rel,
                    tol="max|err| <= 1e-3 max|Vhat|, rel L2 <= 1e-4")

    def cpu_baseline(self, budget_s=12.0):
        """The oracle (query transform and fp64 causal attention over the dequantised cache of
        layer 0, calibration and dequantisation done once beforehand, untimed) on random query
        positions of sequence 0, all 32 heads, one BLAS thread, for a bounded time; positions
        per second scaled by the mean causal length, divided by the layer count."""
        from threadpoolctl import threadpool_limits
        rng = np.random.default_rng(5)
        with threadpool_limits(limits=1):
            self._oracle_inputs()
            done, pairs = 0, 0
            t0 = time.perf_counter()
            while True:
                pos = int(rng.integers(0, self.T))
                self._oracle_rows(0, [pos])
                done += 1
                pairs += pos + 1
                el = time.perf_counter() - t0
                if el >= budget_s:
                    break
        # full-window tokens per second: the oracle's (position, key) pair rate over the
        # window's T (T + 1) / 2 pairs per sequence
        pair_rate = pairs / el
        tok_s = pair_rate / (self.T * (self.T + 1) / 2) * self.T
        return dict(value=round(tok_s / self.L, 4), unit="tokens/s", cores=1, kind="oracle",
                    sample=f"{done} random query positions of sequence 0, layer 0, all {self.hq} heads "
                           f"({pairs} causal (position, key) pairs) in {el:.1f} s on 1 core of "
                           f"{len(os.sched_getaffinity(0))}; scaled to full {self.T}-position windows and "
                           f"divided by {self.L} layers",
                    oracle_tflops=round(pair_rate * 4 * 128 * self.hq / 1e12, 6))

    def describe(self):
        c = self.c
        return (f"{self.name}: causal prefill attention of batch {c['B']} x {c['T']} positions (full window) "
                f"over each of {c['layers']} layers' 16-token paged NVFP4 cache (shuffled pages), "
                f"{c['hkv']} KV heads x 128, {c['hq']} query heads, {self.variant['label']}")


def capture(torch, fn):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def time_graphs(torch, graphs, steps, warmup):
    for i in range(warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        graphs[i % len(graphs)].replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


def decode_launch_times(torch, wl, reps, mode="decode"):
    """Average duration of one decode launch (the kernel back to back, no host gaps): a HIP
    graph of the calls of all layers of a cache copy is replayed between two HIP events on
    the launch stream; one sample per replay, divided by the layer count."""
    graphs = [capture(torch, lambda cp=cp: [wl.layer_step(cp, l, mode) for l in range(wl.L)])
              for cp in range(wl.copies)]
    for gr in graphs:
        gr.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for r in range(reps):
        ev[r][0].record(stream)
        graphs[r % len(graphs)].replay()
        ev[r][1].record(stream)
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in ev]) * 1e-3 / wl.L     # seconds per call


def sweep_splits(torch, wl, splits):
    """Average decode launch time per split size (tuning aid, printed to stderr)."""
    saved = (wl.split_tokens, wl.wsb, wl.ws)
    res = {}
    for sp in splits:
        wl.split_tokens = sp
        wl.wsb = wl.nk.decode_workspace_bytes(wl.B, wl.hq, wl.hkv, wl.T, sp)
        wl.ws = torch.zeros(max(wl.wsb, 256), dtype=torch.uint8, device="cuda")
        d = decode_launch_times(torch, wl, reps=10, mode=wl.mode if wl.mode == "fused" else "decode")
        res[sp] = (float(np.mean(d)) * 1e6, float(np.min(d)) * 1e6)
        print(f"[sweep] split_tokens={sp}: avg {res[sp][0]:.2f} us  min {res[sp][1]:.2f} us  "
              f"-> {wl.launch_bytes() / np.mean(d) / 1e9:.0f} GB/s", file=sys.stderr, flush=True)
    wl.split_tokens, wl.wsb, wl.ws = saved
    return res


def _oracle_decode_inputs(wl):
    """Oracle calibration, query and per-sequence codes for layer 0, from the same bf16 inputs
    as the GPU path; computed once and kept (the codes are row-wise, so the codes of the first
    T-1 rows are a prefix of those of all T rows)."""
    from oracle import nvfp4_oracle as O
    if getattr(wl, "_oracle", None) is None:
        torch = wl.torch
        keep, kw, vw = wl.layer0
        kwf = f32_of(torch, kw)
        s, r, g = O.calibrate(kwf, f32_of(torch, vw), True, wl.flags)
        basis = O.klt_basis(kwf, r, wl.flags)[0] if wl.flags & O.FLAG_KLT else None
        qf = f32_of(torch, wl.q[0].cpu()).astype(np.float64)
        seqs = {}
        for b in wl.sample_b:
            kf, vf = f32_of(torch, keep[b][0]), f32_of(torch, keep[b][1])
            kc = ks = None
            if wl.k_fmt == 1:
                kc, ks = O.quantize_keys(O.key_transform(kf, r[None], wl.flags, basis), g[0], wl.flags)
            vc, vs = O.quantize_rows(vf, g[1])
            seqs[b] = (kf, vf, (kc, ks, vc, vs))
        wl._oracle = (s, r, g, qf, seqs, basis)
    return (O,) + wl._oracle


def _oracle_sequence(O, wl, s, r, g, qf, kf, vf, b, codes, append_last, basis=None):
    """Oracle decode of one sequence: the codes of its T cached rows (with append_last, the
    codes of the first T-1 rows plus the appended row quantised here), dequantisation and fp64
    attention for every query head."""
    T, hq, hkv = wl.T, wl.hq, wl.hkv
    kc, ks, vc, vs = codes
    if append_last:
        if wl.k_fmt == 1:
            nkc, nks = O.quantize_keys(O.key_transform(kf[T - 1:], r[None], wl.flags, basis), g[0], wl.flags)
            kc, ks = np.concatenate([kc[:T - 1], nkc]), np.concatenate([ks[:T - 1], nks])
        nvc, nvs = O.quantize_rows(vf[T - 1:], g[1])
        vc, vs = np.concatenate([vc[:T - 1], nvc]), np.concatenate([vs[:T - 1], nvs])
    if wl.k_fmt == 1:
        khat = O.dequantize(kc, ks, g[0])
        qp = O.query_transform(qf[b:b + 1], np.repeat(s, hq // hkv, 0)[None], wl.flags,
                               None if basis is None else np.repeat(basis, hq // hkv, 0)[None])
    else:
        khat = kf.astype(np.float64)
        qp = qf[b:b + 1]
    vhat = O.dequantize(vc, vs, g[1])
    return O.attention(qp, [khat], [vhat], [T], SM_SCALE)[0], vhat


def decode_check_against_oracle(wl):
    """Sampled parity of the timed configuration: layer 0, the sampled sequences, every query
    head, against the oracle built from the same bf16 inputs (calibration included)."""
    O, s, r, g, qf, seqs, basis = _oracle_decode_inputs(wl)
    got_all = wl.out[0].cpu().numpy().astype(np.float64)
    worst_err = worst_rel = 0.0
    ok = True
    # with the KLT basis the library calibrates its own basis (fp64 Jacobi), which agrees with
    # the oracle's (LAPACK) to rounding: end to end, held to the same bar
    klt = basis is not None
    atol, rtol = 1e-3, 1e-4
    for b in wl.sample_b:
        kf, vf, codes = seqs[b]
        ref, vhat = _oracle_sequence(O, wl, s, r, g, qf, kf, vf, b, codes, append_last=False, basis=basis)
        got = got_all[b]
        err = float(np.abs(got - ref).max())
        rel = float((np.linalg.norm(got - ref, axis=-1) / np.linalg.norm(ref, axis=-1)).max())
        ok &= err <= atol * float(np.abs(vhat).max()) and rel <= rtol
        worst_err, worst_rel = max(worst_err, err), max(worst_rel, rel)
    tol = f"max|err| <= {atol:g} max|Vhat|, rel L2 <= {rtol:g}"
    if klt:
        tol += " (end to end: the library's own calibrated KLT basis against the oracle's)"
    return dict(ok=bool(ok), sequences=wl.sample_b, max_abs_err=worst_err, max_rel_l2=worst_rel, tol=tol)


def decode_cpu_baseline(wl, budget_s=12.0):
    """The oracle as it stands on a bounded sample: per (layer-0 sequence) unit, quantise the
    new token, dequantise the cache and run fp64 attention for every query head (the codes of
    the T-1 cached rows are built beforehand, untimed).  BLAS is held to one thread.
    Extrapolated to all sequences and layers of the step."""
    from threadpoolctl import threadpool_limits
    B, T, hq, hkv = wl.B, wl.T, wl.hq, wl.hkv
    with threadpool_limits(limits=1):
        O, s, r, g, qf, seqs, basis = _oracle_decode_inputs(wl)
        units = 0
        t0 = time.perf_counter()
        while True:
            for b in wl.sample_b:
                kf, vf, codes = seqs[b]
                _oracle_sequence(O, wl, s, r, g, qf, kf, vf, b, codes, append_last=True, basis=basis)
                units += 1
            el = time.perf_counter() - t0
            if el >= budget_s or units >= B * wl.L:
                break
    step_s = el / units * B * wl.L
    return dict(value=round(B / step_s, 4), unit="tokens/s", cores=1, kind="oracle",
                sample=f"{units} x (one sequence of layer 0: append 1 token + dequantise {T} tokens x {hkv} KV "
                       f"heads + fp64 attention for {hq} query heads), {el:.1f} s on 1 core of "
                       f"{len(os.sched_getaffinity(0))}, extrapolated to {B} sequences x {wl.L} layers",
                oracle_step_s=round(step_s, 3),
                oracle_effective_gbs=round(wl.step_bytes() / step_s / 1e9, 6))


# ---------------------------------------------------------------------------------------
# Measurement helpers (libnvkv_bench.so: a plain streaming-read kernel and the phase-stamped
# decode instance; not the library's C ABI)
# ---------------------------------------------------------------------------------------
_BENCH_LIB = None


def bench_lib():
    global _BENCH_LIB
    if _BENCH_LIB is None:
        import ctypes
        path = os.path.join(ROOT, "nvfp4_bit_kv_amd", "libnvkv_bench.so")
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: build with `python -m nvfp4_bit_kv_amd.build`")
        lib = ctypes.CDLL(path)
        vp, i32, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
        lib.nvkvb_stream_read.argtypes = [vp, vp, ctypes.c_int, vp, ctypes.c_int, vp]
        lib.nvkvb_stream_read.restype = ctypes.c_int
        lib.nvkvb_decode_plan.argtypes = [i32, i32, i32, i32, i32, vp]
        lib.nvkvb_decode_plan.restype = None
        from nvfp4_bit_kv_amd import Layer
        lib.nvkvb_decode_trace.argtypes = [ctypes.POINTER(Layer), vp, vp, vp, i32, i32, i32, vp, i32, vp, i32, f32,
                                           vp, vp, i32, vp, vp]
        lib.nvkvb_decode_trace.restype = ctypes.c_int
        lib.nvkvb_quantize_append_rowwave.argtypes = [ctypes.POINTER(Layer), vp, vp, vp, i32, vp]
        lib.nvkvb_quantize_append_rowwave.restype = ctypes.c_int
        _BENCH_LIB = lib
    return _BENCH_LIB


def stream_reference(torch, wl, reps=10, grids=(256, 512, 1024, 2048)):
    """A plain streaming read of exactly the cache arrays one decode launch reads (codes and
    scales of K and V of the layer), as a graph of one launch per layer and cache copy replayed
    between HIP events; the fastest of a few grid sizes.  Returns (seconds per launch, bytes per
    launch, grid)."""
    import ctypes
    lib = bench_lib()
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    best = None
    for grid in grids:
        keep = []

        def launch_all(cp, grid=grid):
            for l in range(wl.L):
                cache, _ = wl.caches[cp][l]
                arrs = [t for t in (cache.k_data, cache.k_scales, cache.v_data, cache.v_scales) if t is not None]
                ptrs = (ctypes.c_void_p * len(arrs))(*[t.data_ptr() for t in arrs])
                sizes = (ctypes.c_size_t * len(arrs))(*[t.numel() * t.element_size() for t in arrs])
                keep.append((ptrs, sizes))
                st = lib.nvkvb_stream_read(ptrs, sizes, len(arrs), sink.data_ptr(), grid,
                                           torch.cuda.current_stream().cuda_stream)
                if st != 0:
                    raise RuntimeError(f"stream read launch failed: {st}")
        graphs = [capture(torch, lambda cp=cp: launch_all(cp)) for cp in range(wl.copies)]
        for gr in graphs:
            gr.replay()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for r in range(reps):
            ev[r][0].record(stream)
            graphs[r % len(graphs)].replay()
            ev[r][1].record(stream)
        torch.cuda.synchronize()
        t = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e-3 / wl.L
        if best is None or t < best[0]:
            best = (t, grid)
        del graphs
    cache, _ = wl.caches[0][0]
    nbytes = sum(t.numel() * t.element_size() for t in (cache.k_data, cache.k_scales, cache.v_data, cache.v_scales)
                 if t is not None)
    return best[0], nbytes, best[1]


TRACE_SLOTS = 48
TICK_US = 0.01            # s_memrealtime runs at 100 MHz


def trace_phases(torch, wl, dump=""):
    """Phase timeline of the fused decode launch: the phase-stamped instance of the kernel over
    all layers of cache copy 0, captured as one graph of back-to-back launches (as timed) and
    replayed twice; stamps of the second replay.  Reported per launch as medians over its
    workgroups (times in microseconds after the launch's first workgroup started, and
    per-workgroup durations of the phases), then the median and maximum over the launches."""
    import ctypes
    lib = bench_lib()
    fused = wl.mode == "fused"
    plan = (ctypes.c_int32 * 3)()
    lib.nvkvb_decode_plan(wl.B, wl.hkv, wl.T, wl.split_tokens, int(fused), plan)
    n_splits, waves, pipe2 = int(plan[0]), int(plan[1]), int(plan[2])
    if fused and pipe2:
        return {"skipped": "long splits: the fused call issues two launches"}
    n_wg = n_splits * wl.hkv * wl.B
    buf = torch.zeros((wl.L, n_wg, TRACE_SLOTS), dtype=torch.int64, device="cuda")

    def run():
        for l in range(wl.L):
            cache, Ls = wl.caches[0][l]
            st = lib.nvkvb_decode_trace(Ls, wl.q[l].data_ptr(), wl.k_new[l].data_ptr(), wl.v_new[l].data_ptr(),
                                        int(fused), wl.B, wl.hq, wl.table.data_ptr(), wl.pps, wl.seq_lens.data_ptr(),
                                        wl.T, SM_SCALE, wl.out[l].data_ptr(), wl.ws.data_ptr(), wl.split_tokens,
                                        buf[l].data_ptr(), torch.cuda.current_stream().cuda_stream)
            if st != 0:
                raise RuntimeError(f"traced decode launch failed: {st}")
    g = capture(torch, run)
    g.replay()
    g.replay()
    torch.cuda.synchronize()
    raw = buf.cpu().numpy().view(np.uint64)
    if dump:
        np.save(dump, raw)
    t = raw.astype(np.float64)                                         # [L][wg][slot]
    med = lambda x: float(np.nanmedian(x)) if np.isfinite(x).any() else np.nan
    rows = []
    for l in range(wl.L):
        tl = t[l]
        t0 = tl[:, 0].min()
        r = np.where(tl > 0, (tl - t0) * TICK_US, np.nan)
        merger = (tl[:, 7].astype(np.uint64) & np.uint64(1)) == 1
        data_first = np.nanmin(r[:, 16:32], axis=1)
        data_last = np.nanmax(r[:, 16:32], axis=1)
        done = np.nanmax(r[:, 32:48], axis=1)
        last = np.nanmax(np.where(np.isfinite(r[:, 6]), r[:, 6], r[:, 4]))
        rows.append(dict(
            first_wg_to_last_wg_start=np.nanmax(r[:, 0]),
            prologue_done=med(r[:, 1]), first_data=med(data_first), last_data=med(data_last),
            compute_done=med(done), compute_done_last_wg=np.nanmax(done),
            partials_issued=med(r[:, 8]), partials_acked=med(r[:, 3]), arrival_counted=med(r[:, 4]),
            merger_loaded=med(r[merger, 9]), merger_folded=med(r[merger, 5]), end=last,
            gap_to_next_launch=((t[l + 1][:, 0].min() - tl[:, 6].max()) * TICK_US if l + 1 < wl.L else np.nan),
            d_compute=med(done - data_last), d_workgroup_merge=med(r[:, 8] - done), d_store_ack=med(r[:, 3] - r[:, 8]),
            d_arrival=med(r[:, 4] - r[:, 3]), d_merger_load=med(r[merger, 9] - r[merger, 4]),
            d_merger_fold_store=med(r[merger, 6] - r[merger, 9]),
        ))
        if np.isfinite(r[:, 10]).any():     # the KLT basis stamps of wavefront 0
            rows[-1].update(basis_quarter_staged=med(r[:, 10]), basis_barrier=med(r[:, 11]),
                            query_transformed=med(r[:, 12]))
        own = np.isfinite(r[:, 13])          # the workgroups whose split holds the new token
        if own.any():
            rows[-1].update(new_token_begun=med(r[own, 13]), new_token_encoded=med(r[own, 14]),
                            new_token_folded_in=med(r[own, 15]), owner_partials_issued=med(r[own, 8]),
                            d_new_token_encode=med(r[own, 14] - r[own, 13]))
    out = {"launches": wl.L, "workgroups": n_wg, "waves_per_workgroup": waves, "n_splits": n_splits,
           "unit": "us; times after the first workgroup of the launch started, d_* are per-workgroup phase "
                   "durations (s_memrealtime, 100 MHz); medians over a launch's workgroups, then median and "
                   "max over launches"}
    for k in rows[0]:
        vals = np.array([r[k] for r in rows], dtype=np.float64)
        vals = vals[np.isfinite(vals)]
        out[k] = {"median": round(float(np.median(vals)), 3), "max": round(float(np.max(vals)), 3)} if vals.size else None
    return out


COPY_BYTES = 256 << 20


def copy_calibration(torch):
    """A plain device-to-device copy of 256 MiB, five times (reference kernel for the HBM
    byte counters: it reads and writes exactly COPY_BYTES per dispatch)."""
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"[bench] copy calibration: 5 x {COPY_BYTES} B device copies", file=sys.stderr, flush=True)


def kernel_source_hash():
    """sha256 over the sources of the decode, append and prefill-attention kernels and of the
    bench's own kernels (the counter records in profiles/ hold for this exact source)."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "nvfp4_bit_kv_amd", "csrc")
    for name in ("nvkv_decode.hip", "nvkv_encode.hpp", "nvkv_device.hpp", "nvkv_quantize.hip", "nvkv_tiles.hpp",
                 "nvkv_klt.hpp", "nvkv_prefill.hip", "nvkv_bench.hip"):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def profile_name(wl):
    """Name of the workload's records in profiles/: the workload name, with the append kernel
    appended when the bench times the comparison layout instead of the library's."""
    ak = getattr(wl, "append_kernel", "library")
    return wl.name if ak == "library" else f"{wl.name}-{ak}"


def traffic_per_launch(wl):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3 FETCH_SIZE +
    WRITE_SIZE summary of this workload, or None when there is none or the kernel sources
    changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{profile_name(wl)}.md")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        text = f.read()
    if "```json" not in text:
        return None
    rec = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    if rec.get("kernel_source_sha256") != kernel_source_hash() or rec.get("kernel") != wl.kernel_label:
        return None
    return rec.get("hbm_bytes_per_launch")


def sq_counters(wl):
    """VALU / MFMA activity of the dominant kernel from the committed rocprofv3 SQ-counter
    summary of this workload (profiles/sq_<workload>.md), or None when there is none or the
    kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"sq_{profile_name(wl)}.md")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        text = f.read()
    if "```json" not in text:
        return None
    rec = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    if rec.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return {k: rec[k] for k in ("valu_busy", "mfma_busy", "valu_insts_per_wave", "mfma_insts_per_wave") if k in rec}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1 "
                                   "(the sharding design is described in the design notes)"}))
        sys.exit(2)
    if args.workload not in VARIANTS:
        sys.exit(f"unknown workload {args.workload!r}; choose from {sorted(VARIANTS)}")
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.profile_pass:
        args.steps, args.warmup, args.no_cpu_baseline = min(args.steps, 20), min(args.warmup, 5), True
    print(f"[bench] building workload {args.workload}", file=sys.stderr, flush=True)
    if VARIANTS[args.workload].get("attention"):
        wl = PrefillAttention(args.workload)
    elif VARIANTS[args.workload]["cfg"] == "prefill":
        wl = PrefillAppend(args.workload, args.append_kernel)
    else:
        wl = DecodeStep(args.workload, args.copies, args.split_tokens, fused=not args.separate)

    # eager pass and its result, then one graph per cache copy
    wl.step(0)
    torch.cuda.synchronize()
    eager0 = wl.snapshot()
    graphs = [capture(torch, lambda cp=cp: wl.step(cp)) for cp in range(wl.copies)]
    print(f"[bench] captured {len(graphs)} step graphs; timing {args.steps} steps", file=sys.stderr, flush=True)
    ms = time_graphs(torch, graphs, args.steps, args.warmup) / args.steps
    graphs[0].replay()                       # replays must reproduce the eager result
    torch.cuda.synchronize()
    replay_ok = bool(torch.equal(wl.snapshot(), eager0))
    del eager0
    # the pages' timing protocol: 3 repetitions x 30 runs; median and spread per step
    protocol = None
    if not args.profile_pass:
        reps = []
        runs = getattr(wl, "protocol_runs", 30)
        for _ in range(3):
            reps.append(time_graphs(torch, graphs, runs, min(3, runs)) / runs)
        protocol = {"repetitions": 3, "runs": runs, "median_ms": round(float(np.median(reps)), 5),
                    "min_ms": round(float(np.min(reps)), 5), "max_ms": round(float(np.max(reps)), 5)}
    # the same decode step as two calls per layer, for comparison
    separate_ms = None
    if isinstance(wl, DecodeStep) and wl.mode == "fused" and not args.profile_pass:
        sgraphs = [capture(torch, lambda cp=cp: wl.step(cp, "separate")) for cp in range(wl.copies)]
        separate_ms = round(time_graphs(torch, sgraphs, max(10, args.steps // 4), 3) / max(10, args.steps // 4), 5)
        del sgraphs

    print("[bench] per-launch timing of the dominant kernel", file=sys.stderr, flush=True)
    durs = wl.launch_times(max(3, min(30, args.steps // 5)))
    avg_launch = float(np.mean(durs))
    mfma = getattr(wl, "roofline_bound", "hbm") == "mfma"
    achieved = wl.launch_flops() / avg_launch / 1e12 if mfma else wl.launch_bytes() / avg_launch / 1e9

    if args.sweep_splits and isinstance(wl, DecodeStep):
        sweep_splits(torch, wl, [int(x) for x in args.sweep_splits.split(",")])
    if args.copy_calibration:
        copy_calibration(torch)
    stream_ref = None
    if isinstance(wl, DecodeStep) and not args.no_stream_reference and not args.profile_pass:
        print("[bench] plain streaming read of the same cache bytes", file=sys.stderr, flush=True)
        st_s, st_bytes, st_grid = stream_reference(torch, wl)
        st_gbs = st_bytes / st_s / 1e9
        stream_ref = {"kernel": "k_stream_read (libnvkv_bench.so): every 16-byte word of the layer's K/V codes and "
                                "scales read once, non-temporal, one launch per layer, graph of back-to-back launches",
                      "bytes_per_launch": st_bytes, "avg_launch_us": round(st_s * 1e6, 3),
                      "achieved_gbs": round(st_gbs, 2), "grid": st_grid}
    phases = None
    if args.trace_phases and isinstance(wl, DecodeStep):
        print("[bench] phase-stamped decode instance", file=sys.stderr, flush=True)
        phases = trace_phases(torch, wl, args.trace_dump)
        print("[bench] phase timeline: " + json.dumps(phases), file=sys.stderr, flush=True)
    print("[bench] oracle check / cpu baseline", file=sys.stderr, flush=True)
    check = None if args.no_check else wl.check()
    base = None if args.no_cpu_baseline else wl.cpu_baseline()

    step_s = ms * 1e-3
    gbs = wl.step_bytes() / step_s / 1e9
    tflops = wl.step_flops() / step_s / 1e12 if mfma else None
    c = wl.c
    line = {
        "metric": wl.metric,
        "value": round(tflops, 2) if mfma else round(gbs, 2),
        "unit": "TFLOP/s" if mfma else "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "arithmetic": "f16 MFMA on exact operand splits, f32 accumulate; codec in f32",
        "cache_format": "nvfp4: e2m1 codes, e4m3 block scales per 16, f32 tensor scale",
        "data": "synthetic",
        "config": {
            "workload": wl.describe(),
            "global_batch": c["B"], "seq_len": c["T"], "layers": c["layers"], "parallelism": "none (1 GPU)",
            "split_tokens": args.split_tokens or "auto",
            "append_kernel": getattr(wl, "append_kernel", "library"),
        },
        "tokens_per_s": round(wl.tokens_per_step() / step_s, 2),
        "hbm_frac_of_step": round(gbs / HBM_PEAK_GBS, 4),
        "roofline": {
            "bound": "mfma" if mfma else "hbm", "achieved": round(achieved, 2),
            "peak": MFMA_F16_PEAK_TFLOPS if mfma else HBM_PEAK_GBS, "unit": "TFLOP/s" if mfma else "GB/s",
            "frac": round(achieved / (MFMA_F16_PEAK_TFLOPS if mfma else HBM_PEAK_GBS), 4),
            "traffic": traffic_per_launch(wl),
            "kernel": wl.kernel_label,
            "bytes_per_launch": wl.launch_bytes(), "avg_launch_us": round(avg_launch * 1e6, 3),
            "min_launch_us": round(float(np.min(durs)) * 1e6, 3),
            **({"flops_per_launch": wl.launch_flops()} if mfma else {}),
        },
        "cpu_baseline": base,
        "stream_reference": stream_ref,
        "stream_frac": (round(achieved / stream_ref["achieved_gbs"], 4) if stream_ref and not mfma else None),
        "sq_counters": sq_counters(wl),
        "phase_timeline": phases,
        "graph_replay_matches_eager": replay_ok,
        "timing_protocol": protocol,
        "separate_calls_ms_per_step": separate_ms,
        "oracle_check": check,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
