#!/usr/bin/env python3
"""Benchmark of the NVFP4 KV-cache hot path on one MI355X.

Default workload: one decode step of a Qwen3-8B-shaped attention cache -- 36 layers x 8 KV
heads x head_dim 128, 32 query heads, batch 4 x 2304 cached tokens, 16-token pages with a
shuffled page table, keys and values NVFP4 with static per-channel key smoothing.  A step
runs, for every layer, quantize_append_kv of the new token of each sequence followed by
decode_attention_nvfp4 over all 2304 tokens (the whole hot path: quantise -> pack -> split-K
decode -> merge).  Steps replay HIP graphs over 3 rotating copies of the 36-layer cache
(1.15 GB, beyond the 256 MB last-level cache).

Printed: one JSON line with the step throughput (algorithmic bytes / step time), tokens/s,
the roofline of the decode kernel (algorithmic bytes per launch / average launch time from
HIP events), and the CPU oracle timed on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--workload step36|step36-vonly|step36-hadamard|long]
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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="step36")
    ap.add_argument("--copies", type=int, default=3)
    ap.add_argument("--split-tokens", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-check", action="store_true")
    ap.add_argument("--sweep-splits", default="",
                    help="comma-separated split sizes: report the decode launch time of each")
    ap.add_argument("--profile-pass", action="store_true",
                    help="short run for rocprofv3: few steps, no CPU baseline")
    return ap.parse_args()


VARIANTS = {
    "step36": dict(cfg="step36", k_fmt=1, flags=1, label="K+V NVFP4, K smoothed"),
    "step36-vonly": dict(cfg="step36", k_fmt=0, flags=0, label="K bf16, V NVFP4"),
    "step36-hadamard": dict(cfg="step36", k_fmt=1, flags=2, label="K+V NVFP4, K Hadamard-128"),
    "step36-had-smooth": dict(cfg="step36", k_fmt=1, flags=3, label="K+V NVFP4, K smoothed + Hadamard-128"),
    "long": dict(cfg="long", k_fmt=1, flags=1, label="K+V NVFP4, K smoothed"),
}


def row_bytes(fmt):
    return 256 if fmt == 0 else 72


class Workload:
    def __init__(self, name, copies, split_tokens):
        import torch
        import nvfp4_bit_kv_amd as nk
        from synth import kv_inputs as S
        self.torch, self.nk, self.S = torch, nk, S
        v = VARIANTS[name]
        c = S.CONFIGS[v["cfg"]]
        self.name, self.v, self.c = name, v, c
        self.B, self.T, self.hkv, self.hq, self.L = c["B"], c["T"], c["hkv"], c["hq"], c["layers"]
        self.k_fmt, self.flags = v["k_fmt"], v["flags"]
        self.copies = copies
        self.split_tokens = split_tokens
        B, T, hkv = self.B, self.T, self.hkv
        self.pps = (T + PAGE - 1) // PAGE
        self.num_pages = B * self.pps
        rng = np.random.default_rng(1234)
        self.table_np = rng.permutation(self.num_pages).reshape(B, self.pps).astype(np.int32)
        dev = "cuda"
        self.table = torch.from_numpy(self.table_np).to(dev)
        t = np.arange(T)
        slots = self.table_np[:, t // PAGE] * PAGE + t % PAGE          # [B][T]
        self.slots_np = slots.astype(np.int32)
        self.seq_lens = torch.full((B,), T, dtype=torch.int32, device=dev)
        self.new_slots = torch.from_numpy(np.ascontiguousarray(self.slots_np[:, T - 1])).to(dev)
        self.caches = [[None] * self.L for _ in range(copies)]
        self.k_new, self.v_new, self.q = [], [], []
        self.out = torch.empty((self.L, B, self.hq, 128), dtype=torch.float32, device=dev)
        self.wsb = nk.decode_workspace_bytes(B, self.hq, hkv, T, split_tokens)
        self.ws = torch.zeros(max(self.wsb, 256), dtype=torch.uint8, device=dev)
        self._build()

    def _build(self):
        torch, nk, S = self.torch, self.nk, self.S
        c, B, T, hkv = self.c, self.B, self.T, self.hkv
        chunk = max(1, (1 << 22) // (T * hkv))          # sequences per prefill append call
        for l in range(self.L):
            k = S.make_keys_device(c["kind"], c["cfg"], l, B, T, hkv)
            v = S.make_values_device(c["cfg"], l, B, T, hkv)
            kw = torch.cat([S.make_keys_device(c["kind"], c["cfg"], l, 1, c["Tw"], hkv, role=S.ROLE_WIN0 + w)
                            for w in range(4)])
            vw = torch.cat([S.make_values_device(c["cfg"], l, 1, c["Tw"], hkv, role=S.ROLE_WIN0 + 4 + w)
                            for w in range(4)])
            s = torch.empty((hkv, 128), dtype=torch.float32, device="cuda")
            r = torch.empty_like(s)
            g = torch.empty(2, dtype=torch.float32, device="cuda")
            nk.calibrate_key_smoothing(kw, vw, 4, c["Tw"], hkv, True, self.flags, s, r, g)
            for cp in range(self.copies):
                cache = nk.CacheLayer(self.num_pages, PAGE, hkv, k_fmt=self.k_fmt, k_flags=self.flags)
                cache.smooth.copy_(s)
                cache.inv_smooth.copy_(r)
                cache.gscale.copy_(g)
                Ls = cache.struct()
                for b0 in range(0, B, chunk):
                    b1 = min(B, b0 + chunk)
                    n = (b1 - b0) * (T - 1)
                    sl = torch.from_numpy(np.ascontiguousarray(self.slots_np[b0:b1, :T - 1]).reshape(-1)).cuda()
                    nk.quantize_append_kv(Ls, k[b0:b1, :T - 1].contiguous(), v[b0:b1, :T - 1].contiguous(), sl, n)
                self.caches[cp][l] = (cache, Ls)
            self.k_new.append(k[:, T - 1].contiguous())
            self.v_new.append(v[:, T - 1].contiguous())
            self.q.append(S.make_queries_device(c["cfg"], l, B, self.hq))
            if l == 0:
                self.layer0 = (k.cpu(), v.cpu(), kw.cpu(), vw.cpu())
            del k, v, kw, vw
        torch.cuda.synchronize()

    # one layer of the hot path: append the new token, then attend over the whole cache
    def layer_step(self, cp, l, decode_only=False):
        nk = self.nk
        cache, Ls = self.caches[cp][l]
        if not decode_only:
            nk.quantize_append_kv(Ls, self.k_new[l], self.v_new[l], self.new_slots, self.B)
        nk.decode_attention_nvfp4(Ls, self.q[l], self.B, self.hq, self.table, self.pps, self.seq_lens, self.T,
                                  1.0 / math.sqrt(128), self.out[l], self.ws, self.wsb, self.split_tokens)

    def step(self, cp):
        for l in range(self.L):
            self.layer_step(cp, l)

    # algorithmic bytes (what the method must move)
    def decode_bytes_per_layer(self):
        per_tok = row_bytes(self.k_fmt) + 72
        return self.B * self.hkv * self.T * per_tok + self.B * self.hq * (256 + 512)

    def append_bytes_per_layer(self):
        return self.B * self.hkv * ((256 + row_bytes(self.k_fmt)) + (256 + 72))

    def step_bytes(self):
        return self.L * (self.decode_bytes_per_layer() + self.append_bytes_per_layer())


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


def capture(torch, fn):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def decode_launch_times(torch, wl, reps):
    """Average duration of one decode_attention_nvfp4 call (its kernels back to back, no host
    gaps): a HIP graph of the decode calls of all layers of a cache copy is replayed between
    two HIP events on the launch stream; one sample per replay, divided by the layer count."""
    graphs = [capture(torch, lambda cp=cp: [wl.layer_step(cp, l, decode_only=True) for l in range(wl.L)])
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
        d = decode_launch_times(torch, wl, reps=10)
        res[sp] = (float(np.mean(d)) * 1e6, float(np.min(d)) * 1e6)
        print(f"[sweep] split_tokens={sp}: avg {res[sp][0]:.2f} us  min {res[sp][1]:.2f} us  "
              f"-> {wl.decode_bytes_per_layer() / np.mean(d) / 1e9:.0f} GB/s", file=sys.stderr, flush=True)
    wl.split_tokens, wl.wsb, wl.ws = saved
    return res


def check_against_oracle(wl):
    """Sampled parity of the timed configuration: layer 0, every sequence and query head,
    against the oracle built from the same bf16 inputs (calibration included)."""
    from oracle import nvfp4_oracle as O
    torch, S = wl.torch, wl.S
    k, v, kw, vw = wl.layer0
    f = lambda t: S.bf16_to_f32(t.view(torch.int16).numpy().view(np.uint16))
    s, r, g = O.calibrate(f(kw), f(vw), True, wl.flags)
    B, T, hq = wl.B, wl.T, wl.hq
    qf = f(wl.q[0].cpu()).astype(np.float64)
    if wl.k_fmt == 1:
        kc, ks = O.quantize_rows(O.key_transform(f(k), r[None, None], wl.flags), g[0])
        khat = [O.dequantize(kc[b], ks[b], g[0]) for b in range(B)]
        qp = O.query_transform(qf, np.repeat(s, hq // wl.hkv, 0)[None], wl.flags)
    else:
        khat = [f(k[b]).astype(np.float64) for b in range(B)]
        qp = qf
    vc, vs = O.quantize_rows(f(v), g[1])
    vhat = [O.dequantize(vc[b], vs[b], g[1]) for b in range(B)]
    ref = O.attention(qp, khat, vhat, [T] * B, 1.0 / math.sqrt(128))
    got = wl.out[0].cpu().numpy().astype(np.float64)
    vmax = max(float(np.abs(x).max()) for x in vhat)
    err = float(np.abs(got - ref).max())
    rel = float((np.linalg.norm(got - ref, axis=-1) / np.linalg.norm(ref, axis=-1)).max())
    ok = err <= 1e-3 * vmax and rel <= 1e-4
    return dict(ok=bool(ok), max_abs_err=err, tol_abs=1e-3 * vmax, max_rel_l2=rel, tol_rel_l2=1e-4)


def cpu_baseline(wl, budget_s=12.0):
    """The oracle as it stands on a bounded sample: per layer and for all B sequences, quantise
    the new token, dequantise the cache and run fp64 attention for every query head (the oracle
    needs the cached codes, which it builds itself beforehand, untimed).  BLAS is held to one
    thread.  Extrapolated to the 36-layer step."""
    from threadpoolctl import threadpool_limits
    from oracle import nvfp4_oracle as O
    torch, S = wl.torch, wl.S
    k, v, kw, vw = wl.layer0
    f = lambda t: S.bf16_to_f32(t.view(torch.int16).numpy().view(np.uint16))
    B, T, hq, hkv = wl.B, wl.T, wl.hq, wl.hkv
    with threadpool_limits(limits=1):
        s, r, g = O.calibrate(f(kw), f(vw), True, wl.flags)
        kf, vf = f(k), f(v)
        if wl.k_fmt == 1:
            kc, ks = O.quantize_rows(O.key_transform(kf[:, :T - 1], r[None, None], wl.flags), g[0])
        vc, vs = O.quantize_rows(vf[:, :T - 1], g[1])
        qf = f(wl.q[0].cpu()).astype(np.float64)
        layers = 0
        t0 = time.perf_counter()
        while True:
            if wl.k_fmt == 1:
                nkc, nks = O.quantize_rows(O.key_transform(kf[:, T - 1:], r[None, None], wl.flags), g[0])
                khat = [O.dequantize(np.concatenate([kc[b], nkc[b]]), np.concatenate([ks[b], nks[b]]), g[0])
                        for b in range(B)]
                qp = O.query_transform(qf, np.repeat(s, hq // hkv, 0)[None], wl.flags)
            else:
                khat = [kf[b].astype(np.float64) for b in range(B)]
                qp = qf
            nvc, nvs = O.quantize_rows(vf[:, T - 1:], g[1])
            vhat = [O.dequantize(np.concatenate([vc[b], nvc[b]]), np.concatenate([vs[b], nvs[b]]), g[1])
                    for b in range(B)]
            O.attention(qp, khat, vhat, [T] * B, 1.0 / math.sqrt(128))
            layers += 1
            el = time.perf_counter() - t0
            if el >= budget_s or layers >= wl.L:
                break
    per_layer = el / layers
    step_s = per_layer * wl.L
    return dict(value=round(B / step_s, 4), unit="tokens/s", cores=1, kind="oracle",
                sample=f"{layers} x (layer 0 of {wl.L}, all {B} sequences: append 1 token + dequantise "
                       f"{T} tokens x {hkv} KV heads + fp64 attention for {hq} query heads), "
                       f"{el:.1f} s on 1 core of {len(os.sched_getaffinity(0))}, extrapolated x{wl.L} layers",
                oracle_step_s=round(step_s, 3),
                oracle_effective_gbs=round(wl.step_bytes() / step_s / 1e9, 6))


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1 "
                                   "(sharding design is described in the design notes)"}))
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.profile_pass:
        args.steps, args.warmup, args.no_cpu_baseline = min(args.steps, 20), min(args.warmup, 5), True
    print(f"[bench] building workload {args.workload}", file=sys.stderr, flush=True)
    wl = Workload(args.workload, args.copies, args.split_tokens)

    # eager warm-up and reference outputs per copy, then graph capture per copy
    wl.step(0)
    torch.cuda.synchronize()
    eager0 = wl.out.clone()
    graphs = [capture(torch, lambda cp=cp: wl.step(cp)) for cp in range(wl.copies)]
    print(f"[bench] captured {len(graphs)} step graphs; timing {args.steps} steps", file=sys.stderr, flush=True)
    ms = time_graphs(torch, graphs, args.steps, args.warmup) / args.steps
    # replays must reproduce the eager result
    graphs[0].replay()
    torch.cuda.synchronize()
    replay_ok = bool(torch.equal(wl.out, eager0))

    print("[bench] per-launch decode timing", file=sys.stderr, flush=True)
    durs = decode_launch_times(torch, wl, reps=max(3, min(30, args.steps // 5)))
    avg_launch = float(np.mean(durs))
    dec_bytes = wl.decode_bytes_per_layer()
    achieved = dec_bytes / avg_launch / 1e9

    if args.sweep_splits:
        sweep_splits(torch, wl, [int(x) for x in args.sweep_splits.split(",")])
    check = None if args.no_check else check_against_oracle(wl)
    base = None if args.no_cpu_baseline else cpu_baseline(wl)

    step_s = ms * 1e-3
    gbs = wl.step_bytes() / step_s / 1e9
    c = wl.c
    line = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4 cache (e2m1 + e4m3 scales); f16 MFMA on exact operands, f32 accumulate",
        "data": "synthetic",
        "config": {
            "workload": f"{args.workload}: Qwen3-8B-shaped decode step, {c['layers']} layers x {c['hkv']} KV heads "
                        f"x 128, {c['hq']} query heads, batch {c['B']} x {c['T']} context, 16-token paged "
                        f"cache, {wl.v['label']}; per layer append 1 token + split-K decode",
            "global_batch": c["B"], "seq_len": c["T"], "layers": c["layers"], "parallelism": "none (1 GPU)",
            "split_tokens": args.split_tokens or "auto",
        },
        "tokens_per_s": round(c["B"] / step_s, 2),
        "hbm_frac_of_step": round(gbs / HBM_PEAK_GBS, 4),
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
            "kernel": "k_decode (decode_attention_nvfp4: split-K decode + in-kernel cross-split merge), per layer",
            "bytes_per_launch": dec_bytes, "avg_launch_us": round(avg_launch * 1e6, 3),
            "min_launch_us": round(float(np.min(durs)) * 1e6, 3),
        },
        "cpu_baseline": base,
        "graph_replay_matches_eager": replay_ok,
        "oracle_check": check,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
