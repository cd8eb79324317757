"""Build libnvfp4kv.so in-tree with hipcc for gfx950.

    python -m nvfp4_bit_kv_amd.build

The quantise/calibrate and KLT-calibration translation units are compiled with
-ffp-contract=off (their fp32 key transform is part of the bit-exact encoding); the decode unit with -fno-honor-nans (its
scores are finite or -inf and every code and scale decodes finite, so max operations need
no NaN quieting), and so is the prefill-attention unit; all HIP code is compiled without
packed fp32 instructions.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libnvfp4kv.so")
ARCH = os.environ.get("NVKV_OFFLOAD_ARCH", "gfx950")

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fvisibility=hidden", "-Wall", "-Wno-unused-function"]
SOURCES = {
    "nvkv_capi.hip": [],
    "nvkv_quantize.hip": ["-ffp-contract=off"],
    "nvkv_klt.hip": ["-ffp-contract=off"],
    "nvkv_decode.hip": ["-fno-honor-nans"],
    "nvkv_prefill.hip": ["-fno-honor-nans"],
    "nvkv_bench.hip": [],
}
# The library proper, and the bench's measurement helpers (a plain streaming-read kernel and
# the phase-stamped decode instance; linked with the same decode object, loaded only by the bench).
LIB_OBJECTS = ["nvkv_capi.hip", "nvkv_quantize.hip", "nvkv_klt.hip", "nvkv_decode.hip", "nvkv_prefill.hip"]
BENCH_LIB = os.path.join(PKG, "libnvkv_bench.so")
BENCH_OBJECTS = ["nvkv_bench.hip", "nvkv_decode.hip"]


def _hipcc() -> str:
    for cand in ("/opt/rocm/bin/hipcc", "hipcc"):
        if os.path.isabs(cand) and os.path.exists(cand):
            return cand
    return "hipcc"


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    procs = []
    objs = []
    for src, extra in SOURCES.items():
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        cmd = [hipcc, *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        objs.append(obj)
    failed = []
    for src, cmd, p in procs:
        out, _ = p.communicate()
        noise = "is not a recognized feature for this target"
        lines = [ln for ln in out.splitlines() if noise not in ln and "(ignoring feature)" not in ln]
        if p.returncode != 0:
            failed.append((src, "\n".join(lines)))
        elif verbose and lines:
            print("\n".join(lines))
    if failed:
        msg = "\n".join(f"--- {s} ---\n{o}" for s, o in failed)
        raise RuntimeError(f"hipcc failed:\n{msg}")
    obj_of = {src: os.path.join(BUILD, src.replace(".hip", ".o")) for src in SOURCES}
    for lib, members in ((LIB, LIB_OBJECTS), (BENCH_LIB, BENCH_OBJECTS)):
        tmp = lib + ".tmp"
        cmd = [hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *[obj_of[m] for m in members], "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stdout}")
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
