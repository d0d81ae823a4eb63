"""Build libw4.so in-tree with hipcc for gfx950.

    python -m int4_group_wise_amd.build

Each HIP translation unit is compiled to an object under ``_build/`` and the
objects are linked into ``int4_group_wise_amd/libw4.so``.  Every build
recompiles from source.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libw4.so")
# the streaming-read floor the benchmark reports beside the HBM peak
# (measurement only, a library of its own)
BENCH_LIB = os.path.join(PKG, "libw4_bench.so")
BENCH_SOURCE = "bench_read.hip"
ARCH = "gfx950"

# Every translation unit: gfx950 only, no packed-fp32 instructions.
COMMON = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", INCLUDE, "-I", CSRC]
# Codec units must reproduce the fp32 definition bit for bit: no fused
# multiply-add contraction (divisions stay IEEE correctly rounded by default).
EXTRA = {"w4_codec.hip": ["-ffp-contract=off"]}
SOURCES = ["w4_api.hip", "w4_codec.hip", "w4_linear.hip", "w4_stream.hip", "w4_batched.hip", "w4_actmma.hip", "w4_gemm.hip", "w4_grad.hip", "w4_lora.hip", "w4_formats.hip"]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found")
    return path


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        cmd = [cc, *COMMON, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the GPU target feature; that note is harmless
        text = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            failed.append(f"{src}:\n{text}")
        elif verbose and text.strip():
            print(text)
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n".join(failed))
    tmp = LIB + ".tmp"
    cmd = [cc, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    tmp = BENCH_LIB + ".tmp"
    cmd = [cc, *COMMON, "-shared", os.path.join(CSRC, BENCH_SOURCE), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout.decode(errors="replace"))
    os.replace(tmp, BENCH_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
