"""Benchmark of the W4A16 group-wise int4 hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-secondary]

A step is one w4_linear call on the decode workload (x bf16 [1, 4096],
W [14336, 4096] zero-point int4, G = 128, bf16 bias).  Steps run as HIP-graph
replays that rotate over enough weight copies to overflow the 256 MB
Infinity Cache, so each call streams its weights from HBM as it would in a
model with many layers.  The JSON line reports whole-job HBM GB/s of the
algorithmic bytes, the decode kernel's roofline (its average launch duration
measured with HIP events on the launch stream), and the CPU oracle on a
bounded sample.  Secondary entries cover a hot-cache decode figure (labelled
as such), the prefill GEMM (TFLOP/s), the
batched decode, the input gradient (decode and prefill shapes), the LoRA
merge, the codec round trip, the GGUF Q4_0 codec and the zero-point packing.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFS = 2516.6    # MI355X dense bf16 matrix cores
MALL_BYTES = 256 << 20         # Infinity Cache
FP64_VEC_PEAK_TFS = 78.6       # MI355X fp64 vector
GPU_LEAD_CYCLES = 200_000      # device-side wait before a timed region (about 0.1 ms)


def algorithmic_bytes_linear(M, N, K, G, asym, bias):
    NG = -(-K // G)
    b = N * ((K + 1) // 2) + 4 * N * NG + M * K * 2 + M * N * 2
    if asym:
        b += N * NG
    if bias:
        b += 2 * N
    return b


def codec_bytes(N, K, G, w_bytes):
    NG = -(-K // G)
    packed = N * ((K + 1) // 2) + 4 * N * NG
    return N * K * w_bytes + packed, packed + N * K * 2   # quantize_pack, dequantize (bf16 out)


class Rotation:
    """B independent copies of the packed weight, enough to exceed twice the
    Infinity Cache, used round-robin by consecutive calls."""

    def __init__(self, tensors, min_bytes):
        per = sum(t.numel() * t.element_size() for t in tensors if t is not None)
        self.count = max(2, math.ceil(min_bytes / per))
        self.sets = [tuple(None if t is None else t.clone() for t in tensors) for _ in range(self.count)]
        self.bytes_per_set = per


def time_graph(call, n_calls, steps, warmup, rot_count):
    """Capture `n_calls` calls (call(i) uses rotation set i % rot_count) in one
    graph; replay it so that exactly `warmup` then `steps` calls run.  Returns
    milliseconds of the timed region measured by events on the replay stream
    and by the host clock."""
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.stream(cap):
        call(0)                                  # eager warm call (loads code objects)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=cap):
        for i in range(n_calls):
            call(i % rot_count)
    tail = None
    if steps % n_calls:
        tail = torch.cuda.CUDAGraph()
        with torch.cuda.graph(tail, stream=cap):
            for i in range(steps % n_calls):
                call(i % rot_count)
    for _ in range(max(1, -(-warmup // n_calls))):
        g.replay()
    if tail is not None:
        tail.replay()          # a graph's first replay carries a one-time cost: keep it out of the timing
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    # a short device-side wait ahead of the start event, so that the graph
    # launches below are already queued when the timed region begins: the
    # events then time the calls, not the host's first graph submission
    torch.cuda._sleep(GPU_LEAD_CYCLES)
    e0.record()
    for _ in range(steps // n_calls):
        g.replay()
    if tail is not None:
        tail.replay()
    e1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return e0.elapsed_time(e1), (t1 - t0) * 1e3


def bench_decode(w4, steps, warmup, packed_zeros=False):
    """The decode workload; with packed_zeros the zero-points are stored two
    per byte (W4_ASYM_PACKED) and read that way by the kernel."""
    from int4_group_wise_amd.workloads import workload, generate
    wl = workload("decode")
    t = generate(wl)
    dev = "cuda:0"
    codes, scales, zeros = w4.quantize_pack(t["w"].to(dev), wl.G, wl.mode)
    mode = wl.mode
    if packed_zeros:
        zeros, mode = w4.pack_zeros(zeros), "asym_packed"
    x = t["x"].to(dev)
    bias = t["bias"].to(dev)
    rot = Rotation([codes, scales, zeros, bias], 2 * MALL_BYTES)
    ys = [torch.empty(wl.M, wl.N, dtype=torch.bfloat16, device=dev) for _ in range(rot.count)]
    del codes, scales, zeros

    def call(i):
        c, s, z, b = rot.sets[i]
        w4.linear(x, c, s, z, None, wl.K, wl.G, mode, b, out=ys[i])

    n_calls = rot.count * max(1, 128 // rot.count)
    ev_ms, host_ms = time_graph(call, n_calls, steps, warmup, rot.count)
    nbytes = algorithmic_bytes_linear(wl.M, wl.N, wl.K, wl.G, True, True)
    if packed_zeros:
        ng = -(-wl.K // wl.G)
        nbytes -= wl.N * (ng - (ng + 1) // 2)
    return wl, nbytes, ev_ms, host_ms, rot


def bench_decode_hot(w4, steps=2000):
    """The decode workload on one weight copy, resident in the Infinity Cache:
    a hot-cache figure, not the headline (which streams from HBM)."""
    from int4_group_wise_amd.workloads import workload, generate
    wl = workload("decode")
    t = generate(wl)
    dev = "cuda:0"
    c, s, z = w4.quantize_pack(t["w"].to(dev), wl.G, wl.mode)
    x, b = t["x"].to(dev), t["bias"].to(dev)
    y = torch.empty(wl.M, wl.N, dtype=torch.bfloat16, device=dev)
    ev_ms, _ = time_graph(lambda i: w4.linear(x, c, s, z, None, wl.K, wl.G, wl.mode, b, out=y), 100, steps, 100, 1)
    nbytes = algorithmic_bytes_linear(wl.M, wl.N, wl.K, wl.G, True, True)
    gbs = nbytes * steps / (ev_ms * 1e-3) / 1e9
    return {"metric": "W4A16 linear GB/s M=1, hot cache (one weight copy, Infinity-Cache resident; not HBM-bound)",
            "value": round(gbs, 1), "unit": "GB/s", "us_per_call": round(ev_ms * 1e3 / steps, 3),
            "config": {"workload": "decode", "M": wl.M, "N": wl.N, "K": wl.K, "G": wl.G, "mode": wl.mode,
                       "weight_copies_rotated": 1}}


def stream_read_lib():
    """The streaming-read probe (libw4_bench.so, built next to libw4.so)."""
    import ctypes
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "int4_group_wise_amd", "libw4_bench.so")
    lib = ctypes.CDLL(path)
    lib.w4bench_stream_read.restype = ctypes.c_int
    lib.w4bench_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    return lib


def bench_streaming_floor(nbytes, steps=4000):
    """What one launch moving the same number of HBM bytes achieves in this
    harness: a plain streaming read of `nbytes` (16-byte non-temporal loads,
    U per thread issued together, a workgroup reading U x 4 KB contiguously;
    libw4_bench.so), torch's sum and amax reductions over the same fp32
    buffer, and a device copy of nbytes / 2 bytes (read plus write), each
    rotated past the Infinity Cache.  The fastest is reported as the practical
    single-launch rate next to the 8 TB/s peak."""
    dev = "cuda:0"
    count = max(2, math.ceil(2 * MALL_BYTES / nbytes))
    bufs = [torch.empty(nbytes // 4, dtype=torch.float32, device=dev).normal_() for _ in range(count)]
    halves = [torch.empty(nbytes // 4, dtype=torch.bfloat16, device=dev) for _ in range(count)]
    sink = torch.zeros(max(1, nbytes // 8192), dtype=torch.int32, device=dev)
    lib = stream_read_lib()

    def read(u):
        def fn(i):
            err = lib.w4bench_stream_read(bufs[i].data_ptr(), nbytes, u, sink.data_ptr(),
                                          torch.cuda.current_stream().cuda_stream)
            if err:
                raise RuntimeError(f"stream_read U={u}: HIP error {err}")
        return fn

    cases = [(f"stream_read U={u}", read(u)) for u in (4, 8, 16) if nbytes % (4096 * u) == 0]
    res = {}
    for name, fn in (*cases,
                     ("torch.sum", lambda i: torch.sum(bufs[i])),
                     ("torch.amax", lambda i: torch.amax(bufs[i])),
                     ("copy_ (read + write)", lambda i: halves[i].copy_(bufs[i][: nbytes // 8].view(torch.bfloat16)))):
        ev_ms, _ = time_graph(fn, count * max(1, 64 // count), steps, count, count)
        us = ev_ms * 1e3 / steps
        res[name] = {"us_per_launch": round(us, 3), "GB/s": round(nbytes / us / 1e3, 1)}
    best = max(res, key=lambda k: res[k]["GB/s"])
    del bufs, halves, sink
    return {"GB/s": res[best]["GB/s"], "kernel": best, "bytes_per_launch": nbytes, "measured": res}


PROFILES = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "gemv_stream_decode_traffic.txt")
DECODE_SOURCES = ("w4_stream.hip", "w4_dot.h", "w4_device.h", "w4_internal.h")


def decode_source_hash():
    """sha256 over the sources of the decode kernel (counters taken on other
    sources no longer describe it)."""
    import hashlib
    h = hashlib.sha256()
    base = os.path.join(os.path.dirname(os.path.abspath(__file__)), "int4_group_wise_amd", "csrc")
    for f in DECODE_SOURCES:
        with open(os.path.join(base, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per decode launch from the committed counter summary, or None
    when it is missing or was taken on different kernel sources."""
    try:
        kv = {}
        with open(TRAFFIC_FILE) as fh:
            for ln in fh:
                if ":" in ln and not ln.startswith("#"):
                    k, v = ln.split(":", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("source_sha256") != decode_source_hash():
            return None
        return int(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def run_counters(w4):
    """Eager launches for rocprofv3 --pmc: 12 decode calls over 3 weight
    copies, then 3 plain device copies of 256 MiB that calibrate the counters,
    then 8 batched-decode calls over 2 weight copies, 8 act-order decode calls
    over 2 weight copies, 2 codec round trips (quantize_pack + dequantize),
    3 prefill calls and 3 prefill-shape input-gradient calls."""
    from int4_group_wise_amd.workloads import workload, generate
    dev = "cuda:0"
    wl = workload("decode")
    t = generate(wl)
    sets = [w4.quantize_pack(t["w"].to(dev), wl.G, wl.mode) for _ in range(3)]
    x, b = t["x"].to(dev), t["bias"].to(dev)
    y = torch.empty(wl.M, wl.N, dtype=torch.bfloat16, device=dev)
    src = torch.empty(128 << 20, dtype=torch.bfloat16, device=dev).normal_()
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for i in range(12):
        c, s, z = sets[i % 3]
        w4.linear(x, c, s, z, None, wl.K, wl.G, wl.mode, b, out=y)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del sets, src, dst, t
    # batched decode
    wl = workload("batched_decode")
    t = generate(wl)
    sets = [w4.quantize_pack(t["w"].to(dev), wl.G, wl.mode) for _ in range(2)]
    del t["w"]
    x = t["x"].to(dev)
    y = torch.empty(wl.M, wl.N, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(1, w4.linear_workspace_bytes(wl.M, wl.N, wl.K, wl.G, wl.mode)), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    for i in range(8):
        c, s, _ = sets[i % 2]
        w4.linear(x, c, s, None, None, wl.K, wl.G, wl.mode, None, out=y, workspace=ws)
    torch.cuda.synchronize()
    del sets, x, y, ws, t
    # act-order decode (the decode shape with a permuted g_idx)
    wl = workload("decode", act_order=True)
    t = generate(wl)
    gi = t["g_idx"].to(dev)
    sets = [w4.quantize_pack(t["w"].to(dev), wl.G, wl.mode, gi) for _ in range(2)]
    x, b = t["x"].to(dev), t["bias"].to(dev)
    y = torch.empty(wl.M, wl.N, dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    for i in range(8):
        c, s, z = sets[i % 2]
        w4.linear(x, c, s, z, gi, wl.K, wl.G, wl.mode, b, out=y)
    torch.cuda.synchronize()
    del sets, x, b, y, t, gi
    # codec round trip
    wl = workload("codec")
    w = generate(wl)["w"].to(dev)
    for _ in range(2):
        c, s, z = w4.quantize_pack(w, wl.G, wl.mode)
        d = w4.dequantize(c, s, z, None, wl.K, wl.G, wl.mode, torch.bfloat16)
        del c, s, z, d
    torch.cuda.synchronize()
    del w
    # prefill (act-order dequantize + GEMM)
    wl = workload("prefill")
    t = generate(wl)
    gi = t["g_idx"].to(dev)
    c, s, z = w4.quantize_pack(t["w"].to(dev), wl.G, wl.mode, gi)
    x = t["x"].to(dev)
    y = torch.empty(wl.M, wl.N, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(w4.linear_workspace_bytes(wl.M, wl.N, wl.K, wl.G, wl.mode, True), dtype=torch.uint8, device=dev)
    for _ in range(3):
        w4.linear(x, c, s, z, gi, wl.K, wl.G, wl.mode, None, out=y, workspace=ws)
    torch.cuda.synchronize()
    # prefill-shape input gradient (transposed dequantize + GEMM)
    dy = y.clone()
    for _ in range(3):
        w4.linear_grad_input(dy, c, s, z, gi, wl.K, wl.G, wl.mode)
    torch.cuda.synchronize()
    print("counter launches done", flush=True)


def bench_secondary(w4):
    """Secondary entries (prefill quantize and GEMM, batched decode, input
    gradient, LoRA merge, codecs), each timed the same way."""
    from int4_group_wise_amd.workloads import workload, generate
    dev = "cuda:0"
    out = {}

    # decode with the zero-points packed two per byte
    wl, nb, ev_ms, _, rot = bench_decode(w4, 4000, 400, packed_zeros=True)
    gbs = nb * 4000 / (ev_ms * 1e-3) / 1e9
    out["decode_packed_zeros"] = {"metric": "W4A16 linear HBM GB/s M=1, zero-points packed two per byte",
                                  "value": round(gbs, 1), "unit": "GB/s", "us_per_call": round(ev_ms * 1e3 / 4000, 3),
                                  "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                                               "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)},
                                  "config": {"workload": "decode", "M": wl.M, "N": wl.N, "K": wl.K, "G": wl.G,
                                             "mode": "asym_packed", "algorithmic_bytes": nb,
                                             "weight_copies_rotated": rot.count}}
    del rot
    torch.cuda.empty_cache()

    # act-order decode: the decode shape with g_idx = perm // 128 (a scattered
    # group per column, as in the prefill workload's weight)
    wl = workload("decode", act_order=True)
    t = generate(wl)
    gi = t["g_idx"].to(dev)
    c, s, z = w4.quantize_pack(t["w"].to(dev), wl.G, wl.mode, gi)
    x, b = t["x"].to(dev), t["bias"].to(dev)
    del t
    rot = Rotation([c, s, z], 2 * MALL_BYTES)
    del c, s, z
    ys = [torch.empty(wl.M, wl.N, dtype=torch.bfloat16, device=dev) for _ in range(rot.count)]

    def call_a(i):
        cc, ss, zz = rot.sets[i]
        w4.linear(x, cc, ss, zz, gi, wl.K, wl.G, wl.mode, b, out=ys[i])

    steps = 2000
    ev_ms, _ = time_graph(call_a, rot.count * 4, steps, rot.count * 4, rot.count)
    nb = algorithmic_bytes_linear(wl.M, wl.N, wl.K, wl.G, True, True) + wl.K * 4   # + g_idx
    gbs = nb * steps / (ev_ms * 1e-3) / 1e9
    out["decode_act_order"] = {"metric": "W4A16 linear HBM GB/s M=1, act-order g_idx", "value": round(gbs, 1),
                               "unit": "GB/s", "us_per_call": round(ev_ms * 1e3 / steps, 3),
                               "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                                            "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)},
                               "config": {"workload": "decode", "M": wl.M, "N": wl.N, "K": wl.K, "G": wl.G,
                                          "mode": wl.mode, "act_order": True, "weight_copies_rotated": rot.count}}
    del rot, ys, x, b, gi
    torch.cuda.empty_cache()

    # prefill: M = 2048, act-order zero-point weights
    wl = workload("prefill")
    t = generate(wl)
    gi = t["g_idx"].to(dev)
    wf = t["w"].to(dev)
    c, s, z = w4.quantize_pack(wf, wl.G, wl.mode, gi)
    # its act-order quantize: fp32 W [4096, 4096] -> codes, scales, zero-points
    ev_ms, _ = time_graph(lambda i: w4.quantize_pack(wf, wl.G, wl.mode, gi, out=(c, s, z)), 20, 1000, 200, 1)
    qb = wf.numel() * 4 + gi.numel() * 4 + c.numel() + s.numel() * 4 + z.numel()
    gq = qb * 1000 / (ev_ms * 1e-3) / 1e9
    out["prefill_quantize"] = {"metric": "act-order quantize_pack HBM GB/s", "value": round(gq, 1), "unit": "GB/s",
                               "us_per_call": round(ev_ms * 1e3 / 1000, 2),
                               "roofline": {"bound": "hbm", "achieved": round(gq, 1), "peak": HBM_PEAK_GBS,
                                            "unit": "GB/s", "frac": round(gq / HBM_PEAK_GBS, 4)},
                               "config": {"workload": "prefill", "N": wl.N, "K": wl.K, "G": wl.G, "mode": wl.mode,
                                          "w_dtype": "f32", "act_order": True}}
    del wf
    x = t["x"].to(dev)
    y = torch.empty(wl.M, wl.N, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(w4.linear_workspace_bytes(wl.M, wl.N, wl.K, wl.G, wl.mode, True), dtype=torch.uint8, device=dev)
    # 400 warm-up calls (about 30 ms): the first few hundred calls of a process run a few
    # percent slower than the steady state that 1000 timed calls then measure
    steps = 1000
    ev_ms, host_ms = time_graph(lambda i: w4.linear(x, c, s, z, gi, wl.K, wl.G, wl.mode, None, out=y, workspace=ws),
                                20, steps, 400, 1)
    flops = 2.0 * wl.M * wl.N * wl.K
    tfs = flops * steps / (ev_ms * 1e-3) / 1e12
    out["prefill_gemm"] = {"metric": "W4A16 linear TFLOP/s M=2048", "value": round(tfs, 2), "unit": "TFLOP/s",
                           "us_per_call": round(ev_ms * 1e3 / steps, 2),
                           "roofline": {"bound": "mfma", "achieved": round(tfs, 2), "peak": BF16_MFMA_PEAK_TFS,
                                        "unit": "TFLOP/s", "frac": round(tfs / BF16_MFMA_PEAK_TFS, 4)},
                           "config": {"workload": "prefill", "M": wl.M, "N": wl.N, "K": wl.K, "G": wl.G,
                                      "mode": wl.mode, "act_order": True}}
    del c, s, z, x, y, ws, t, gi

    # batched decode: M = 16
    wl = workload("batched_decode")
    t = generate(wl)
    c, s, z = w4.quantize_pack(t["w"].to(dev), wl.G, wl.mode)
    del t["w"]
    x = t["x"].to(dev)
    rot = Rotation([c, s], 2 * MALL_BYTES)
    del c, s
    y = torch.empty(wl.M, wl.N, dtype=torch.bfloat16, device=dev)
    bws = torch.empty(max(1, w4.linear_workspace_bytes(wl.M, wl.N, wl.K, wl.G, wl.mode)), dtype=torch.uint8, device=dev)
    steps = 1000   # about 40 ms timed, as long as the headline's warm-up

    def call_b(i):
        cc, ss = rot.sets[i]
        w4.linear(x, cc, ss, None, None, wl.K, wl.G, wl.mode, None, out=y, workspace=bws)

    ev_ms, _ = time_graph(call_b, rot.count * 10, steps, rot.count * 10, rot.count)
    nb = algorithmic_bytes_linear(wl.M, wl.N, wl.K, wl.G, False, False)
    gbs = nb * steps / (ev_ms * 1e-3) / 1e9
    out["batched_decode"] = {"metric": "W4A16 linear HBM GB/s M=16", "value": round(gbs, 1), "unit": "GB/s",
                             "us_per_call": round(ev_ms * 1e3 / steps, 2),
                             "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                                          "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)},
                             "config": {"workload": "batched_decode", "M": wl.M, "N": wl.N, "K": wl.K,
                                        "G": wl.G, "mode": wl.mode}}
    del rot, x, y

    # input gradient dx = dy . Wd at the decode layer's shape (M = 1) and the
    # prefill shape (M = 2048, act-order)
    wl = workload("decode")
    t = generate(wl)
    c, s, z = w4.quantize_pack(t["w"].to(dev), wl.G, wl.mode)
    del t
    dy = torch.randn(1, wl.N, generator=torch.Generator().manual_seed(1)).to(torch.bfloat16).to(dev)
    rot = Rotation([c, s, z], 2 * MALL_BYTES)
    del c, s, z
    dx = torch.empty(1, wl.K, dtype=torch.bfloat16, device=dev)
    gws = torch.empty(w4.linear_grad_input_workspace_bytes(1, wl.N, wl.K, wl.G, wl.mode), dtype=torch.uint8, device=dev)
    steps = 2000

    def call_g(i):
        cc, ss, zz = rot.sets[i]
        w4.linear_grad_input(dy, cc, ss, zz, None, wl.K, wl.G, wl.mode, out=dx, workspace=gws)

    ev_ms, _ = time_graph(call_g, rot.count * 4, steps, rot.count * 4, rot.count)
    nb = algorithmic_bytes_linear(1, wl.N, wl.K, wl.G, True, False)   # same operands, dy/dx for x/y
    gbs = nb * steps / (ev_ms * 1e-3) / 1e9
    out["grad_input_decode"] = {"metric": "W4A16 input gradient HBM GB/s M=1", "value": round(gbs, 1), "unit": "GB/s",
                                "us_per_call": round(ev_ms * 1e3 / steps, 2),
                                "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                                             "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)},
                                "config": {"workload": "decode", "M": 1, "N": wl.N, "K": wl.K, "G": wl.G, "mode": wl.mode}}
    del rot, dx, gws, dy
    wl = workload("prefill")
    t = generate(wl)
    gi = t["g_idx"].to(dev)
    c, s, z = w4.quantize_pack(t["w"].to(dev), wl.G, wl.mode, gi)
    dy = torch.randn(wl.M, wl.N, generator=torch.Generator().manual_seed(2)).to(torch.bfloat16).to(dev)
    del t
    dx = torch.empty(wl.M, wl.K, dtype=torch.bfloat16, device=dev)
    gws = torch.empty(w4.linear_grad_input_workspace_bytes(wl.M, wl.N, wl.K, wl.G, wl.mode, True), dtype=torch.uint8, device=dev)
    steps = 1000   # warm-up and length as the prefill linear's
    ev_ms, _ = time_graph(lambda i: w4.linear_grad_input(dy, c, s, z, gi, wl.K, wl.G, wl.mode, out=dx, workspace=gws),
                          20, steps, 400, 1)
    tfs = 2.0 * wl.M * wl.N * wl.K * steps / (ev_ms * 1e-3) / 1e12
    out["grad_input_prefill"] = {"metric": "W4A16 input gradient TFLOP/s M=2048", "value": round(tfs, 2), "unit": "TFLOP/s",
                                 "us_per_call": round(ev_ms * 1e3 / steps, 2),
                                 "roofline": {"bound": "mfma", "achieved": round(tfs, 2), "peak": BF16_MFMA_PEAK_TFS,
                                              "unit": "TFLOP/s", "frac": round(tfs / BF16_MFMA_PEAK_TFS, 4)},
                                 "config": {"workload": "prefill", "M": wl.M, "N": wl.N, "K": wl.K, "G": wl.G,
                                            "mode": wl.mode, "act_order": True}}
    del c, s, z, gi, dy, dx, gws

    # LoRA merge at the decode layer's shape, rank 16: dequantize, add the
    # fp64-accumulated update, quantize again (fp64 FMA bound)
    wl = workload("decode")
    t = generate(wl)
    c, s, z = w4.quantize_pack(t["w"].to(dev), wl.G, wl.mode)
    del t
    rank = 16
    gen = torch.Generator().manual_seed(3)
    la = (torch.randn(wl.K, rank, generator=gen) * 0.05).to(dev)
    lb = (torch.randn(rank, wl.N, generator=gen) * 0.05).to(dev)
    outs = (torch.empty_like(c), torch.empty_like(s), torch.empty_like(z))
    steps = 200
    ev_ms, _ = time_graph(lambda i: w4.lora_merge(c, s, z, None, wl.K, wl.G, wl.mode, la, lb, 2.0, out=outs),
                          20, steps, 100, 1)
    sec = ev_ms * 1e-3 / steps
    fl = 2.0 * wl.N * wl.K * rank                        # fp64 multiply-adds of the update
    nbytes = 2 * (c.numel() + s.numel() * 4 + z.numel()) + (la.numel() + lb.numel()) * 4
    out["lora_merge"] = {"metric": "LoRA merge fp64 GFLOP/s (rank 16)", "value": round(fl / sec / 1e9, 1),
                         "unit": "GFLOP/s", "us_per_call": round(sec * 1e6, 2),
                         "gbs_algorithmic": round(nbytes / sec / 1e9, 1),
                         "roofline": {"bound": "alu", "achieved": round(fl / sec / 1e12, 3), "peak": FP64_VEC_PEAK_TFS,
                                      "unit": "TFLOP/s", "frac": round(fl / sec / 1e12 / FP64_VEC_PEAK_TFS, 4)},
                         "config": {"workload": "decode", "N": wl.N, "K": wl.K, "G": wl.G, "mode": wl.mode,
                                    "rank": rank}}
    del c, s, z, la, lb, outs

    # codec: bf16 W [28672, 8191] -> quantize_pack -> dequantize (bf16)
    wl = workload("codec")
    t = generate(wl)
    w = t["w"].to(dev)
    del t
    c, s, _ = w4.quantize_pack(w, wl.G, wl.mode)
    d = torch.empty(wl.N, wl.K, dtype=torch.bfloat16, device=dev)
    # 100 untimed calls, then 200 timed (about 30 ms): the quantizers are
    # VALU-bound and their per-call time follows the clock under sustained load
    # (about 120-170 us within one run), so the average is taken over a longer run
    steps, warm = 200, 100
    c2, s2 = torch.empty_like(c), torch.empty_like(s)
    ev_q, _ = time_graph(lambda i: w4.quantize_pack(w, wl.G, wl.mode, out=(c2, s2, None)), 5, steps, warm, 1)
    ev_d, _ = time_graph(lambda i: w4.dequantize(c, s, None, None, wl.K, wl.G, wl.mode, out=d), 5, steps, warm, 1)
    qb, db = codec_bytes(wl.N, wl.K, wl.G, 2)
    gq = qb * steps / (ev_q * 1e-3) / 1e9
    gd = db * steps / (ev_d * 1e-3) / 1e9
    out["codec"] = {"metric": "codec HBM GB/s (quantize_pack + dequantize)",
                    "value": round((qb + db) * steps / ((ev_q + ev_d) * 1e-3) / 1e9, 1), "unit": "GB/s",
                    "quantize_pack": {"GB/s": round(gq, 1), "us": round(ev_q * 1e3 / steps, 1), "frac": round(gq / HBM_PEAK_GBS, 4)},
                    "dequantize": {"GB/s": round(gd, 1), "us": round(ev_d * 1e3 / steps, 1), "frac": round(gd / HBM_PEAK_GBS, 4)},
                    "config": {"workload": "codec", "N": wl.N, "K": wl.K, "G": wl.G, "mode": wl.mode, "w_dtype": "bf16"}}
    del c, s, d, c2, s2, w

    # GGUF Q4_0 blocks of the codec weight at K = 8192 (bf16 [28672, 8192]):
    # quantize (2 B read + 18/32 B written per weight) and dequantize to bf16
    wl = workload("codec", K=8192)
    t = generate(wl)
    w = t["w"].to(dev)
    del t
    blocks = w4.q4_0_quantize(w)
    d = torch.empty(wl.N, wl.K, dtype=torch.bfloat16, device=dev)
    ev_q, _ = time_graph(lambda i: w4.q4_0_quantize(w, out=blocks), 5, steps, warm, 1)
    ev_d, _ = time_graph(lambda i: w4.q4_0_dequantize(blocks, torch.bfloat16, out=d), 5, steps, warm, 1)
    nb = wl.N * wl.K * 2 + blocks.numel()
    gq = nb * steps / (ev_q * 1e-3) / 1e9
    gd = nb * steps / (ev_d * 1e-3) / 1e9
    out["q4_0_codec"] = {"metric": "GGUF Q4_0 codec HBM GB/s (quantize + dequantize)",
                         "value": round(2 * nb * steps / ((ev_q + ev_d) * 1e-3) / 1e9, 1), "unit": "GB/s",
                         "quantize": {"GB/s": round(gq, 1), "us": round(ev_q * 1e3 / steps, 1), "frac": round(gq / HBM_PEAK_GBS, 4)},
                         "dequantize": {"GB/s": round(gd, 1), "us": round(ev_d * 1e3 / steps, 1), "frac": round(gd / HBM_PEAK_GBS, 4)},
                         "config": {"workload": "codec", "N": wl.N, "K": wl.K, "w_dtype": "bf16", "format": "Q4_0"}}
    del blocks, d, w

    # packed zero-points of a [28672, 256]-group table (pack + unpack)
    zt = torch.randint(0, 16, (28672, 256), dtype=torch.uint8, device=dev)
    zp = w4.pack_zeros(zt)
    zu = torch.empty_like(zt)
    ev_p, _ = time_graph(lambda i: w4.pack_zeros(zt, out=zp), 20, 2000, 200, 1)
    ev_u, _ = time_graph(lambda i: w4.unpack_zeros(zp, 256, out=zu), 20, 2000, 200, 1)
    zb = zt.numel() + zp.numel()
    out["packed_zeros"] = {"metric": "zero-point pack / unpack HBM GB/s", "unit": "GB/s",
                           "pack": {"GB/s": round(zb * 2000 / (ev_p * 1e-3) / 1e9, 1), "us": round(ev_p * 1e3 / 2000, 2)},
                           "unpack": {"GB/s": round(zb * 2000 / (ev_u * 1e-3) / 1e9, 1), "us": round(ev_u * 1e3 / 2000, 2)},
                           "config": {"N": 28672, "NG": 256}}
    return out


def _repeat(fn, seconds):
    n, t0 = 0, time.perf_counter()
    while True:
        fn()
        n += 1
        if time.perf_counter() - t0 >= seconds:
            return n, time.perf_counter() - t0


def cpu_baseline(seconds=10.0, stage_seconds=3.0, prefill_seconds=8.0):
    """The oracle, untuned, on bounded samples of the two linear workloads,
    with NumPy's BLAS allowed every core this process may run on:

    * decode: the linear (dequantize to bf16, fp64 matmul, bias) on the first
      1024 of the 14336 weight rows, repeated for `seconds`; bytes scaled per
      row.  Its quantize_pack and dequantize stages on the same rows follow.
    * prefill: the act-order linear on the first 128 of the 4096 weight rows
      (all 2048 activation rows), repeated for `prefill_seconds`; flops
      2 M rows K per repetition."""
    from oracle import w4_oracle as O
    from int4_group_wise_amd.workloads import workload, generate, bf16_bits
    from threadpoolctl import threadpool_limits, threadpool_info
    cores = len(os.sched_getaffinity(0))
    out = {}
    with threadpool_limits(limits=cores):
        blas_threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
        wl = workload("decode")
        t = generate(wl)
        rows = 1024
        wr = t["w"][:rows].numpy()
        codes, sc, z = O.quantize_pack(wr, wl.G, O.ASYM)
        xb = bf16_bits(t["x"])
        bb = bf16_bits(t["bias"])[:rows]
        n, el = _repeat(lambda: O.linear(xb, codes, sc, z, None, wl.K, wl.G, O.ASYM, bb), seconds)
        per_row = algorithmic_bytes_linear(wl.M, wl.N, wl.K, wl.G, True, True) / wl.N
        gbs = per_row * rows * n / el / 1e9
        ng = (wl.K + wl.G - 1) // wl.G
        packed = rows * ((wl.K + 1) // 2 + 5 * ng)
        nq, tq = _repeat(lambda: O.quantize_pack(wr, wl.G, O.ASYM), stage_seconds)
        nd, td = _repeat(lambda: O.dequantize(codes, sc, z, None, wl.K, wl.G, O.ASYM, "bf16"), stage_seconds)
        stages = {"quantize_pack": {"GB/s": round((rows * wl.K * 4 + packed) * nq / tq / 1e9, 4), "repetitions": nq,
                                    "seconds": round(tq, 1)},
                  "dequantize_bf16": {"GB/s": round((packed + rows * wl.K * 2) * nd / td / 1e9, 4), "repetitions": nd,
                                      "seconds": round(td, 1)}}
        del t
        # prefill: act-order zero-point weight, 128 output features
        wp = workload("prefill")
        tp = generate(wp)
        prow = 128
        gnp = tp["g_idx"].numpy()
        pc, ps, pz = O.quantize_pack(tp["w"][:prow].numpy(), wp.G, O.ASYM, gnp)
        xp = bf16_bits(tp["x"])
        npf, tpf = _repeat(lambda: O.linear(xp, pc, ps, pz, gnp, wp.K, wp.G, O.ASYM, None), prefill_seconds)
        tfs = 2.0 * wp.M * prow * wp.K * npf / tpf / 1e12
        out["prefill"] = {"value": round(tfs, 5), "unit": "TFLOP/s", "cores": cores, "blas_threads": blas_threads,
                          "kind": "oracle",
                          "sample": f"oracle act-order linear (dequantize to bf16 through g_idx, fp64 matmul) on the "
                                    f"first {prow} of {wp.N} weight rows with all {wp.M} activation rows of the "
                                    f"prefill workload, {npf} repetitions in {tpf:.1f} s"}
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": cores, "blas_threads": blas_threads, "kind": "oracle",
            "sample": f"oracle linear (dequantize to bf16, fp64 matmul, bias) on the first {rows} of "
                      f"{wl.N} weight rows of the decode workload, {n} repetitions in {el:.1f} s, "
                      f"bytes scaled per row; stages: quantize_pack (fp32 rows in) and dequantize "
                      f"(bf16 out) on the same rows; NumPy's element-wise steps run on one thread, "
                      f"the fp64 matmul on blas_threads",
            "stages": stages, "prefill": out["prefill"]}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20000)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--counters", action="store_true",
                    help="only the eager launches profiled by rocprofv3 --pmc (no JSON line)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    from int4_group_wise_amd import w4
    w4.load()
    if args.counters:
        run_counters(w4)
        return

    wl, nbytes, ev_ms, host_ms, rot = bench_decode(w4, args.steps, args.warmup)
    us_per = ev_ms * 1e3 / args.steps
    gbs = nbytes * args.steps / (ev_ms * 1e-3) / 1e9
    line = {
        "metric": "W4A16 linear: GEMV HBM GB/s (%peak) M=1; GEMM TFLOPS (%MFMA peak) M=2048",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ev_ms / args.steps, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode", "M": wl.M, "N": wl.N, "K": wl.K, "G": wl.G, "mode": wl.mode,
                   "bias": True, "weight_copies_rotated": rot.count,
                   "rotated_bytes": rot.count * rot.bytes_per_set,
                   "algorithmic_bytes_per_step": nbytes, "host_ms": round(host_ms, 3)},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                     "kernel": "gemv_stream_kernel<7, 1, 2, 1>", "us_per_launch": round(us_per, 3)},
    }
    del rot
    torch.cuda.empty_cache()
    floor = bench_streaming_floor(nbytes)
    line["roofline"]["practical_peak"] = floor["GB/s"]
    line["roofline"]["practical_peak_source"] = floor
    torch.cuda.empty_cache()
    if not args.no_secondary:
        line["secondary"] = {"decode_hot_cache": bench_decode_hot(w4)}
        line["secondary"].update(bench_secondary(w4))
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
