"""Seeded synthetic inputs for the group-wise int4 workloads.

This module only draws random tensors; it holds none of the quantization or
linear arithmetic, so both the HIP path and the CPU oracle can take their
inputs from it.  Every tensor is drawn on the CPU from one
``torch.Generator().manual_seed(seed)`` per workload, in the fixed order:
weight, outlier mask, column permutation, activations, bias.

Named workloads (sizes as in the weight-only int4 layers the pages describe):
  tiny            M=4     N=256    K=512   G=32   signed,     bias of zeros
  decode          M=1     N=14336  K=4096  G=128  zero-point, bias ~N(0, 0.01)
  batched_decode  M=16    N=28672  K=8192  G=64   signed,     0.1% outliers x8
  prefill         M=2048  N=4096   K=4096  G=128  zero-point, act-order g_idx
  codec           -       N=28672  K=8191  G=32   signed,     bf16 weight
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    M: int             # activation rows (0: codec only, no linear)
    N: int             # output features = weight rows
    K: int             # input features = weight columns
    G: int             # group size
    mode: str          # "sym" (signed codes) or "asym" (codes + zero-points)
    w_std: float
    w_dtype: str = "f32"          # "f32" or "bf16"
    outlier_frac: float = 0.0     # fraction of weights multiplied by outlier_mul
    outlier_mul: float = 1.0
    act_order: bool = False       # g_idx = (random permutation of columns) // G
    bias: str = "none"            # "none", "zero" or "randn"
    bias_std: float = 0.0
    seed: int = 0


WORKLOADS = {
    "tiny": Workload("tiny", 4, 256, 512, 32, "sym", 0.02, bias="zero"),
    "decode": Workload("decode", 1, 14336, 4096, 128, "asym", 0.02,
                       bias="randn", bias_std=0.01),
    "batched_decode": Workload("batched_decode", 16, 28672, 8192, 64, "sym", 0.015,
                               outlier_frac=1e-3, outlier_mul=8.0),
    "prefill": Workload("prefill", 2048, 4096, 4096, 128, "asym", 0.02,
                        act_order=True),
    "codec": Workload("codec", 0, 28672, 8191, 32, "sym", 0.02, w_dtype="bf16"),
}


def workload(name: str, **overrides) -> Workload:
    """A named workload, optionally with fields replaced (smaller shapes for
    tests keep the same value distributions)."""
    return replace(WORKLOADS[name], **overrides)


def generate(wl: Workload) -> dict:
    """Draw the inputs of ``wl``.  Returns CPU tensors:
    ``w`` [N, K] fp32 or bf16, ``x`` bf16 [M, K] or None, ``bias`` bf16 [N] or
    None, ``g_idx`` int32 [K] or None."""
    g = torch.Generator().manual_seed(wl.seed)
    w = torch.randn(wl.N, wl.K, generator=g) * wl.w_std
    if wl.outlier_frac > 0:
        mask = torch.rand(wl.N, wl.K, generator=g) < wl.outlier_frac
        w[mask] *= wl.outlier_mul
    if wl.w_dtype == "bf16":
        w = w.to(torch.bfloat16)
    g_idx = None
    if wl.act_order:
        perm = torch.randperm(wl.K, generator=g)
        g_idx = (perm // wl.G).to(torch.int32)
    x = None
    if wl.M > 0:
        x = torch.randn(wl.M, wl.K, generator=g).to(torch.bfloat16)
    bias = None
    if wl.bias == "zero":
        bias = torch.zeros(wl.N, dtype=torch.bfloat16)
    elif wl.bias == "randn":
        bias = (torch.randn(wl.N, generator=g) * wl.bias_std).to(torch.bfloat16)
    return {"w": w, "x": x, "bias": bias, "g_idx": g_idx}


def bf16_bits(t: torch.Tensor):
    """uint16 numpy view of a bf16 CPU tensor's bit patterns."""
    import numpy as np
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)
