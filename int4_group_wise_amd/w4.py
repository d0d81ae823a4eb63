"""Thin Python binding of libw4.so (C ABI in include/w4.h).

Argument marshalling only: these functions check tensor dtypes, shapes and
devices, allocate outputs with torch on the tensors' device, and pass raw
device pointers plus the current HIP stream to the library.  Every step of the
computation runs in the library's HIP kernels; there is no fallback.  If the
library is not built, the first call raises W4Error.
"""
from __future__ import annotations

import ctypes
import os

import torch

SYM = 0    # W4_SYM: signed two's-complement nibbles
ASYM = 1   # W4_ASYM: unsigned nibbles with per-group zero-points
ASYM_PACKED = 2   # W4_ASYM_PACKED: the same, zero-points packed two per byte
_F32, _BF16 = 0, 1

_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "HIP error"}
_LIB = None


class W4Error(RuntimeError):
    """A libw4 call failed (status and the library's message)."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


ABI_VERSION = 2   # W4_ABI_VERSION of include/w4.h


def library_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "libw4.so")


def load() -> ctypes.CDLL:
    """Load libw4.so once and declare its signatures."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise W4Error(-1, f"{path} is not built (run: python -m int4_group_wise_amd.build)")
    lib = ctypes.CDLL(path)
    P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    lib.w4_abi_version.restype = I32
    lib.w4_abi_version.argtypes = []
    if lib.w4_abi_version() != ABI_VERSION:
        raise W4Error(-1, f"{path} has ABI version {lib.w4_abi_version()}, this binding needs {ABI_VERSION} (rebuild it)")
    lib.w4_status_string.restype = ctypes.c_char_p
    lib.w4_status_string.argtypes = [I32]
    lib.w4_last_error.restype = ctypes.c_char_p
    lib.w4_last_error.argtypes = []
    lib.w4_quantize_pack.restype = I32
    lib.w4_quantize_pack.argtypes = [P, I32, I64, I64, I64, I32, P, P, P, P, P]
    lib.w4_dequantize.restype = I32
    lib.w4_dequantize.argtypes = [P, P, P, P, I64, I64, I64, I32, P, I32, P]
    lib.w4_linear_workspace_bytes.restype = SZ
    lib.w4_linear_workspace_bytes.argtypes = [I64, I64, I64, I64, I32, I32]
    lib.w4_linear.restype = I32
    lib.w4_linear.argtypes = [P, I64, P, P, P, P, I64, I64, I64, I32, P, P, P, SZ, P]
    lib.w4_linear_noalloc_max_scratch_bytes.restype = SZ
    lib.w4_linear_noalloc_max_scratch_bytes.argtypes = []
    lib.w4_linear_noalloc.restype = I32
    lib.w4_linear_noalloc.argtypes = [P, I64, P, P, P, P, I64, I64, I64, I32, P, P, P]
    lib.w4_linear_grad_input_workspace_bytes.restype = SZ
    lib.w4_linear_grad_input_workspace_bytes.argtypes = [I64, I64, I64, I64, I32, I32]
    lib.w4_linear_grad_input.restype = I32
    lib.w4_linear_grad_input.argtypes = [P, I64, P, P, P, P, I64, I64, I64, I32, P, P, SZ, P]
    lib.w4_lora_merge_workspace_bytes.restype = SZ
    lib.w4_lora_merge_workspace_bytes.argtypes = [I64, I64, I64, I32, I32, I64]
    lib.w4_lora_merge.restype = I32
    lib.w4_lora_merge.argtypes = [P, P, P, P, I64, I64, I64, I32, P, P, I64, ctypes.c_float, P, P, P, P, SZ, P]
    lib.w4_pack_zeros.restype = I32
    lib.w4_pack_zeros.argtypes = [P, I64, I64, P, P]
    lib.w4_unpack_zeros.restype = I32
    lib.w4_unpack_zeros.argtypes = [P, I64, I64, P, P]
    lib.w4_q4_0_quantize.restype = I32
    lib.w4_q4_0_quantize.argtypes = [P, I32, I64, I64, P, P]
    lib.w4_q4_0_dequantize.restype = I32
    lib.w4_q4_0_dequantize.argtypes = [P, I64, I64, P, I32, P]
    _LIB = lib
    return lib


def _check(lib, status: int) -> None:
    if status != 0:
        raise W4Error(status, lib.w4_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype, shape=None) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _mode(mode) -> int:
    if mode in (SYM, "sym"):
        return SYM
    if mode in (ASYM, "asym"):
        return ASYM
    if mode in (ASYM_PACKED, "asym_packed"):
        return ASYM_PACKED
    raise ValueError("mode must be 'sym', 'asym' or 'asym_packed'")


PER_CHANNEL = -1   # group size: one group per row (W4_PER_CHANNEL)


def n_groups(K: int, G: int) -> int:
    """Groups per row: ceil(K / G), or 1 for per-channel (G = -1 or G >= K)."""
    if G == PER_CHANNEL or G >= K:
        return 1
    return -(-K // G) if G > 0 else 0


def _format_args(N, K, G, mode, codes, scales, zeros, g_idx):
    NG = n_groups(K, G)
    _dev(codes, "codes", torch.uint8, (N, (K + 1) // 2))
    _dev(scales, "scales", torch.float32, (N, NG))
    if mode in (ASYM, ASYM_PACKED):
        if zeros is None:
            raise ValueError("zero-point mode needs zeros")
        _dev(zeros, "zeros", torch.uint8, (N, NG) if mode == ASYM else (N, (NG + 1) // 2))
    elif zeros is not None:
        raise ValueError("signed mode takes no zeros")
    if g_idx is not None:
        _dev(g_idx, "g_idx", torch.int32, (K,))


def quantize_pack(w: torch.Tensor, G: int, mode="sym", g_idx: torch.Tensor | None = None, out=None):
    """Quantize ``w`` [N, K] (fp32 or bf16, on the GPU) group-wise and pack it.
    Returns ``(codes uint8 [N, ceil(K/2)], scales fp32 [N, ceil(K/G)],
    zeros uint8 [N, ceil(K/G)] or None)``; ``out`` may hold that tuple
    preallocated.  ``G = -1`` (or any G >= K) is per-channel: one group per
    row."""
    lib = load()
    mode = _mode(mode)
    if w.dim() != 2:
        raise ValueError("w must be a matrix")
    if w.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("w must be float32 or bfloat16")
    _dev(w, "w", w.dtype)
    N, K = w.shape
    NG = n_groups(K, G)
    if out is None:
        codes = torch.empty((N, (K + 1) // 2), dtype=torch.uint8, device=w.device)
        scales = torch.empty((N, NG), dtype=torch.float32, device=w.device)
        zeros = torch.empty((N, NG), dtype=torch.uint8, device=w.device) if mode == ASYM else None
    else:
        codes, scales, zeros = out
    if NG > 0:
        _format_args(N, K, G, mode, codes, scales, zeros, None)
    if g_idx is not None:
        _dev(g_idx, "g_idx", torch.int32, (K,))
    _check(lib, lib.w4_quantize_pack(_ptr(w), _BF16 if w.dtype == torch.bfloat16 else _F32,
                                     N, K, G, mode, _ptr(g_idx), _ptr(codes), _ptr(scales),
                                     _ptr(zeros), _stream(w.device)))
    return codes, scales, zeros


def dequantize(codes, scales, zeros, g_idx, K: int, G: int, mode="sym",
               out_dtype=torch.bfloat16, out=None) -> torch.Tensor:
    """Dense weight [N, K] (bf16 or fp32) from packed codes; ``out`` may be a
    preallocated [N, K] tensor of ``out_dtype``."""
    lib = load()
    mode = _mode(mode)
    N = codes.shape[0]
    _format_args(N, K, G, mode, codes, scales, zeros, g_idx)
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("out_dtype must be bfloat16 or float32")
    if out is None:
        out = torch.empty((N, K), dtype=out_dtype, device=codes.device)
    _dev(out, "out", out_dtype, (N, K))
    _check(lib, lib.w4_dequantize(_ptr(codes), _ptr(scales), _ptr(zeros), _ptr(g_idx), N, K, G,
                                  mode, _ptr(out), _BF16 if out_dtype == torch.bfloat16 else _F32,
                                  _stream(codes.device)))
    return out


def linear_workspace_bytes(M: int, N: int, K: int, G: int, mode="sym", has_g_idx=False) -> int:
    lib = load()
    return int(lib.w4_linear_workspace_bytes(M, N, K, G, _mode(mode), int(bool(has_g_idx))))


def linear(x, codes, scales, zeros, g_idx, K: int, G: int, mode="sym", bias=None,
           out=None, workspace=None) -> torch.Tensor:
    """``y = x . dequant(W)^T + bias`` with x bf16 [M, K]; returns bf16 [M, N].
    ``out`` (bf16 [M, N]) and ``workspace`` (uint8, at least
    ``linear_workspace_bytes`` bytes) may be passed in to avoid allocation."""
    lib = load()
    mode = _mode(mode)
    N = codes.shape[0]
    _format_args(N, K, G, mode, codes, scales, zeros, g_idx)
    if x.dim() != 2 or x.shape[1] != K:
        raise ValueError(f"x must be [M, {K}]")
    _dev(x, "x", torch.bfloat16)
    M = x.shape[0]
    if bias is not None:
        _dev(bias, "bias", torch.bfloat16, (N,))
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _dev(out, "out", torch.bfloat16, (M, N))
    need = int(lib.w4_linear_workspace_bytes(M, N, K, G, mode, int(g_idx is not None)))
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib, lib.w4_linear(_ptr(x), M, _ptr(codes), _ptr(scales), _ptr(zeros), _ptr(g_idx),
                              N, K, G, mode, _ptr(bias), _ptr(out), _ptr(workspace), ws_bytes,
                              _stream(x.device)))
    return out


def linear_noalloc(x, codes, scales, zeros, g_idx, K: int, G: int, mode="sym", bias=None, out=None) -> torch.Tensor:
    """``linear`` through w4_linear_noalloc: the library's fixed per-device
    scratch array instead of a workspace (calls that overlap on one GPU race
    on it)."""
    lib = load()
    mode = _mode(mode)
    N = codes.shape[0]
    _format_args(N, K, G, mode, codes, scales, zeros, g_idx)
    if x.dim() != 2 or x.shape[1] != K:
        raise ValueError(f"x must be [M, {K}]")
    _dev(x, "x", torch.bfloat16)
    M = x.shape[0]
    if bias is not None:
        _dev(bias, "bias", torch.bfloat16, (N,))
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _dev(out, "out", torch.bfloat16, (M, N))
    _check(lib, lib.w4_linear_noalloc(_ptr(x), M, _ptr(codes), _ptr(scales), _ptr(zeros), _ptr(g_idx),
                                      N, K, G, mode, _ptr(bias), _ptr(out), _stream(x.device)))
    return out


def linear_grad_input_workspace_bytes(M: int, N: int, K: int, G: int, mode="sym", has_g_idx=False) -> int:
    lib = load()
    return int(lib.w4_linear_grad_input_workspace_bytes(M, N, K, G, _mode(mode), int(bool(has_g_idx))))


def linear_grad_input(dy, codes, scales, zeros, g_idx, K: int, G: int, mode="sym",
                      out=None, workspace=None) -> torch.Tensor:
    """``dx = dy . dequant(W)`` with dy bf16 [M, N]; returns bf16 [M, K].
    ``out`` (bf16 [M, K]) and ``workspace`` (uint8, at least
    ``linear_grad_input_workspace_bytes`` bytes) may be passed in to avoid
    allocation."""
    lib = load()
    mode = _mode(mode)
    N = codes.shape[0]
    _format_args(N, K, G, mode, codes, scales, zeros, g_idx)
    if dy.dim() != 2 or dy.shape[1] != N:
        raise ValueError(f"dy must be [M, {N}]")
    _dev(dy, "dy", torch.bfloat16)
    M = dy.shape[0]
    if out is None:
        out = torch.empty((M, K), dtype=torch.bfloat16, device=dy.device)
    _dev(out, "out", torch.bfloat16, (M, K))
    need = int(lib.w4_linear_grad_input_workspace_bytes(M, N, K, G, mode, int(g_idx is not None)))
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=dy.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib, lib.w4_linear_grad_input(_ptr(dy), M, _ptr(codes), _ptr(scales), _ptr(zeros), _ptr(g_idx),
                                         N, K, G, mode, _ptr(out), _ptr(workspace), ws_bytes,
                                         _stream(dy.device)))
    return out


def lora_merge_workspace_bytes(N: int, K: int, G: int, mode="sym", has_g_idx=False, rank=1) -> int:
    lib = load()
    return int(lib.w4_lora_merge_workspace_bytes(N, K, G, _mode(mode), int(bool(has_g_idx)), rank))


def lora_merge(codes, scales, zeros, g_idx, K: int, G: int, mode, lora_a, lora_b, lora_scale: float,
               out=None, workspace=None):
    """Fold ``lora_scale * (lora_a @ lora_b)`` (lora_a fp32 [K, r], lora_b
    fp32 [r, N]) into the packed weight and quantize again with the same
    grouping.  Returns ``(codes, scales, zeros)``; ``out`` may be that tuple
    preallocated, or the inputs themselves to merge in place."""
    lib = load()
    mode = _mode(mode)
    N = codes.shape[0]
    _format_args(N, K, G, mode, codes, scales, zeros, g_idx)
    if lora_a.dim() != 2 or lora_a.shape[0] != K:
        raise ValueError(f"lora_a must be [{K}, rank]")
    r = lora_a.shape[1]
    _dev(lora_a, "lora_a", torch.float32, (K, r))
    _dev(lora_b, "lora_b", torch.float32, (r, N))
    if out is None:
        out = (torch.empty_like(codes), torch.empty_like(scales), None if zeros is None else torch.empty_like(zeros))
    co, so, zo = out
    _format_args(N, K, G, mode, co, so, zo, None)
    need = int(lib.w4_lora_merge_workspace_bytes(N, K, G, mode, int(g_idx is not None), r))
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=codes.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib, lib.w4_lora_merge(_ptr(codes), _ptr(scales), _ptr(zeros), _ptr(g_idx), N, K, G, mode,
                                  _ptr(lora_a), _ptr(lora_b), r, float(lora_scale), _ptr(co), _ptr(so), _ptr(zo),
                                  _ptr(workspace), ws_bytes, _stream(codes.device)))
    return co, so, zo


def pack_zeros(zeros: torch.Tensor, out=None) -> torch.Tensor:
    """uint8 [N, NG] zero-points -> uint8 [N, ceil(NG/2)], two per byte."""
    lib = load()
    if zeros.dim() != 2:
        raise ValueError("zeros must be a matrix")
    _dev(zeros, "zeros", torch.uint8)
    N, NG = zeros.shape
    if out is None:
        out = torch.empty((N, (NG + 1) // 2), dtype=torch.uint8, device=zeros.device)
    _dev(out, "out", torch.uint8, (N, (NG + 1) // 2))
    _check(lib, lib.w4_pack_zeros(_ptr(zeros), N, NG, _ptr(out), _stream(zeros.device)))
    return out


def unpack_zeros(packed: torch.Tensor, NG: int, out=None) -> torch.Tensor:
    """uint8 [N, ceil(NG/2)] -> uint8 [N, NG]."""
    lib = load()
    _dev(packed, "packed", torch.uint8, (packed.shape[0], (NG + 1) // 2))
    N = packed.shape[0]
    if out is None:
        out = torch.empty((N, NG), dtype=torch.uint8, device=packed.device)
    _dev(out, "out", torch.uint8, (N, NG))
    _check(lib, lib.w4_unpack_zeros(_ptr(packed), N, NG, _ptr(out), _stream(packed.device)))
    return out


def q4_0_quantize(w: torch.Tensor, out=None) -> torch.Tensor:
    """GGUF Q4_0 blocks of ``w`` [N, K] (fp32 or bf16, K % 32 == 0):
    uint8 [N, K/32, 18]."""
    lib = load()
    if w.dim() != 2 or w.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("w must be a float32 or bfloat16 matrix")
    _dev(w, "w", w.dtype)
    N, K = w.shape
    if K % 32:
        raise ValueError("Q4_0 needs K to be a multiple of 32")
    if out is None:
        out = torch.empty((N, K // 32, 18), dtype=torch.uint8, device=w.device)
    _dev(out, "out", torch.uint8, (N, K // 32, 18))
    _check(lib, lib.w4_q4_0_quantize(_ptr(w), _BF16 if w.dtype == torch.bfloat16 else _F32, N, K, _ptr(out),
                                     _stream(w.device)))
    return out


def q4_0_dequantize(blocks: torch.Tensor, out_dtype=torch.bfloat16, out=None) -> torch.Tensor:
    """Dense [N, 32 * nb] weight from Q4_0 blocks uint8 [N, nb, 18]."""
    lib = load()
    if blocks.dim() != 3 or blocks.shape[2] != 18:
        raise ValueError("blocks must be [N, K/32, 18]")
    _dev(blocks, "blocks", torch.uint8)
    N, nb = blocks.shape[0], blocks.shape[1]
    K = 32 * nb
    if out is None:
        out = torch.empty((N, K), dtype=out_dtype, device=blocks.device)
    _dev(out, "out", out_dtype, (N, K))
    _check(lib, lib.w4_q4_0_dequantize(_ptr(blocks), N, K, _ptr(out),
                                       _BF16 if out_dtype == torch.bfloat16 else _F32, _stream(blocks.device)))
    return out
