"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/w4.h declares, and rejects malformed requests on the
host before any launch, returning a status and a message."""
import ctypes
import os
import re

import pytest

from int4_group_wise_amd import w4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(w4.library_path()):
        from int4_group_wise_amd import build
        build.build()
    return w4.load()


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "w4.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_0-9]+\s*\*?\s*(w4_[a-z_0-9]+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for f in ("w4_quantize_pack", "w4_dequantize", "w4_linear", "w4_linear_workspace_bytes",
              "w4_linear_grad_input", "w4_linear_grad_input_workspace_bytes",
              "w4_lora_merge", "w4_lora_merge_workspace_bytes",
              "w4_pack_zeros", "w4_unpack_zeros", "w4_q4_0_quantize", "w4_q4_0_dequantize",
              "w4_abi_version", "w4_status_string", "w4_last_error"):
        assert f in names


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_library_has_gfx950_code_object():
    data = open(w4.library_path(), "rb").read()
    assert b"gfx950" in data


def test_version_and_status_strings(lib):
    assert lib.w4_abi_version() == 2
    assert lib.w4_status_string(0) == b"ok"
    assert lib.w4_status_string(1) == b"invalid argument"
    assert lib.w4_status_string(2) == b"unsupported"
    assert lib.w4_status_string(3) == b"HIP error"


FAKE = ctypes.c_void_p(1 << 20)          # aligned, never dereferenced: calls fail before launch
ODD = ctypes.c_void_p((1 << 20) + 2)


@pytest.mark.parametrize("args,status,msg", [
    # (w, dtype, N, K, G, mode, g_idx, codes, scales, zeros, stream)
    ((FAKE, 0, 0, 16, 8, 0, None, FAKE, FAKE, None, None), 1, "N and K"),
    ((FAKE, 0, 4, 0, 8, 0, None, FAKE, FAKE, None, None), 1, "N and K"),
    ((FAKE, 0, 4, 16, 12, 0, None, FAKE, FAKE, None, None), 1, "group size"),
    ((FAKE, 0, 4, 16, 0, 0, None, FAKE, FAKE, None, None), 1, "group size"),
    ((FAKE, 0, 4, 16, -2, 0, None, FAKE, FAKE, None, None), 1, "group size"),
    ((FAKE, 0, 4, 100, 4, 0, None, FAKE, FAKE, None, None), 1, "group size"),
    ((FAKE, 7, 4, 100, -1, 0, None, FAKE, FAKE, None, None), 1, "w_dtype"),   # per-channel G passes
    ((FAKE, 7, 4, 100, 100, 0, None, FAKE, FAKE, None, None), 1, "w_dtype"),  # G = K passes
    ((FAKE, 7, 4, 100, 101, 0, None, FAKE, FAKE, None, None), 1, "w_dtype"),  # G > K passes
    ((FAKE, 0, 4, 16, 8, 7, None, FAKE, FAKE, None, None), 1, "mode"),
    ((FAKE, 0, 4, 16, 8, 1, None, FAKE, FAKE, None, None), 1, "zero-points"),
    ((FAKE, 0, 4, 16, 8, 0, None, FAKE, FAKE, FAKE, None), 1, "no zero-points"),
    ((FAKE, 5, 4, 16, 8, 0, None, FAKE, FAKE, None, None), 1, "w_dtype"),
    ((None, 0, 4, 16, 8, 0, None, FAKE, FAKE, None, None), 1, "non-NULL"),
    ((ODD, 0, 4, 16, 8, 0, None, FAKE, FAKE, None, None), 1, "aligned"),
    ((FAKE, 0, 4, 1 << 20, 8, 0, None, FAKE, FAKE, None, None), 2, "groups per row"),
    ((FAKE, 0, 4, (1 << 30) + 1, 8, 0, None, FAKE, FAKE, None, None), 2, "2^30"),
])
def test_quantize_pack_rejects(lib, args, status, msg):
    assert lib.w4_quantize_pack(*args) == status
    assert msg in lib.w4_last_error().decode()


def test_dequantize_rejects(lib):
    assert lib.w4_dequantize(FAKE, FAKE, None, None, 4, 16, 8, 0, FAKE, 9, None) == 1
    assert "out_dtype" in lib.w4_last_error().decode()
    assert lib.w4_dequantize(FAKE, None, None, None, 4, 16, 8, 0, FAKE, 1, None) == 1
    assert lib.w4_dequantize(FAKE, FAKE, None, ODD, 4, 16, 8, 0, FAKE, 1, None) == 1
    assert "g_idx" in lib.w4_last_error().decode()


def test_linear_rejects_and_workspace(lib):
    # M = 0 is an empty batch: nothing to do, no launch
    assert lib.w4_linear(FAKE, 0, FAKE, FAKE, None, None, 4, 16, 8, 0, None, FAKE, None, 0, None) == 0
    assert lib.w4_last_error() == b""
    assert lib.w4_linear(FAKE, -1, FAKE, FAKE, None, None, 4, 16, 8, 0, None, FAKE, None, 0, None) == 1
    assert lib.w4_linear(None, 2, FAKE, FAKE, None, None, 4, 16, 8, 0, None, FAKE, None, 0, None) == 1
    assert lib.w4_linear(FAKE, 2, FAKE, FAKE, None, None, 4, 16, 8, 0, ODD, FAKE, None, 0, None) == 1
    # prefill sizes need the bf16 weight staged in a workspace
    need = lib.w4_linear_workspace_bytes(64, 32, 128, 32, 0, 0)
    assert need == 32 * 128 * 2
    assert lib.w4_linear_workspace_bytes(16, 32, 128, 32, 0, 0) == 0
    assert lib.w4_linear(FAKE, 64, FAKE, FAKE, None, None, 32, 128, 32, 0, None, FAKE, None, 0, None) == 1
    assert "workspace" in lib.w4_last_error().decode()
    assert lib.w4_linear(FAKE, 64, FAKE, FAKE, None, None, 32, 128, 32, 0, None, FAKE, FAKE, need - 1, None) == 1
    # batched decode (4 < M <= 16): the one-launch kernel (K % 1024 == 0, at
    # most 32 groups, 16 with zero-points, in a quarter of K) needs nothing
    assert lib.w4_linear_workspace_bytes(16, 28672, 8192, 64, 0, 0) == 0
    assert lib.w4_linear_workspace_bytes(16, 64, 8192, 64, 0, 0) == 0
    assert lib.w4_linear_workspace_bytes(8, 256, 4096, 128, 1, 0) == 0
    # other batched shapes take the K-split kernel, which splits K when the
    # grid would hold fewer than 4096 waves (16 rows each), doubling within
    # the 512-column batches: fp32 partials [splits, M, N]
    assert lib.w4_linear_workspace_bytes(16, 28672, 8192, 32, 0, 0) == 4 * 16 * 28672 * 4   # 64 groups a quarter
    assert lib.w4_linear_workspace_bytes(16, 64, 8320, 64, 0, 0) == 16 * 16 * 64 * 4        # K % 1024 != 0
    assert lib.w4_linear_workspace_bytes(16, 100, 512, 64, 0, 0) == 0          # one batch: no split
    assert lib.w4_linear_workspace_bytes(4, 28672, 8192, 64, 0, 0) == 0        # M <= 4: other kernels
    assert lib.w4_linear_workspace_bytes(16, 28672, 8192, 64, 0, 1) == 0       # act-order: generic kernel
    assert lib.w4_linear_workspace_bytes(16, 28672, 8192, 48, 0, 0) == 0       # G not 32, 64 or k 128
    split = lib.w4_linear_workspace_bytes(8, 256, 4224, 128, 1, 0)
    assert split > 0
    assert lib.w4_linear(FAKE, 8, FAKE, FAKE, FAKE, None, 256, 4224, 128, 1, None, FAKE, FAKE, split - 1, None) == 1
    assert "workspace" in lib.w4_last_error().decode()


def test_linear_noalloc_rejects_before_any_launch(lib):
    # the scratch array's size is fixed; shapes needing more are refused on the host
    cap = lib.w4_linear_noalloc_max_scratch_bytes()
    assert cap == 16 << 20
    assert lib.w4_linear_workspace_bytes(64, 8192, 8192, 128, 0, 0) > cap
    assert lib.w4_linear_noalloc(FAKE, 64, FAKE, FAKE, None, None, 8192, 8192, 128, 0, None, FAKE, None) == 2
    assert "scratch" in lib.w4_last_error().decode()
    assert lib.w4_linear_noalloc(FAKE, 0, FAKE, FAKE, None, None, 4, 16, 8, 0, None, FAKE, None) == 0
    assert lib.w4_linear_noalloc(FAKE, 2, FAKE, FAKE, None, None, 4, 16, 8, 3, None, FAKE, None) == 1


def test_grad_input_rejects_and_workspace(lib):
    f = lib.w4_linear_grad_input
    assert f(FAKE, 0, FAKE, FAKE, None, None, 4, 16, 8, 0, FAKE, None, 0, None) == 0
    assert lib.w4_last_error() == b""
    assert f(FAKE, -1, FAKE, FAKE, None, None, 4, 16, 8, 0, FAKE, FAKE, 1 << 20, None) == 1
    assert f(None, 2, FAKE, FAKE, None, None, 4, 16, 8, 0, FAKE, FAKE, 1 << 20, None) == 1
    assert f(FAKE, 2, FAKE, FAKE, None, None, 4, 16, 8, 0, ODD, FAKE, 1 << 20, None) == 1
    assert "aligned" in lib.w4_last_error().decode()
    assert f(FAKE, 2, FAKE, FAKE, FAKE, None, 4, 16, 8, 0, FAKE, FAKE, 1 << 20, None) == 1   # zeros with signed codes
    # M <= 16: fp32 partials of row slices; M > 16: the transposed bf16 weight
    small = lib.w4_linear_grad_input_workspace_bytes(2, 14336, 4096, 128, 1, 0)
    assert small > 0 and small % (2 * 4096 * 4) == 0 and small <= 16 << 20
    assert lib.w4_linear_grad_input_workspace_bytes(64, 32, 128, 32, 0, 0) == 32 * 128 * 2
    need = lib.w4_linear_grad_input_workspace_bytes(2, 4, 16, 8, 0, 0)
    assert f(FAKE, 2, FAKE, FAKE, None, None, 4, 16, 8, 0, FAKE, FAKE, need - 1, None) == 1
    assert "workspace" in lib.w4_last_error().decode()
    assert f(FAKE, 2, FAKE, FAKE, None, None, 4, 16, 8, 0, FAKE, None, need, None) == 1


def test_lora_merge_rejects_and_workspace(lib):
    f = lib.w4_lora_merge
    B2 = ctypes.c_void_p((1 << 21))                 # a second buffer, disjoint from FAKE's spans
    B3 = ctypes.c_void_p((1 << 22))
    SC = ctypes.c_void_p((1 << 20) + 1024)          # scales, merged in place with the codes
    ok = (FAKE, SC, None, None, 4, 16, 8, 0, B2, B3, 2, 1.0, FAKE, SC, None, None, 0, None)

    def call(**kw):
        args = list(ok)
        names = ["codes", "scales", "zeros", "g_idx", "N", "K", "G", "mode", "a", "b", "rank", "c",
                 "co", "so", "zo", "ws", "wsb", "stream"]
        for k, v in kw.items():
            args[names.index(k)] = v
        return f(*args)

    assert call(rank=0) == 1 and "rank" in lib.w4_last_error().decode()
    assert call(rank=65) == 2 and "rank" in lib.w4_last_error().decode()
    assert call(a=None) == 1 and "non-NULL" in lib.w4_last_error().decode()
    assert call(zo=FAKE) == 1 and "zeros_out" in lib.w4_last_error().decode()
    assert call(co=ODD) == 1 and "aligned" in lib.w4_last_error().decode()
    # an output that overlaps another input (codes_out on top of scales)
    assert call(co=ctypes.c_void_p((1 << 20) + 16), so=B3) == 1
    assert "overlaps" in lib.w4_last_error().decode()
    # one pass for contiguous power-of-two groups up to 512, else the fp32 merged weight
    assert lib.w4_lora_merge_workspace_bytes(4, 16, 8, 0, 0, 2) == 0
    assert lib.w4_lora_merge_workspace_bytes(4, 16, 8, 0, 1, 2) == 4 * 16 * 4
    assert lib.w4_lora_merge_workspace_bytes(4, 4096, -1, 0, 0, 2) == 4 * 4096 * 4
    assert lib.w4_lora_merge_workspace_bytes(4, 640, 40, 0, 0, 2) == 4 * 640 * 4
    assert lib.w4_lora_merge_workspace_bytes(4, 640, 64, 0, 0, 64) == 0
    assert call(g_idx=FAKE, wsb=4 * 16 * 4 - 1, ws=B2) == 1 and "workspace" in lib.w4_last_error().decode()


def test_formats_reject(lib):
    assert lib.w4_q4_0_quantize(FAKE, 0, 4, 48, FAKE, None) == 1 and "multiple of 32" in lib.w4_last_error().decode()
    assert lib.w4_q4_0_quantize(FAKE, 0, 0, 64, FAKE, None) == 1
    assert lib.w4_q4_0_quantize(FAKE, 5, 4, 64, FAKE, None) == 1 and "w_dtype" in lib.w4_last_error().decode()
    assert lib.w4_q4_0_quantize(ODD, 0, 4, 64, FAKE, None) == 1 and "aligned" in lib.w4_last_error().decode()
    assert lib.w4_q4_0_dequantize(FAKE, 4, 64, FAKE, 9, None) == 1 and "out_dtype" in lib.w4_last_error().decode()
    assert lib.w4_q4_0_dequantize(None, 4, 64, FAKE, 1, None) == 1
    assert lib.w4_q4_0_quantize(FAKE, 0, 4, (1 << 30) + 32, FAKE, None) == 2
    assert lib.w4_pack_zeros(FAKE, 0, 4, FAKE, None) == 1
    assert lib.w4_pack_zeros(None, 2, 4, FAKE, None) == 1
    assert lib.w4_unpack_zeros(FAKE, 2, 0, FAKE, None) == 1


def test_binding_validates_before_calling():
    import torch
    with pytest.raises(ValueError):
        w4.quantize_pack(torch.zeros(4, 8), 8)          # CPU tensor
    with pytest.raises(ValueError):
        w4._mode("int8")
