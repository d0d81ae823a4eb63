"""w4_linear_noalloc: the allocation-free variant of w4_linear (its scratch is
the library's fixed per-device array) gives the same bits as w4_linear with a
caller workspace, on consecutive calls whose second input is smaller, and
rejects shapes whose scratch would not fit."""
import numpy as np
import pytest
import torch

from oracle import w4_oracle as O
from int4_group_wise_amd import w4
from int4_group_wise_amd.workloads import workload, generate, bf16_bits

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _case(M, N, K, G, mode, bias, seed):
    wl = workload("tiny", M=M, N=N, K=K, G=G, mode=mode, bias=bias, bias_std=0.01, seed=seed)
    t = generate(wl)
    codes, scales, zeros = w4.quantize_pack(t["w"].to(DEV), G, mode)
    b = None if t["bias"] is None else t["bias"].to(DEV)
    return wl, t, t["x"].to(DEV), codes, scales, zeros, b


def _check_against_linear(wl, t, x, codes, scales, zeros, b):
    lib = w4.load()
    need = lib.w4_linear_workspace_bytes(wl.M, wl.N, wl.K, wl.G, w4._mode(wl.mode), 0)
    assert 0 < need <= lib.w4_linear_noalloc_max_scratch_bytes()
    y_ref = w4.linear(x, codes, scales, zeros, None, wl.K, wl.G, wl.mode, b)
    y = torch.full((wl.M, wl.N), float("nan"), dtype=torch.bfloat16, device=DEV)
    st = lib.w4_linear_noalloc(x.data_ptr(), wl.M, codes.data_ptr(), scales.data_ptr(),
                               None if zeros is None else zeros.data_ptr(), None, wl.N, wl.K, wl.G,
                               w4._mode(wl.mode), None if b is None else b.data_ptr(), y.data_ptr(),
                               torch.cuda.current_stream().cuda_stream)
    assert st == 0, lib.w4_last_error()
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), "noalloc differs from w4_linear"
    # and the linear's bar against the oracle
    oc, osc, oz = O.quantize_pack(t["w"].numpy(), wl.G, O.SYM if wl.mode == "sym" else O.ASYM)
    yr = O.linear(bf16_bits(t["x"]), oc, osc, oz, None, wl.K, wl.G, O.SYM if wl.mode == "sym" else O.ASYM,
                  None if t["bias"] is None else bf16_bits(t["bias"]))
    yg = y.float().cpu().numpy().astype(np.float64)
    assert np.linalg.norm(yg - yr) / np.linalg.norm(yr) <= 5e-3
    assert np.abs(yg - yr).max() <= 2e-2 * np.abs(yr).max()


def test_noalloc_matches_linear_on_consecutive_calls():
    # a prefill whose staged bf16 weight takes 12 MB of the scratch, then a
    # smaller prefill (512 KB), then the first again
    big = _case(64, 1536, 4096, 128, "sym", "none", 1)
    small = _case(48, 256, 1024, 128, "asym", "randn", 3)
    for c in (big, small, big):
        _check_against_linear(*c)


@pytest.mark.parametrize("M,N,K,G,mode", [(1, 512, 4096, 128, "asym"), (16, 1024, 4096, 64, "sym")])
def test_noalloc_via_binding_and_decode_without_scratch(M, N, K, G, mode):
    # decode and batched decode need no scratch
    wl, t, x, codes, scales, zeros, b = _case(M, N, K, G, mode, "randn", 4)
    assert w4.load().w4_linear_workspace_bytes(M, N, K, G, w4._mode(mode), 0) == 0
    y = w4.linear_noalloc(x, codes, scales, zeros, None, wl.K, wl.G, wl.mode, b)
    y_ref = w4.linear(x, codes, scales, zeros, None, wl.K, wl.G, wl.mode, b)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))


def test_noalloc_rejects_scratch_beyond_its_array():
    lib = w4.load()
    M, N, K = 64, 8192, 8192                          # prefill: 128 MB staged weight
    assert lib.w4_linear_workspace_bytes(M, N, K, 128, 0, 0) > lib.w4_linear_noalloc_max_scratch_bytes()
    x = torch.zeros(M, K, dtype=torch.bfloat16, device=DEV)
    codes = torch.zeros(N, K // 2, dtype=torch.uint8, device=DEV)
    scales = torch.ones(N, K // 128, dtype=torch.float32, device=DEV)
    y = torch.zeros(M, N, dtype=torch.bfloat16, device=DEV)
    st = lib.w4_linear_noalloc(x.data_ptr(), M, codes.data_ptr(), scales.data_ptr(), None, None, N, K, 128, 0,
                               None, y.data_ptr(), None)
    assert st == 2 and b"scratch" in lib.w4_last_error()
    torch.cuda.synchronize()
    assert int(y.view(torch.int16).abs().sum()) == 0   # nothing was launched
