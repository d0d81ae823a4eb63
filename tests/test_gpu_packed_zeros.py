"""Zero-points packed two per byte (W4_ASYM_PACKED) read directly by every
dequantize, linear and input-gradient kernel.

The packed table is the w4_pack_zeros layout (group 2j in the low nibble of
byte j; the keras dense.py diff page keeps kernel_zero as 4-bit values, the
LoopQ packed_weight.py page fixes the nibble order of the codes).  Each case
checks the packed call bit for bit against the same call with one zero-point
per byte (whose parity with the oracle the other GPU tests establish), and
the dequantized weight against the oracle fed with the oracle's own unpacking
of the packed table.  Shapes reach every kernel family, with odd group counts
(the last byte's high nibble unused)."""
import numpy as np
import pytest
import torch

from oracle import w4_oracle as O
from int4_group_wise_amd import w4
from int4_group_wise_amd.workloads import workload, generate, bf16_bits

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _weights(N, K, G, act, seed):
    gen = torch.Generator().manual_seed(seed)
    w = torch.randn(N, K, generator=gen) * 0.02
    ng = O.n_groups(K, G)
    g_idx = (torch.randperm(K, generator=gen) // G % ng).to(torch.int32) if act else None
    gi = None if g_idx is None else g_idx.to(DEV)
    codes, scales, zeros = w4.quantize_pack(w.to(DEV), G, "asym", gi)
    packed = w4.pack_zeros(zeros)
    return g_idx, gi, codes, scales, zeros, packed


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy()


LINEAR_CASES = [
    # M, N, K, G, act-order: the kernel each reaches
    (1, 300, 4096, 128, False),     # streaming decode GEMV
    (1, 300, 4096, -1, False),      # streaming decode GEMV, one group per row (odd count)
    (1, 200, 2080, 32, False),      # decode GEMV, 65 groups
    (3, 200, 1024, 128, False),     # matrix-core decode
    (3, 96, 640, 32, False),        # matrix-core decode, transposed quarters, 20 groups
    (16, 256, 8192, 64, False),     # batched decode, split K
    (12, 200, 1152, 128, False),    # batched decode, 9 groups
    (4, 64, 512, 128, True),        # act-order decode (generic)
    (1, 300, 4096, 128, True),      # act-order decode on the matrix cores
    (1, 70, 2048, 128, True),       # the same, 16 groups (one half)
    (16, 256, 4096, 128, False),    # one-launch batched decode
    (12, 16500, 2048, 64, False),   # one-launch batched decode, 258 workgroups
    (64, 256, 1024, 128, True),     # prefill, tiled weight, act-order
    (48, 256, 2048, 128, False),    # prefill, tiled weight
    (40, 130, 640, 64, False),      # prefill, row-major weight (N % 128 != 0), 10 groups
    (20, 100, 1000, 40, False),     # prefill, K % 64 != 0, 25 groups
]


@pytest.mark.parametrize("case", LINEAR_CASES, ids=lambda c: "M%d_N%d_K%d_G%d%s" % (c[0], c[1], c[2], c[3], "_act" if c[4] else ""))
def test_linear_with_packed_zero_points(case):
    M, N, K, G, act = case
    g_idx, gi, codes, scales, zeros, packed = _weights(N, K, G, act, M + N + K)
    x = (torch.randn(M, K, generator=torch.Generator().manual_seed(K)).to(torch.bfloat16)).to(DEV)
    bias = (torch.randn(N, generator=torch.Generator().manual_seed(N)) * 0.01).to(torch.bfloat16).to(DEV)
    y_byte = w4.linear(x, codes, scales, zeros, gi, K, G, "asym", bias)
    y_pack = w4.linear(x, codes, scales, packed, gi, K, G, "asym_packed", bias)
    torch.cuda.synchronize()
    assert torch.equal(y_pack.view(torch.int16), y_byte.view(torch.int16)), f"packed zero-points change y {case}"
    # the linear against the oracle, with the packed table unpacked by the oracle
    NG = O.n_groups(K, G)
    oz = O.unpack_zeros(packed.cpu().numpy(), NG)
    gnp = None if g_idx is None else g_idx.numpy()
    yr = O.linear(bf16_bits(x.cpu()), codes.cpu().numpy(), scales.cpu().numpy(), oz, gnp, K, G, O.ASYM,
                  bf16_bits(bias.cpu()))
    yg = y_pack.float().cpu().numpy().astype(np.float64)
    assert np.linalg.norm(yg - yr) / np.linalg.norm(yr) <= 5e-3
    assert np.abs(yg - yr).max() <= 2e-2 * np.abs(yr).max()


DEQUANT_CASES = [
    (37, 2048, 128, False),         # row dequantizer
    (20, 1000, 40, False),          # general dequantizer, 25 groups
    (16, 1024, 64, True),           # act-order table dequantizer
    (10, 256, 32, True),            # act-order, short rows (staged tables)
    (9, 300, 8, True),              # act-order, 38 groups
]


@pytest.mark.parametrize("case", DEQUANT_CASES, ids=lambda c: "N%d_K%d_G%d%s" % (c[0], c[1], c[2], "_act" if c[3] else ""))
def test_dequantize_with_packed_zero_points(case):
    N, K, G, act = case
    g_idx, gi, codes, scales, zeros, packed = _weights(N, K, G, act, N + K)
    NG = O.n_groups(K, G)
    oz = O.unpack_zeros(packed.cpu().numpy(), NG)
    assert np.array_equal(oz, zeros.cpu().numpy())          # the pack kernel, checked by the oracle's unpack
    gnp = None if g_idx is None else g_idx.numpy()
    for dt, kind in ((torch.bfloat16, "bf16"), (torch.float32, "f32")):
        d = w4.dequantize(codes, scales, packed, gi, K, G, "asym_packed", dt)
        torch.cuda.synchronize()
        ref = O.dequantize(codes.cpu().numpy(), scales.cpu().numpy(), oz, gnp, K, G, O.ASYM, kind)
        got = _bits(d) if kind == "bf16" else d.cpu().numpy().view(np.uint32)
        exp = ref.view(np.int16) if kind == "bf16" else ref.view(np.uint32)
        assert np.array_equal(got, exp), f"{kind} dequantize differs {case}"


@pytest.mark.parametrize("M,N,K,G,act", [(1, 512, 1024, 128, False), (3, 300, 640, 64, False),
                                         (32, 256, 512, 64, True), (24, 200, 384, 32, False)])
def test_grad_input_with_packed_zero_points(M, N, K, G, act):
    g_idx, gi, codes, scales, zeros, packed = _weights(N, K, G, act, M + K)
    dy = (torch.randn(M, N, generator=torch.Generator().manual_seed(N)).to(torch.bfloat16)).to(DEV)
    a = w4.linear_grad_input(dy, codes, scales, zeros, gi, K, G, "asym")
    b = w4.linear_grad_input(dy, codes, scales, packed, gi, K, G, "asym_packed")
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_packed_mode_is_refused_where_zero_points_are_written():
    _, _, codes, scales, zeros, packed = _weights(8, 256, 32, False, 1)
    lib = w4.load()
    w = torch.zeros(8, 256, device=DEV)
    c = torch.empty_like(codes)
    s = torch.empty_like(scales)
    st = lib.w4_quantize_pack(w.data_ptr(), 0, 8, 256, 32, 2, None, c.data_ptr(), s.data_ptr(), packed.data_ptr(), None)
    assert st == 2 and b"w4_pack_zeros" in lib.w4_last_error()
    la = torch.zeros(256, 2, device=DEV)
    lb = torch.zeros(2, 8, device=DEV)
    with pytest.raises(w4.W4Error):
        w4.lora_merge(codes, scales, packed, None, 256, 32, "asym_packed", la, lb, 1.0)
