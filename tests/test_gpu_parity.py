"""Parity of the HIP path (through the C ABI) with the CPU oracle.

quantize_pack and dequantize must be bit-exact; the linear must reach
normwise relative error <= 5e-3 and per-element error <= 2e-2 * max|y_ref|
against the fp64 oracle, and must be exact on an identity activation (one
non-zero product per output).  The five workloads are compared in full at
their real sizes (every weight row, every output), in the launch
configuration the benchmark times; small shapes cover ragged tails and the
degenerate cases.
"""
import numpy as np
import pytest
import torch

from oracle import w4_oracle as O
from int4_group_wise_amd import w4
from int4_group_wise_amd.workloads import workload, generate, bf16_bits

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
NORM_TOL = 5e-3
ELEM_TOL = 2e-2


def _np_w(w: torch.Tensor) -> np.ndarray:
    if w.dtype == torch.bfloat16:
        return O.bf16_bits_to_f32(bf16_bits(w))
    return w.numpy()


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _mode(m):
    return O.SYM if m in ("sym", 0) else O.ASYM


def _check_codec(w, G, mode, g_idx=None, rows=None, label=""):
    """GPU quantize_pack + dequantize vs the oracle on `rows` (all if None)."""
    N, K = w.shape
    gi = None if g_idx is None else g_idx.to(DEV)
    codes, scales, zeros = w4.quantize_pack(w.to(DEV), G, mode, gi)
    torch.cuda.synchronize()
    sel = np.arange(N) if rows is None else rows
    tsel = torch.from_numpy(sel).to(DEV)
    gnp = None if g_idx is None else g_idx.numpy()
    oc, osc, oz = O.quantize_pack(_np_w(w[torch.from_numpy(sel)]), G, _mode(mode), gnp)
    assert np.array_equal(codes[tsel].cpu().numpy(), oc), f"codes differ {label}"
    assert np.array_equal(scales[tsel].cpu().numpy().view(np.uint32), osc.view(np.uint32)), f"scales differ {label}"
    if oz is not None:
        assert np.array_equal(zeros[tsel].cpu().numpy(), oz), f"zeros differ {label}"
    for dt, kind in ((torch.bfloat16, "bf16"), (torch.float32, "f32")):
        d = w4.dequantize(codes, scales, zeros, gi, K, G, mode, dt)
        got = d[tsel].cpu()
        ref = O.dequantize(oc, osc, oz, gnp, K, G, _mode(mode), kind)
        if kind == "bf16":
            assert np.array_equal(_bits(got), ref), f"bf16 dequant differs {label}"
        else:
            assert np.array_equal(got.numpy().view(np.uint32), ref.view(np.uint32)), f"f32 dequant differs {label}"
        del d
    return codes, scales, zeros, (oc, osc, oz, sel)


def _check_linear(x, codes, scales, zeros, g_idx, K, G, mode, bias, oracle_rows, label=""):
    oc, osc, oz, sel = oracle_rows
    gi = None if g_idx is None else g_idx.to(DEV)
    xb = x.to(DEV)
    bb = None if bias is None else bias.to(DEV)
    y = w4.linear(xb, codes, scales, zeros, gi, K, G, mode, bb)
    y2 = w4.linear(xb, codes, scales, zeros, gi, K, G, mode, bb)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), f"linear not deterministic {label}"
    yg = y[:, torch.from_numpy(sel).to(DEV)].float().cpu().numpy().astype(np.float64)
    bsel = None if bias is None else _bits(bias)[sel]
    gnp = None if g_idx is None else g_idx.numpy()
    yr = O.linear(_bits(x), oc, osc, oz, gnp, K, G, _mode(mode), bsel)
    err = yg - yr
    scale = np.abs(yr).max()
    nrm = np.linalg.norm(yr)
    rel = np.linalg.norm(err) / nrm if nrm > 0 else np.linalg.norm(err)
    assert rel <= NORM_TOL, f"normwise {rel:.3e} {label}"
    assert np.abs(err).max() <= ELEM_TOL * max(scale, 1e-30), f"max err {np.abs(err).max():.3e} vs {scale:.3e} {label}"
    return rel


# ---------------------------------------------------------------------------
# the five workloads at full size
# ---------------------------------------------------------------------------
def test_tiny_full():
    wl = workload("tiny")
    t = generate(wl)
    c, s, z, orc = _check_codec(t["w"], wl.G, wl.mode, label="tiny")
    _check_linear(t["x"], c, s, z, None, wl.K, wl.G, wl.mode, t["bias"], orc, "tiny")


@pytest.mark.timeout(900)
def test_decode_full_size():
    """Every one of the 14336 rows: codes, scales, zero-points, both
    dequantized forms and every output of the linear."""
    wl = workload("decode")
    t = generate(wl)
    c, s, z, orc = _check_codec(t["w"], wl.G, wl.mode, label="decode")
    _check_linear(t["x"], c, s, z, None, wl.K, wl.G, wl.mode, t["bias"], orc, "decode")


@pytest.mark.timeout(900)
def test_batched_decode_full_size():
    """Every one of the 28672 rows, and all 16 x 28672 outputs."""
    wl = workload("batched_decode")
    t = generate(wl)
    c, s, z, orc = _check_codec(t["w"], wl.G, wl.mode, label="batched_decode")
    del t["w"]
    _check_linear(t["x"], c, s, z, None, wl.K, wl.G, wl.mode, None, orc, "batched_decode")


@pytest.mark.timeout(900)
def test_prefill_full_size():
    """Every weight row and all 2048 x 4096 outputs (act-order)."""
    wl = workload("prefill")
    t = generate(wl)
    c, s, z, orc = _check_codec(t["w"], wl.G, wl.mode, t["g_idx"], label="prefill")
    _check_linear(t["x"], c, s, z, t["g_idx"], wl.K, wl.G, wl.mode, None, orc, "prefill")


@pytest.mark.timeout(900)
def test_codec_full_size():
    """Every one of the 28672 odd-width bf16 rows."""
    wl = workload("codec")
    t = generate(wl)
    _check_codec(t["w"], wl.G, wl.mode, label="codec")
    # the same codes also drive an odd-K skinny linear (x bf16 [1, 8191] ~ N(0, 1))
    g = torch.Generator().manual_seed(0)
    x = torch.randn(1, wl.K, generator=g).to(torch.bfloat16)
    c, s, z, orc = _check_codec(t["w"][:2048], wl.G, wl.mode, label="codec-head")
    _check_linear(x, c, s, z, None, wl.K, wl.G, wl.mode, None, orc, "codec-linear")


# ---------------------------------------------------------------------------
# small shapes: every path, ragged tails, degenerate inputs
# ---------------------------------------------------------------------------
CASES = [
    # M, N, K, G, mode, act_order, w_dtype, bias
    (1, 1, 1, 8, "sym", False, "f32", "none"),
    (1, 33, 128, 128, "asym", False, "f32", "randn"),   # matrix-core decode: one k-block, row tail
    (3, 50, 1024, 64, "sym", False, "f32", "none"),     # matrix-core decode, transposed quarters
    (2, 40, 640, 32, "asym", False, "bf16", "randn"),
    (1, 24, 14336, 128, "sym", False, "f32", "none"),   # long K: activations staged in two batches
    (4, 16, 2048, 256, "asym", False, "f32", "randn"),
    (3, 5, 7, 8, "asym", False, "f32", "randn"),
    (1, 33, 96, 32, "sym", False, "f32", "randn"),      # decode kernel, row tail
    (2, 64, 2080, 32, "asym", False, "f32", "none"),    # decode kernel, 65 slices per row
    (4, 19, 4096, 128, "asym", False, "bf16", "randn"),
    (5, 40, 256, 64, "sym", False, "f32", "none"),      # generic skinny
    (16, 100, 512, 64, "sym", False, "f32", "randn"),   # matrix-core batched decode
    (5, 70, 640, 32, "asym", False, "f32", "randn"),     # batch tail (5 blocks of 128 columns)
    (12, 200, 1024, 256, "sym", False, "bf16", "none"),
    (16, 64, 8192, 64, "sym", False, "f32", "none"),
    # one-launch batched decode (K % 1024 == 0): 1, 3 and 5 batch pairs per
    # wave (loop, tail, both), G from 32 to 512 (a group wider than a wave's
    # quarter of K), row tails, zero-points
    (5, 70, 1024, 32, "asym", False, "f32", "randn"),
    (9, 64, 3072, 64, "asym", False, "f32", "none"),
    (16, 1000, 5120, 128, "asym", False, "bf16", "randn"),
    (6, 65, 2048, 128, "asym", False, "f32", "none"),
    (7, 300, 1024, 512, "sym", False, "f32", "randn"),
    (16, 257, 4096, 64, "sym", False, "bf16", "none"),
    (11, 129, 2048, 32, "sym", False, "f32", "randn"),
    # 4, 6, 7 and 12 batch pairs per wave: the prefetch rings' rounds of six
    # pairs and every tail length
    (16, 130, 4096, 128, "asym", False, "f32", "randn"),
    (8, 96, 6144, 64, "sym", False, "f32", "none"),
    (13, 200, 7168, 128, "asym", False, "bf16", "randn"),
    (16, 64, 12288, 128, "sym", False, "f32", "randn"),
    # the one-launch batched decode over hundreds of workgroups (more than one
    # per CU): 1, 3 and 4 batch pairs per wave, row tails
    (5, 16400, 1024, 32, "asym", False, "f32", "randn"),
    (16, 20000, 3072, 64, "sym", False, "bf16", "none"),
    (12, 17000, 4096, 128, "sym", False, "f32", "randn"),
    (1, 37, 2048, 64, "asym", False, "f32", "randn"),   # staged decode, row tail
    (1, 50, 4096, 256, "sym", False, "bf16", "none"),   # staged decode, signed
    (1, 24, 16384, 256, "asym", False, "f32", "randn"), # staged decode, longest row, 64 groups
    (1, 8, 640, 32, "sym", False, "f32", "randn"),      # staged decode, partial round
    # streaming decode GEMV (M = 1, K = 4096): 2, 4, 8 and 14 rows per wave
    # pair, a last workgroup with one row set past N, row tails
    (1, 4097, 4096, 32, "asym", False, "f32", "randn"),
    (1, 14339, 4096, 64, "sym", False, "f32", "none"),
    (1, 20001, 4096, 128, "asym", False, "bf16", "randn"),
    (1, 64, 512, 128, "asym", True, "f32", "none"),     # act-order decode
    # act-order decode with LDS value tables (M <= 4; K = 2048, 4096, 8192):
    # 2, 4, 7 and 8 rows per set, one and two waves per set, row tails
    (1, 300, 4096, 128, "asym", True, "f32", "randn"),
    (2, 37, 2048, 64, "sym", True, "bf16", "none"),
    (4, 14339, 4096, 128, "asym", True, "f32", "randn"),
    (3, 5000, 8192, 64, "sym", True, "f32", "none"),
    (1, 20000, 2048, 32, "asym", True, "bf16", "randn"),
    (16, 48, 1000, 40, "asym", True, "bf16", "none"),
    # act-order decode on the matrix cores (M = 1, at most 32 groups, K % 1024
    # == 0): one and two 16-group halves, 1, 4 and 8 batch pairs per wave,
    # row tails, a group size that is not a power of two
    (1, 4097, 4096, 256, "sym", True, "bf16", "none"),
    (1, 130, 2048, 64, "asym", True, "f32", "randn"),
    (1, 1000, 8192, 256, "asym", True, "f32", "none"),
    (1, 33, 3072, 96, "sym", True, "f32", "randn"),
    (1, 14336, 4096, 128, "asym", True, "bf16", "randn"),
    (17, 130, 200, 8, "asym", False, "f32", "randn"),   # prefill, K % 64 != 0, N tail
    (40, 70, 99, 16, "sym", False, "f32", "none"),      # prefill, K % 8 != 0
    (300, 260, 1024, 128, "asym", True, "f32", "randn"),
    (129, 128, 4096, 4096, "sym", False, "bf16", "none"),  # one group per row
    # prefill through the fragment-tiled weight (K % 64 == 0): one and two
    # K-steps, a step count that is not a multiple of 3, M and N tails
    (33, 40, 64, 16, "sym", False, "f32", "randn"),
    (18, 256, 128, 128, "asym", False, "f32", "none"),
    (257, 300, 640, 32, "asym", True, "f32", "none"),
    (65, 33, 128, 64, "sym", False, "bf16", "randn"),
    # prefill with contiguous groups and K % 64 == 0 (dequantize + pipelined
    # GEMM): 1, 2, 3, 4 and 17 K-steps, M and N tile tails, G from 32 to 256,
    # a partial last group, one group per row
    (17, 300, 64, 64, "sym", False, "bf16", "none"),
    (40, 512, 128, 32, "asym", False, "f32", "none"),
    (200, 96, 192, 64, "sym", False, "f32", "randn"),
    (130, 257, 256, 32, "asym", False, "f32", "randn"),
    (33, 64, 1088, 256, "sym", False, "f32", "none"),
    (64, 256, 2048, 128, "asym", False, "bf16", "randn"),
    (300, 520, 512, 128, "sym", False, "f32", "randn"),
    (1300, 500, 256, 128, "asym", False, "f32", "randn"),  # 6 x 4 GEMM tiles: per-XCD runs, last row group partial
    (96, 80, 1024, -1, "sym", False, "f32", "none"),
    # prefill with the fragment-tiled weight (N % 128 == 0, K % 64 == 0):
    # act-order, G = 32 with 128 groups, G = 512, per-channel, M tails
    (257, 384, 640, 64, "asym", True, "f32", "randn"),
    (129, 256, 4096, 32, "sym", False, "bf16", "none"),
    (65, 128, 1024, 512, "asym", False, "f32", "randn"),
    (33, 128, 1024, -1, "sym", False, "f32", "none"),
    # per-channel (G = -1, or any G >= K): one scale per row
    (1, 40, 100, -1, "sym", False, "f32", "randn"),
    (4, 33, 4096, -1, "sym", False, "bf16", "none"),     # matrix-core decode
    (1, 24, 14336, -1, "asym", False, "f32", "randn"),   # decode kernel, one group over 14336 columns
    (16, 64, 8192, -1, "asym", False, "f32", "none"),    # matrix-core batched decode
    (20, 64, 8191, -1, "sym", False, "bf16", "none"),    # prefill, odd K
    (3, 10, 5000, 6000, "sym", False, "f32", "randn"),   # G > K, not a multiple of 8
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "M%d_N%d_K%d_G%d_%s%s" % (c[0], c[1], c[2], c[3], c[4], "_act" if c[5] else ""))
def test_small_shapes(case):
    M, N, K, G, mode, act, wdt, bias = case
    wl = workload("tiny", M=M, N=N, K=K, G=G, mode=mode, act_order=act, w_dtype=wdt, bias=bias,
                  bias_std=0.01, seed=K + N)
    if act and K % G:
        pytest.skip("act-order workloads use whole groups")
    t = generate(wl)
    c, s, z, orc = _check_codec(t["w"], G, mode, t["g_idx"], label=str(case))
    _check_linear(t["x"], c, s, z, t["g_idx"], K, G, mode, t["bias"], orc, str(case))


def test_codec_alignment_classes_and_long_rows():
    g = torch.Generator().manual_seed(7)
    for (N, K, G, dt) in [(37, 8191, 32, torch.bfloat16), (11, 8191, 32, torch.float32),
                          (9, 20000, 64, torch.float32), (9, 20001, 64, torch.bfloat16),
                          (8, 3, 8, torch.bfloat16)]:
        w = (torch.randn(N, K, generator=g) * 0.02).to(dt)
        for mode in ("sym", "asym"):
            _check_codec(w, G, mode, label=f"{N}x{K} G{G} {dt} {mode}")


CODEC_SHAPES = [
    # N, K, G, weight dtype: row-register quantizer (power-of-two G <= 512,
    # K <= 16384) and flat dequantizer (K >= 2048) around their edges
    (5, 2048, 8, torch.float32), (7, 2049, 32, torch.bfloat16), (3, 2050, 512, torch.float32),
    (6, 4100, 128, torch.bfloat16), (4, 3000, 256, torch.float32), (3, 16384, 512, torch.bfloat16),
    (2, 16383, 8, torch.float32), (3, 16385, 64, torch.bfloat16), (9, 2047, 16, torch.bfloat16),
    (13, 2111, 64, torch.float32), (3, 6000, 48, torch.bfloat16),
    # groups of 32 (a lane per group, runs of 64 groups): one partial group, a partial
    # third run with rows at 4-byte offsets, fp32 rows past two runs
    (5, 21, 32, torch.float32), (6, 4190, 32, torch.bfloat16), (3, 6145, 32, torch.float32),
]


@pytest.mark.parametrize("shape", CODEC_SHAPES, ids=lambda c: "N%d_K%d_G%d_%s" % (c[0], c[1], c[2], str(c[3])[6:]))
def test_codec_fast_paths(shape):
    N, K, G, dt = shape
    g = torch.Generator().manual_seed(K + G)
    w = (torch.randn(N, K, generator=g) * 0.05).to(dt)
    for mode in ("sym", "asym"):
        _check_codec(w, G, mode, label=f"{N}x{K} G{G} {dt} {mode}")


def test_codec_near_rounding_ties():
    """Weights at and a few ulps either side of (q + 1/2) times the scale,
    where the last bit of the quotient decides the code.  Scales have short
    significands so that each group's range pins them exactly."""
    N, K, G = 6, 4096, 32
    NG = K // G
    rng = np.random.default_rng(11)
    s = (rng.integers(2 ** 12, 2 ** 16, size=(N, NG)) * 2.0 ** rng.integers(-40, 0, size=(N, NG))).astype(np.float32)
    sk = np.repeat(s, G, axis=1).astype(np.float64)
    for mode, lo, hi in (("sym", -7, 6), ("asym", -8, 6)):
        q = rng.integers(lo, hi + 1, size=(N, K)).astype(np.float64) + 0.5
        w = (q * sk).astype(np.float32)
        step = rng.integers(-2, 3, size=(N, K)).astype(np.int32)
        w = (w.view(np.int32) + step).view(np.float32)
        w[:, ::G] = 7.0 * s                      # max: 7 s
        w[:, 1::G] = -7.0 * s if mode == "sym" else -8.0 * s
        for dt in (torch.float32, torch.bfloat16):
            _check_codec(torch.from_numpy(w).to(dt), G, mode, label=f"ties {mode} {dt}")


def test_dequantize_act_order_large_group_table():
    """More groups per row than the staged act-order table holds (G = 8,
    8200 groups): the dequantizer gathers scales from global memory."""
    N, K, G = 3, 65600, 8
    rng = np.random.default_rng(12)
    gnp = (rng.permutation(K) // G).astype(np.int32)
    w = rng.standard_normal((N, K)).astype(np.float32) * 0.02
    for mode in (O.SYM, O.ASYM):
        # w4_quantize_pack takes at most 4096 groups per row; these codes come from the oracle
        oc, osc, oz = O.quantize_pack(w, G, mode, gnp)
        zeros = None if oz is None else torch.from_numpy(oz).to(DEV)
        for dt, kind in ((torch.bfloat16, "bf16"), (torch.float32, "f32")):
            d = w4.dequantize(torch.from_numpy(oc).to(DEV), torch.from_numpy(osc).to(DEV), zeros,
                              torch.from_numpy(gnp).to(DEV), K, G, mode, dt).cpu()
            ref = O.dequantize(oc, osc, oz, gnp, K, G, mode, kind)
            got = _bits(d) if kind == "bf16" else d.numpy().view(np.uint32)
            assert np.array_equal(got, ref if kind == "bf16" else ref.view(np.uint32)), f"{mode} {kind}"


def test_codec_degenerate_values():
    """All-zero groups, one-signed groups, exact ties, tiny (subnormal-scale)
    and large magnitudes."""
    N, K, G = 8, 64, 16
    w = torch.zeros(N, K)
    w[1] = torch.linspace(0.01, 1.0, K)                       # all positive
    w[2] = -torch.linspace(0.01, 1.0, K)                      # all negative
    w[3, :G] = torch.tensor([7.0, -2.5, 1.5, 0.25, 3.5, -0.5, 0.5, 5.5] * 2)   # s = 1: ties
    w[4] = torch.randn(K, generator=torch.Generator().manual_seed(1)) * 1e-39  # subnormal range
    w[5] = torch.randn(K, generator=torch.Generator().manual_seed(2)) * 1e30
    w[6, ::7] = 1.0                                           # sparse
    w[7] = -0.0
    wide = w.repeat(1, 2048 // K)                             # the same rows at K = 2048
    for gs in (G, 32):                                        # 32: the lane-per-group quantizer
        for mode in ("sym", "asym"):
            for x, lab in ((w, ""), (wide, " wide")):
                _check_codec(x, gs, mode, label=f"degenerate{lab} G{gs} {mode}")
                _check_codec(x.to(torch.bfloat16), gs, mode, label=f"degenerate{lab} G{gs} bf16 {mode}")


def _subnormal_scale_rows(K, G):
    """fp32 rows whose groups have max|w| = 10 * 2^-149 or 17 * 2^-149: the
    signed scale amax / 7 is then a subnormal rounded far from the quotient
    (17 * 2^-149 gives s = 2 * 2^-149 and w / s = 8.5), so only the clamp to
    [-7, 7] keeps the codes in range."""
    u = 2.0 ** -149
    pattern = torch.tensor([17.0, -17.0, 10.0, -10.0, 5.0, 3.0, -1.0, 0.0, 8.0, -9.0, 16.0, 2.0], dtype=torch.float64)
    rows = []
    for amax in (10.0, 17.0):
        r = pattern.clamp(-amax, amax).repeat(-(-K // len(pattern)))[:K].clone()
        r[::G] = amax                                        # every group reaches amax
        rows += [r, -r, r.roll(5)]
    return (torch.stack(rows) * u).to(torch.float32)


def test_codec_subnormal_scale_clamp():
    """Regression: signed codes stay in [-7, 7] when the group scale is a
    subnormal (the fast row quantizer, the general one, and act-order)."""
    for K, G in ((64, 32), (2048, 32), (4096, 128), (72, 8)):
        w = _subnormal_scale_rows(K, G)
        assert w.abs().max().item() > 0 and w.abs().max().item() < 1e-43
        _check_codec(w, G, "sym", label=f"subnormal K={K} G={G}")
        _check_codec(w, G, "asym", label=f"subnormal asym K={K} G={G}")
    w = _subnormal_scale_rows(1024, 64)
    g_idx = (torch.randperm(1024, generator=torch.Generator().manual_seed(9)) // 64).to(torch.int32)
    _check_codec(w, 64, "sym", g_idx=g_idx, label="subnormal act-order")


def test_lora_requantize_subnormal_scale_clamp():
    """Regression: the LoRA merge's requantizer clamps signed codes when the
    merged weight's group scale is subnormal.  Zero codes plus an update
    c * A B with c = 2^-140 and A holding multiples of 2^-9 give merged weights
    that are exact multiples of 2^-149 with max|w| of 10 or 17 units."""
    N, K, G = 6, 512, 32
    units = (_subnormal_scale_rows(K, G)[3].double() / 2.0 ** -149).round()   # integers, max |.| = 17
    A = (units * 2.0 ** -9).to(torch.float32).reshape(K, 1).numpy()
    B = np.ones((1, N), np.float32)
    B[0, 1::2] = -1.0
    oc = np.zeros((N, K // 2), np.uint8)
    osc = np.ones((N, K // G), np.float32)
    c, s = torch.from_numpy(oc).to(DEV), torch.from_numpy(osc).to(DEV)
    scale = 2.0 ** -140
    c2, s2, _ = w4.lora_merge(c, s, None, None, K, G, "sym", torch.from_numpy(A).to(DEV), torch.from_numpy(B).to(DEV), scale)
    torch.cuda.synchronize()
    merged = O.lora_merged_weight(oc, osc, None, None, K, G, O.SYM, A, B, scale)
    assert np.abs(merged).max() == 17 * 2.0 ** -149
    ec, es, _ = O.lora_merge(oc, osc, None, None, K, G, O.SYM, A, B, scale)
    assert np.array_equal(c2.cpu().numpy(), ec), "merged codes differ (subnormal scales)"
    assert np.array_equal(s2.cpu().numpy().view(np.uint32), es.view(np.uint32)), "merged scales differ (subnormal scales)"


@pytest.mark.parametrize("N,K,G,dt,uniform", [(13, 4096, 128, torch.float32, True), (9, 8192, 512, torch.bfloat16, True),
                                               (20, 512, 8, torch.bfloat16, True), (17, 1024, 64, torch.float32, False),
                                               (11, 2048, 256, torch.bfloat16, False)])
def test_act_order_codec(N, K, G, dt, uniform):
    """Act-order quantize: uniform groups (every group G columns: the
    group-sorted row kernel) and uneven random groups (its per-row fallback)."""
    g = torch.Generator().manual_seed(N + K + G)
    w = (torch.randn(N, K, generator=g) * 0.05).to(dt)
    if uniform:
        g_idx = (torch.randperm(K, generator=g) // G).to(torch.int32)
    else:
        g_idx = torch.randint(0, K // G, (K,), generator=g).to(torch.int32)
    for mode in ("sym", "asym"):
        _check_codec(w, G, mode, g_idx, label=f"act {N}x{K} G{G} {dt} {mode} uniform={uniform}")


def test_act_order_with_unused_groups():
    """A g_idx that leaves some groups empty: those keep scale 1 (zero-point 0)."""
    N, K, G = 6, 64, 16
    w = torch.randn(N, K, generator=torch.Generator().manual_seed(3)) * 0.02
    g_idx = torch.tensor([0, 3] * (K // 2), dtype=torch.int32)
    for mode in ("sym", "asym"):
        _check_codec(w, G, mode, g_idx, label=f"unused groups {mode}")


@pytest.mark.parametrize("G", [-1, 128])
def test_act_order_one_group_per_row(G):
    """A g_idx putting every column in group 0 with one group per row
    (per-channel, or G >= K): the codec, then the linear through the decode,
    batched and prefill paths."""
    N, K = 40, 100
    g = torch.Generator().manual_seed(11)
    w = torch.randn(N, K, generator=g) * 0.02
    g_idx = torch.zeros(K, dtype=torch.int32)
    for mode in ("sym", "asym"):
        c, s, z, orc = _check_codec(w, G, mode, g_idx, label=f"one group G{G} {mode}")
        for M in (1, 8, 40):
            x = torch.randn(M, K, generator=g).to(torch.bfloat16)
            _check_linear(x, c, s, z, g_idx, K, G, mode, None, orc, f"one group G{G} {mode} M{M}")


def test_act_order_uneven_groups_linear():
    """A g_idx leaving some groups empty and others double size, through the
    linear at decode, batched and prefill sizes."""
    N, K, G = 24, 64, 16
    g = torch.Generator().manual_seed(12)
    w = torch.randn(N, K, generator=g) * 0.02
    g_idx = torch.tensor([0, 3] * (K // 2), dtype=torch.int32)
    for mode in ("sym", "asym"):
        c, s, z, orc = _check_codec(w, G, mode, g_idx, label=f"uneven {mode}")
        for M in (1, 8, 40):
            x = torch.randn(M, K, generator=g).to(torch.bfloat16)
            _check_linear(x, c, s, z, g_idx, K, G, mode, None, orc, f"uneven {mode} M{M}")


@pytest.mark.parametrize("M,K,G,mode", [(16, 256, 32, "asym"), (4, 512, 128, "sym"), (1, 96, 32, "asym"),
                                        (7, 100, 8, "sym"), (256, 256, 64, "asym"), (96, 96, 32, "sym"),
                                        (130, 1024, 256, "asym"), (200, 512, 32, "sym"), (48, 640, -1, "sym")])
def test_identity_activation_is_exact(M, K, G, mode):
    """x = rows of the identity: every output is a single product, so
    y[i, n] must equal the bf16 dequantized weight Wd[n, k_i] bit for bit."""
    N = 72
    w = torch.randn(N, K, generator=torch.Generator().manual_seed(M + K)) * 0.02
    cols = np.sort(np.random.default_rng(M).choice(K, size=min(M, K), replace=False))
    x = torch.zeros(len(cols), K)
    x[torch.arange(len(cols)), torch.from_numpy(cols)] = 1.0
    codes, scales, zeros = w4.quantize_pack(w.to(DEV), G, mode)
    y = w4.linear(x.to(torch.bfloat16).to(DEV), codes, scales, zeros, None, K, G, mode)
    wd = w4.dequantize(codes, scales, zeros, None, K, G, mode, torch.bfloat16)
    torch.cuda.synchronize()
    oc, osc, oz = O.quantize_pack(w.numpy(), G, _mode(mode))
    ref = O.dequantize(oc, osc, oz, None, K, G, _mode(mode), "bf16")[:, cols].T
    assert np.array_equal(_bits(y.cpu()), ref)
    assert np.array_equal(_bits(wd.cpu())[:, cols].T, ref)


@pytest.mark.parametrize("M,K,G,mode,act", [(130, 1024, 128, "asym", True), (256, 640, 64, "sym", False),
                                            (40, 4096, 32, "asym", False), (300, 2048, 128, "sym", True)])
def test_identity_activation_is_exact_tiled_prefill(M, K, G, mode, act):
    """The prefill path with the fragment-tiled weight (N % 128 == 0,
    K % 64 == 0): unit activation rows return the bf16 dequantized weight bit
    for bit, which pins the tiled layout, the K order inside a K-step and the
    act-order table lookups."""
    N = 256
    gen = torch.Generator().manual_seed(M + K + G)
    w = torch.randn(N, K, generator=gen) * 0.02
    g_idx = (torch.randperm(K, generator=gen) // G).to(torch.int32) if act else None
    cols = np.sort(np.random.default_rng(M + 1).choice(K, size=min(M, K), replace=False))
    x = torch.zeros(len(cols), K)
    x[torch.arange(len(cols)), torch.from_numpy(cols)] = 1.0
    gi = None if g_idx is None else g_idx.to(DEV)
    codes, scales, zeros = w4.quantize_pack(w.to(DEV), G, mode, gi)
    y = w4.linear(x.to(torch.bfloat16).to(DEV), codes, scales, zeros, gi, K, G, mode)
    torch.cuda.synchronize()
    gnp = None if g_idx is None else g_idx.numpy()
    oc, osc, oz = O.quantize_pack(w.numpy(), G, _mode(mode), gnp)
    ref = O.dequantize(oc, osc, oz, gnp, K, G, _mode(mode), "bf16")[:, cols].T
    assert np.array_equal(_bits(y.cpu()), ref)


def test_empty_batch_and_errors():
    wl = workload("tiny", N=16, K=64)
    t = generate(wl)
    codes, scales, zeros = w4.quantize_pack(t["w"].to(DEV), 32, "sym")
    y = w4.linear(torch.empty(0, 64, dtype=torch.bfloat16, device=DEV), codes, scales, zeros, None, 64, 32, "sym")
    assert y.shape == (0, 16)
    with pytest.raises(w4.W4Error):
        w4.quantize_pack(t["w"].to(DEV), 12, "sym")
    with pytest.raises(ValueError):
        w4.linear(torch.zeros(2, 64, dtype=torch.bfloat16, device=DEV), codes, scales, None, None, 64, 32, "asym")


# ---------------------------------------------------------------------------
# input gradient dx = dy . Wd
# ---------------------------------------------------------------------------
def _check_grad(M, N, K, G, mode, act, seed, cols=None, label=""):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    gnp = (rng.permutation(K) // G % O.n_groups(K, G)).astype(np.int32) if act else None
    oc, osc, oz = O.quantize_pack(w, G, _mode(mode), gnp)
    dy = torch.from_numpy(rng.standard_normal((M, N)).astype(np.float32)).to(torch.bfloat16)
    gi = None if gnp is None else torch.from_numpy(gnp).to(DEV)
    z = None if oz is None else torch.from_numpy(oz).to(DEV)
    c, s = torch.from_numpy(oc).to(DEV), torch.from_numpy(osc).to(DEV)
    dx = w4.linear_grad_input(dy.to(DEV), c, s, z, gi, K, G, mode)
    dx2 = w4.linear_grad_input(dy.to(DEV), c, s, z, gi, K, G, mode)
    torch.cuda.synchronize()
    assert torch.equal(dx.view(torch.int16), dx2.view(torch.int16)), f"grad not deterministic {label}"
    sel = np.arange(K) if cols is None else cols
    wd = O.bf16_bits_to_f32(O.dequantize(oc, osc, oz, gnp, K, G, _mode(mode), "bf16"))[:, sel]
    ref = O.bf16_bits_to_f32(_bits(dy)).astype(np.float64) @ wd.astype(np.float64)
    got = dx[:, torch.from_numpy(sel).to(DEV)].float().cpu().numpy().astype(np.float64)
    err = got - ref
    rel = np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-30)
    assert rel <= NORM_TOL, f"grad normwise {rel:.3e} {label}"
    assert np.abs(err).max() <= ELEM_TOL * max(np.abs(ref).max(), 1e-30), f"grad max err {label}"


GRAD_CASES = [
    # M, N, K, G, mode, act-order: M <= 16 (row slices) and M > 16 (transposed weight + GEMM)
    (1, 64, 512, 128, "asym", False), (4, 33, 1000, 40, "sym", True), (16, 100, 96, 32, "asym", False),
    (3, 50, 99, 8, "sym", False), (2, 7, 8200, 64, "asym", False), (9, 300, 2048, 256, "sym", True),
    (48, 64, 256, 64, "asym", False), (300, 130, 200, 8, "sym", True), (40, 96, 512, 128, "asym", False),
    (17, 1, 64, 16, "sym", False), (20, 24, 2048, 8, "asym", True),   # 256 groups: tables read from memory
    (1, 64, 4100, -1, "asym", False), (2, 50, 4096, -1, "sym", False), (20, 40, 300, -1, "sym", False),
    # transposed weight in the GEMM's tiled layout (N % 64 == 0, K % 128 == 0), through value
    # tables (at most 32 groups per row): one 64-row block, full tables, contiguous and act-order,
    # 9 sub-tiles of 128 columns split over workgroups in runs of 2 (the last run short),
    # one sub-tile of one row block, per-channel (one group)
    (33, 128, 384, 64, "sym", True), (130, 192, 1024, 128, "asym", False),
    (64, 64, 256, 32, "asym", True), (20, 128, 4096, 128, "asym", True), (33, 192, 2048, 64, "asym", False),
    (17, 4096, 1152, 128, "sym", False), (17, 64, 128, 64, "sym", False), (24, 64, 1024, -1, "asym", False),
    # more than 32 groups per row: the tiled layout without value tables
    (24, 64, 4096, 64, "asym", True),
    # one dy row, 32 columns per lane (8-wave slices): 32 slices, the last of 8 rows (one per
    # wave); 3 slices of 25-26 rows (waves of 3 or 4 rows); K % 2048 != 0 (a lane with 24 columns,
    # lanes past K)
    (1, 1000, 2048, 64, "sym", False), (1, 77, 4096, 32, "asym", False), (1, 300, 3000, 64, "asym", False),
]


@pytest.mark.parametrize("case", GRAD_CASES, ids=lambda c: "M%d_N%d_K%d_G%d_%s%s" % (c[0], c[1], c[2], c[3], c[4], "_act" if c[5] else ""))
def test_grad_input_small(case):
    M, N, K, G, mode, act = case
    _check_grad(M, N, K, G, mode, act, seed=M + N + K, label=str(case))


def test_grad_input_decode_size():
    """The decode layer's shape: the reduction runs over all 14336 rows."""
    _check_grad(1, 14336, 4096, 128, "asym", False, seed=30, label="decode-size")


@pytest.mark.timeout(900)
def test_grad_input_prefill_size():
    _check_grad(2048, 4096, 4096, 128, "asym", True, seed=31, cols=None, label="prefill-size")


@pytest.mark.parametrize("M,K,mode,N", [(3, 520, "sym", 40), (24, 256, "asym", 40),
                                        (40, 512, "asym", 128), (64, 256, "sym", 64), (48, 256, "asym", 128)])
def test_grad_input_unit_rows_are_exact(M, K, mode, N):
    """dy row m = e_{n_m}: dx row m is the bf16 dequantized row n_m, bit for bit
    (the last three shapes take the tiled transposed weight, the last two through
    value tables)."""
    G = 8
    rng = np.random.default_rng(32)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    oc, osc, oz = O.quantize_pack(w, G, _mode(mode))
    rows = rng.integers(0, N, size=M)
    dy = torch.zeros(M, N)
    dy[torch.arange(M), torch.from_numpy(rows)] = 1.0
    z = None if oz is None else torch.from_numpy(oz).to(DEV)
    dx = w4.linear_grad_input(dy.to(torch.bfloat16).to(DEV), torch.from_numpy(oc).to(DEV),
                              torch.from_numpy(osc).to(DEV), z, None, K, G, mode)
    wd = O.dequantize(oc, osc, oz, None, K, G, _mode(mode), "bf16")
    assert np.array_equal(_bits(dx.cpu()), wd[rows])


def test_grad_input_empty_and_errors():
    N, K, G = 16, 64, 16
    codes = torch.zeros(N, K // 2, dtype=torch.uint8, device=DEV)
    scales = torch.ones(N, K // G, device=DEV)
    dy = torch.zeros(0, N, dtype=torch.bfloat16, device=DEV)
    assert w4.linear_grad_input(dy, codes, scales, None, None, K, G, "sym").shape == (0, K)
    lib = w4.load()
    dy = torch.zeros(2, N, dtype=torch.bfloat16, device=DEV)
    dx = torch.empty(2, K, dtype=torch.bfloat16, device=DEV)
    need = w4.linear_grad_input_workspace_bytes(2, N, K, G, "sym")
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    st = lib.w4_linear_grad_input(dy.data_ptr(), 2, codes.data_ptr(), scales.data_ptr(), None, None,
                                  N, K, G, 0, dx.data_ptr(), ws.data_ptr(), need - 1, None)
    assert st == 1 and b"workspace" in lib.w4_last_error()
    st = lib.w4_linear_grad_input(dy.data_ptr() + 2, 2, codes.data_ptr(), scales.data_ptr(), None, None,
                                  N, K, G, 0, dx.data_ptr(), ws.data_ptr(), need, None)
    assert st == 1 and b"aligned" in lib.w4_last_error()


# ---------------------------------------------------------------------------
# LoRA merge: codes, scales and zero-points bit-exact against the oracle
# ---------------------------------------------------------------------------
def _lora_inputs(N, K, G, mode, act, r, seed):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    gnp = (rng.permutation(K) // G % O.n_groups(K, G)).astype(np.int32) if act else None
    oc, osc, oz = O.quantize_pack(w, G, _mode(mode), gnp)
    A = (rng.standard_normal((K, r)) * 0.05).astype(np.float32)
    B = (rng.standard_normal((r, N)) * 0.05).astype(np.float32)
    return oc, osc, oz, gnp, A, B


def _check_lora(N, K, G, mode, act, r, scale, seed, rows=None, in_place=False, label=""):
    oc, osc, oz, gnp, A, B = _lora_inputs(N, K, G, mode, act, r, seed)
    c, s = torch.from_numpy(oc).to(DEV), torch.from_numpy(osc).to(DEV)
    z = None if oz is None else torch.from_numpy(oz).to(DEV)
    gi = None if gnp is None else torch.from_numpy(gnp).to(DEV)
    a, b = torch.from_numpy(A).to(DEV), torch.from_numpy(B).to(DEV)
    out = (c, s, z) if in_place else None
    c2, s2, z2 = w4.lora_merge(c, s, z, gi, K, G, mode, a, b, scale, out=out)
    torch.cuda.synchronize()
    sel = np.arange(N) if rows is None else rows
    zsel = None if oz is None else oz[sel]
    ec, es, ez = O.lora_merge(oc[sel], osc[sel], zsel, gnp, K, G, _mode(mode), A, B[:, sel], scale)
    tsel = torch.from_numpy(sel).to(DEV)
    assert np.array_equal(c2[tsel].cpu().numpy(), ec), f"merged codes differ {label}"
    assert np.array_equal(s2[tsel].cpu().numpy().view(np.uint32), es.view(np.uint32)), f"merged scales differ {label}"
    if ez is not None:
        assert np.array_equal(z2[tsel].cpu().numpy(), ez), f"merged zeros differ {label}"
    # the update moved codes (the inputs are sized for it unless scale = 0)
    if scale != 0:
        assert np.mean(ec != oc[sel]) > 0.05, f"update too small to test {label}"


LORA_CASES = [
    # N, K, G, mode, act-order, rank, alpha / rank: one pass (contiguous power-of-two groups <= 512)
    (64, 512, 64, "sym", False, 8, 2.0),
    (37, 1000, 8, "asym", False, 5, 0.5),        # partial column block, rank % 4 != 0
    (33, 777, 32, "sym", False, 3, 1.0),         # odd K: code rows not word aligned
    (20, 1536, 512, "asym", False, 64, 0.25),    # largest group, largest rank
    (10, 64, 16, "asym", False, 1, 4.0),
    (300, 2048, 128, "asym", False, 16, 2.0),    # several row blocks
    # merged fp32 weight + quantizer
    (50, 640, 64, "asym", True, 8, 2.0),         # act-order
    (40, 640, 40, "sym", False, 4, 1.0),         # group size not a power of two
    (24, 4100, -1, "asym", False, 16, 2.0),      # per-channel
    (30, 2048, 1024, "sym", False, 12, 1.0),     # group wider than the column block
]


@pytest.mark.parametrize("case", LORA_CASES, ids=lambda c: "N%d_K%d_G%d_%s%s_r%d" % (c[0], c[1], c[2], c[3], "_act" if c[4] else "", c[5]))
def test_lora_merge_small(case):
    N, K, G, mode, act, r, scale = case
    _check_lora(N, K, G, mode, act, r, scale, seed=N + K + r, label=str(case))


@pytest.mark.parametrize("G,act", [(64, False), (64, True)])
def test_lora_merge_in_place(G, act):
    _check_lora(70, 1024, G, "asym", act, 8, 2.0, seed=5, in_place=True, label="in place")


def test_lora_merge_zero_update():
    _check_lora(40, 512, 32, "sym", False, 4, 0.0, seed=6, label="zero update")


@pytest.mark.timeout(900)
def test_lora_merge_decode_layer():
    """The decode layer's weight (14336 x 4096, G = 128, zero-points), rank 16,
    every row."""
    _check_lora(14336, 4096, 128, "asym", False, 16, 2.0, seed=7, rows=None, label="decode-size")


# ---------------------------------------------------------------------------
# storage formats: GGUF Q4_0 blocks and packed zero-points, bit-exact
# ---------------------------------------------------------------------------
def _q4_weights(N, K, seed):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    nb = K // 32
    if N * nb >= 4:                      # a zero block, a subnormal-scale block, a tie of the stored scale
        w[0, 0:32] = 0
        w.reshape(-1, 32)[1] = 0
        w.reshape(-1, 32)[1][0] = 10 * 2.0 ** -24
        w.reshape(-1, 32)[2][0] = 1.0
        w.reshape(-1, 32)[2][1] = 3.5 * (1170 / 1024 / 8)
    return w


@pytest.mark.parametrize("N,K,wdt", [(1, 32, "f32"), (3, 64, "bf16"), (37, 96, "bf16"), (100, 4096, "f32"),
                                     (65, 32, "f32"), (7, 8192, "bf16")])
def test_q4_0_codec(N, K, wdt):
    w = torch.from_numpy(_q4_weights(N, K, seed=N + K))
    if wdt == "bf16":
        w = w.to(torch.bfloat16)
    blocks = w4.q4_0_quantize(w.to(DEV))
    torch.cuda.synchronize()
    ref = O.q4_0_quantize(_np_w(w))
    assert np.array_equal(blocks.cpu().numpy(), ref), f"Q4_0 blocks differ N{N} K{K} {wdt}"
    for dt, kind in ((torch.bfloat16, "bf16"), (torch.float32, "f32")):
        got = w4.q4_0_dequantize(blocks, dt).cpu()
        exp = O.q4_0_dequantize(ref, kind)
        if kind == "bf16":
            assert np.array_equal(_bits(got), exp), f"Q4_0 bf16 decode differs N{N} K{K}"
        else:
            assert np.array_equal(got.numpy().view(np.uint32), exp.view(np.uint32)), f"Q4_0 f32 decode differs N{N} K{K}"


def test_q4_0_decodes_arbitrary_blocks():
    """Every nibble pattern and finite fp16 scales, including subnormal ones."""
    rng = np.random.default_rng(50)
    N, nb = 40, 70
    blk = rng.integers(0, 256, size=(N, nb, 18), dtype=np.uint8)
    d = rng.standard_normal((N, nb)).astype(np.float16) * np.float16(0.01)
    d[0, :8] = np.float16(2.0 ** -24) * np.arange(1, 9, dtype=np.float16)
    blk[..., 0:2] = d.astype("<f2").view(np.uint8).reshape(N, nb, 2)
    got = w4.q4_0_dequantize(torch.from_numpy(blk).to(DEV), torch.float32).cpu().numpy()
    assert np.array_equal(got.view(np.uint32), O.q4_0_dequantize(blk, "f32").view(np.uint32))


@pytest.mark.timeout(900)
def test_q4_0_full_size():
    """The codec weight's shape at K = 8192 (bf16 [28672, 8192]), every block."""
    wl = workload("codec", K=8192)
    t = generate(wl)
    w = t["w"]
    blocks = w4.q4_0_quantize(w.to(DEV))
    torch.cuda.synchronize()
    ref = O.q4_0_quantize(_np_w(w))
    assert np.array_equal(blocks.cpu().numpy(), ref)


@pytest.mark.parametrize("N,NG", [(1, 1), (5, 7), (300, 32), (1000, 257), (3, 6), (7, 22), (28672, 256)])
def test_packed_zeros_round_trip(N, NG):
    rng = np.random.default_rng(N + NG)
    z = rng.integers(0, 16, size=(N, NG), dtype=np.uint8)
    p = w4.pack_zeros(torch.from_numpy(z).to(DEV))
    assert np.array_equal(p.cpu().numpy(), O.pack_zeros(z))
    u = w4.unpack_zeros(p, NG)
    assert np.array_equal(u.cpu().numpy(), z)
