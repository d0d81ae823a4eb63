"""Pins for the CPU oracle: checks against what the pages and the mathematics
fix, never against the oracle's own formulas retyped.

  * hand-worked examples (tests/golden/hand_worked.json, each with its source);
  * library routines: torch's fp32 -> bf16 conversion, numpy's int8 sign
    extension, a pure-Python brute-force matmul;
  * invariants: code ranges, positive finite scales, the half-step error
    bound, a code of magnitude 7 in every non-zero symmetric group, the zero
    high nibble for odd K, pack/unpack round trip;
  * special cases: G = K against the Gemma per-channel formula (scale as an
    inverse, multiply instead of divide); g_idx = k // G against no g_idx; a
    column permutation against g_idx;
  * the identity activation, whose linear output is the dequantized weight.
"""
import numpy as np
import pytest
import torch

from oracle import w4_oracle as O
from int4_group_wise_amd.workloads import workload, generate, bf16_bits

F32 = np.float32


def _arr(v, dt):
    return None if v is None else np.array(v, dtype=dt)


# --------------------------------------------------------------------------
# hand-worked examples
# --------------------------------------------------------------------------
def test_golden_quantize_pack_dequant(golden):
    for c in golden["cases"]:
        w = np.array(c["w"], F32)
        g_idx = _arr(c["g_idx"], np.int32)
        q, s, z = O.quantize(w, c["G"], c["mode"], g_idx)
        assert q.tolist() == c["q"], c["name"]
        assert s.tolist() == c["scales"], c["name"]
        if c["zeros"] is None:
            assert z is None
        else:
            assert z.tolist() == c["zeros"], c["name"]
        codes, s2, z2 = O.quantize_pack(w, c["G"], c["mode"], g_idx)
        assert codes.tolist() == c["codes"], c["name"]
        d = O.dequantize(codes, s2, z2, g_idx, c["K"], c["G"], c["mode"], "f32")
        assert d.tolist() == c["dequant"], c["name"]
        if "dequant_bf16_bits" in c:
            db = O.dequantize(codes, s2, z2, g_idx, c["K"], c["G"], c["mode"], "bf16")
            assert db.tolist() == c["dequant_bf16_bits"], c["name"]
        O.validate_packed(codes, s2, z2, c["K"], c["G"], c["mode"], g_idx)


def test_golden_decode(golden):
    d = golden["decode"]
    u = O.unpack_nibbles(np.array([d["bytes"]], np.uint8), 4)
    assert O.decode(u, O.SYM).ravel().tolist() == d["values"]
    with pytest.raises(ValueError):
        O.validate_packed(np.array([d["bytes"]], np.uint8), np.ones((1, 1), F32), None, 4, 32, O.SYM)
    O.validate_packed(np.array([d["bytes"]], np.uint8), np.ones((1, 1), F32), None, 4, 32, O.SYM,
                      narrow=False)


def test_golden_linear(golden):
    lin = golden["linear"]
    c = next(c for c in golden["cases"] if c["name"] == lin["case"])
    codes, s, z = O.quantize_pack(np.array(c["w"], F32), c["G"], c["mode"])
    xb = O.f32_to_bf16_bits(np.array(lin["x"], F32))
    bb = O.f32_to_bf16_bits(np.array(lin["bias"], F32))
    y = O.linear(xb, codes, s, z, None, c["K"], c["G"], c["mode"], bb)
    assert y.tolist() == lin["y"]


# --------------------------------------------------------------------------
# bit-level pins against library routines
# --------------------------------------------------------------------------
def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(1)
    parts = [
        rng.standard_normal(200000).astype(F32),
        (rng.standard_normal(50000) * 1e-39).astype(F32),     # fp32 subnormals
        (rng.standard_normal(50000) * 1e30).astype(F32),
        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38], F32),
        # largest bf16 and the values that round past it to infinity
        np.array([0x7F7F0000, 0x7F7F7FFF, 0x7F7F8000, 0x7F7FFFFF,
                  0xFF7F7FFF, 0xFF7F8000, 0xFF7FFFFF], np.uint32).view(F32),
    ]
    # exact ties: low 16 bits = 0x8000, both parities of bit 16
    u = rng.integers(0, 2**32, 100000, dtype=np.uint64).astype(np.uint32)
    u = (u & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    u = u[((u >> 23) & 0xFF) < 0xFE]                          # keep finite after rounding
    parts.append(u.view(F32))
    x = np.concatenate(parts)
    ours = O.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(O.bf16_bits_to_f32(ref), torch.from_numpy(ref.view(np.int16).copy())
                          .view(torch.bfloat16).float().numpy())


def test_all_bytes_decode_against_sign_extension():
    b = np.arange(256, dtype=np.uint8)[None, :]
    u = O.unpack_nibbles(b, 512)
    assert np.array_equal(u[0, 0::2], np.arange(256) & 15)
    assert np.array_equal(u[0, 1::2], np.arange(256) >> 4)
    # two's-complement nibble = arithmetic shift of the nibble placed at the top of an int8
    ref = ((u.astype(np.uint8) << 4).view(np.int8) >> 4).astype(np.int32)
    assert np.array_equal(O.decode(u, O.SYM), ref)
    # closed form (c xor 8) - 8
    assert np.array_equal(O.decode(u, O.SYM), (u.astype(np.int32) ^ 8) - 8)


@pytest.mark.parametrize("K", [1, 2, 7, 8, 33, 64])
def test_pack_unpack_round_trip(K):
    rng = np.random.default_rng(K)
    q = rng.integers(-8, 8, size=(5, K))
    codes = O.pack_nibbles(q)
    assert codes.shape == (5, (K + 1) // 2) and codes.dtype == np.uint8
    assert np.array_equal(O.decode(O.unpack_nibbles(codes, K), O.SYM), q)
    if K % 2:
        assert not np.any(codes[:, -1] >> 4)
    u = rng.integers(0, 16, size=(3, K))
    assert np.array_equal(O.unpack_nibbles(O.pack_nibbles(u), K), u)


# --------------------------------------------------------------------------
# invariants of quantize (|w - dq| <= s/2 up to fp32 rounding)
# --------------------------------------------------------------------------
BOUND = 0.5 + 2.0 ** -19   # half a step plus fp32 rounding of w/s and of v*s


def _check_invariants(w, G, mode, g_idx=None):
    N, K = w.shape
    codes, s, z = O.quantize_pack(w, G, mode, g_idx)
    O.validate_packed(codes, s, z, K, G, mode, g_idx)
    gid = O.group_of_columns(K, G, g_idx)
    u = O.unpack_nibbles(codes, K)
    v = O.decode(u, mode, z, gid)
    d = O.dequantize(codes, s, z, g_idx, K, G, mode, "f32")
    sk = s[:, gid]
    err = np.abs(w.astype(np.float64) - d.astype(np.float64))
    assert np.all(err <= BOUND * sk.astype(np.float64))
    if mode == O.SYM:
        assert v.min() >= -7 and v.max() <= 7
        for g in np.unique(gid):
            cols = gid == g
            nz = np.any(w[:, cols] != 0, axis=1)
            assert np.all(np.max(np.abs(v[:, cols]), axis=1)[nz] == 7)
    else:
        assert u.max() <= 15 and z.max() <= 15
        # the zero-point code dequantizes to exactly 0
        assert np.all(d[u == z[:, gid]] == 0)
    return codes, s, z


@pytest.mark.parametrize("mode", [O.SYM, O.ASYM])
@pytest.mark.parametrize("K,G", [(512, 32), (8191 % 700, 32), (384, 128), (100, 64), (33, 8)])
def test_quantize_invariants(mode, K, G):
    rng = np.random.default_rng(K * 7 + G)
    w = (rng.standard_normal((24, K)) * 0.02).astype(F32)
    w[3] = 0                                       # all-zero row
    w[4, :G] = np.abs(w[4, :G])                    # one-signed groups
    w[5, :G] = -np.abs(w[5, :G])
    w[6, ::5] *= 8                                 # outliers
    _check_invariants(w, G, mode)


def test_quantize_invariants_workload_tiny():
    wl = workload("tiny")
    t = generate(wl)
    _check_invariants(t["w"].numpy(), wl.G, wl.mode)


def test_quantize_invariants_prefill_like_act_order():
    wl = workload("prefill", N=64, K=512, M=4)
    t = generate(wl)
    _check_invariants(t["w"].numpy(), wl.G, wl.mode, t["g_idx"].numpy())


def test_asym_recovers_group_extremes():
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((16, 256)) * 0.02).astype(F32)
    codes, s, z = O.quantize_pack(w, 64, O.ASYM)
    d = O.dequantize(codes, s, z, None, 256, 64, O.ASYM, "f32").reshape(16, 4, 64)
    wg = w.reshape(16, 4, 64)
    tol = BOUND * s[:, :, None]
    assert np.all(np.abs(d.max(-1, keepdims=True) - wg.max(-1, keepdims=True)) <= tol)
    assert np.all(np.abs(d.min(-1, keepdims=True) - wg.min(-1, keepdims=True)) <= tol)


# --------------------------------------------------------------------------
# special cases
# --------------------------------------------------------------------------
def test_per_channel_matches_gemma_uniform_quantize():
    """G = K reduces to per-channel symmetric absmax.  The Gemma page computes
    codes as clip(round(x * (7 / max|x|)), -8, 7), an inverse-scale multiply
    instead of a divide; the two agree except for +-1 at near-ties."""
    rng = np.random.default_rng(11)
    K = 1024
    w = (rng.standard_normal((512, K)) * 0.02).astype(F32)
    q, s, _ = O.quantize(w, O.PER_CHANNEL, O.SYM)
    assert s.shape == (512, 1) and O.n_groups(K, O.PER_CHANNEL) == 1
    qk, sk, _ = O.quantize(w, K, O.SYM)          # G = K and G > K name the same single group
    qb, sb, _ = O.quantize(w, K + 8, O.SYM)
    assert np.array_equal(q, qk) and np.array_equal(q, qb) and np.array_equal(s, sk) and np.array_equal(s, sb)
    inv = (F32(7) * (F32(1) / np.max(np.abs(w), axis=1))).astype(F32)
    qg = np.clip(np.rint((w * inv[:, None]).astype(F32)), -8, 7)
    diff = q.astype(np.int32) - qg.astype(np.int32)
    assert np.all(np.abs(diff) <= 1)
    assert np.mean(diff != 0) < 1e-4
    # every disagreement sits at a near-tie of the exact quotient
    xs = w.astype(np.float64) / s.astype(np.float64)
    frac = np.abs(np.abs(xs - np.floor(xs)) - 0.5)
    assert np.all(frac[diff != 0] < 1e-5)
    # the scale is max|w| / 7 to within one fp32 rounding
    np.testing.assert_allclose(s[:, 0], np.max(np.abs(w), axis=1) / 7.0, rtol=2 ** -23)


@pytest.mark.parametrize("mode", [O.SYM, O.ASYM])
def test_default_g_idx_equals_contiguous(mode):
    rng = np.random.default_rng(3)
    K, G = 300, 32
    w = (rng.standard_normal((20, K)) * 0.02).astype(F32)
    a = O.quantize_pack(w, G, mode)
    b = O.quantize_pack(w, G, mode, (np.arange(K) // G).astype(np.int32))
    for x, y in zip(a, b):
        assert (x is None and y is None) or np.array_equal(x, y)


@pytest.mark.parametrize("mode", [O.SYM, O.ASYM])
def test_g_idx_is_column_permutation(mode):
    """With every group holding exactly G columns, quantizing with g_idx equals
    quantizing the column-sorted matrix with contiguous groups."""
    rng = np.random.default_rng(4)
    K, G = 256, 32
    w = (rng.standard_normal((16, K)) * 0.02).astype(F32)
    g_idx = (rng.permutation(K) // G).astype(np.int32)
    P = np.argsort(g_idx, kind="stable")
    q1, s1, z1 = O.quantize(w, G, mode, g_idx)
    q2, s2, z2 = O.quantize(w[:, P], G, mode)
    assert np.array_equal(q1[:, P], q2) and np.array_equal(s1, s2)
    if mode == O.ASYM:
        assert np.array_equal(z1, z2)
    d1 = O.dequantize(O.pack_nibbles(q1), s1, z1, g_idx, K, G, mode, "bf16")
    d2 = O.dequantize(O.pack_nibbles(q2), s2, z2, None, K, G, mode, "bf16")
    assert np.array_equal(d1[:, P], d2)


def test_dequant_bf16_is_rounded_f32():
    rng = np.random.default_rng(6)
    w = (rng.standard_normal((8, 200)) * 0.02).astype(F32)
    c, s, z = O.quantize_pack(w, 32, O.ASYM)
    f = O.dequantize(c, s, z, None, 200, 32, O.ASYM, "f32")
    b = O.dequantize(c, s, z, None, 200, 32, O.ASYM, "bf16")
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, ref)
    # fp32 product of a small integer and the scale, checked in fp64
    v = O.decode(O.unpack_nibbles(c, 200), O.ASYM, z, np.arange(200) // 32)
    exact = v * s[:, np.arange(200) // 32].astype(np.float64)
    assert np.all(np.abs(f - exact) <= np.abs(exact) * 2.0 ** -24)


# --------------------------------------------------------------------------
# linear
# --------------------------------------------------------------------------
def _brute_linear(xf, wd, b):
    M, K = xf.shape
    N = wd.shape[0]
    y = [[0.0] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc += float(xf[m][k]) * float(wd[n][k])
            y[m][n] = acc + (float(b[n]) if b is not None else 0.0)
    return np.array(y)


def _hand_dequant(codes, s, z, g_idx, N, K, G, mode):
    """bf16-rounded dequantized weight decoded by hand, element by element."""
    gid = np.arange(K) // G if g_idx is None else g_idx
    wd = np.zeros((N, K))
    for n in range(N):
        for k in range(K):
            byte = int(codes[n, k // 2])
            nib = (byte >> 4) if (k & 1) else (byte & 15)
            val = (nib - 16 if nib >= 8 else nib) if mode == O.SYM else nib - int(z[n, gid[k]])
            prod = np.float32(np.float32(val) * s[n, gid[k]])
            wd[n, k] = torch.tensor(float(prod), dtype=torch.float32).to(torch.bfloat16).item()
    return wd


@pytest.mark.parametrize("mode,g_act", [(O.SYM, False), (O.ASYM, True)])
def test_linear_grad_input_brute_force(mode, g_act):
    """dx[m, k] = sum_n dy[m, n] Wd[n, k], summed by explicit loops."""
    rng = np.random.default_rng(19)
    M, N, K, G = 3, 6, 29, 8
    w = (rng.standard_normal((N, K)) * 0.02).astype(F32)
    g_idx = (rng.permutation(K) % O.n_groups(K, G)).astype(np.int32) if g_act else None
    codes, s, z = O.quantize_pack(w, G, mode, g_idx)
    dyb = O.f32_to_bf16_bits(rng.standard_normal((M, N)).astype(F32))
    dx = O.linear_grad_input(dyb, codes, s, z, g_idx, K, G, mode, row_chunk=4)
    wd = _hand_dequant(codes, s, z, g_idx, N, K, G, mode)
    dyf = torch.from_numpy(dyb.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    ref = np.zeros((M, K))
    for m in range(M):
        for k in range(K):
            acc = 0.0
            for n in range(N):
                acc += dyf[m, n] * wd[n, k]
            ref[m, k] = acc
    np.testing.assert_allclose(dx, ref, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("mode", [O.SYM, O.ASYM])
def test_linear_grad_input_is_the_adjoint(mode):
    """<x Wd^T, dy> = <x, dy Wd> for any x, dy: the gradient is the transpose
    of the forward map (a dropped or transposed index breaks the identity)."""
    rng = np.random.default_rng(20)
    M, N, K, G = 4, 33, 64, 16
    w = (rng.standard_normal((N, K)) * 0.02).astype(F32)
    g_idx = (rng.permutation(K) // G).astype(np.int32)
    codes, s, z = O.quantize_pack(w, G, mode, g_idx)
    xb = O.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(F32))
    dyb = O.f32_to_bf16_bits(rng.standard_normal((M, N)).astype(F32))
    y = O.linear(xb, codes, s, z, g_idx, K, G, mode, None)
    dx = O.linear_grad_input(dyb, codes, s, z, g_idx, K, G, mode)
    lhs = float(np.sum(y * O.bf16_bits_to_f32(dyb).astype(np.float64)))
    rhs = float(np.sum(O.bf16_bits_to_f32(xb).astype(np.float64) * dx))
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))


def test_linear_grad_input_unit_rows_return_weight_rows():
    """dy = unit rows e_n gives the bf16 dequantized rows of W exactly."""
    rng = np.random.default_rng(21)
    N, K, G = 7, 48, 16
    w = (rng.standard_normal((N, K)) * 0.02).astype(F32)
    codes, s, z = O.quantize_pack(w, G, O.ASYM)
    dyb = O.f32_to_bf16_bits(np.eye(N, dtype=F32))
    dx = O.linear_grad_input(dyb, codes, s, z, None, K, G, O.ASYM)
    wd = O.bf16_bits_to_f32(O.dequantize(codes, s, z, None, K, G, O.ASYM, "bf16"))
    assert np.array_equal(dx, wd.astype(np.float64))


@pytest.mark.parametrize("mode,g_act", [(O.SYM, False), (O.ASYM, True)])
def test_linear_brute_force(mode, g_act):
    rng = np.random.default_rng(9)
    M, N, K, G = 3, 5, 37, 8
    w = (rng.standard_normal((N, K)) * 0.02).astype(F32)
    g_idx = (rng.permutation(K) % O.n_groups(K, G)).astype(np.int32) if g_act else None
    codes, s, z = O.quantize_pack(w, G, mode, g_idx)
    xb = O.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(F32))
    bb = O.f32_to_bf16_bits((rng.standard_normal(N) * 0.01).astype(F32))
    y = O.linear(xb, codes, s, z, g_idx, K, G, mode, bb, row_chunk=2)
    # brute force from the pieces: unpack by hand, decode, scale, round via torch
    gid = np.arange(K) // G if g_idx is None else g_idx
    wd = np.zeros((N, K))
    for n in range(N):
        for k in range(K):
            byte = int(codes[n, k // 2])
            nib = (byte >> 4) if (k & 1) else (byte & 15)
            if mode == O.SYM:
                val = nib - 16 if nib >= 8 else nib
            else:
                val = nib - int(z[n, gid[k]])
            prod = np.float32(np.float32(val) * s[n, gid[k]])
            wd[n, k] = torch.tensor(float(prod), dtype=torch.float32).to(torch.bfloat16).item()
    xf = torch.from_numpy(xb.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    bf = torch.from_numpy(bb.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    yb = _brute_linear(xf, wd, bf)
    np.testing.assert_allclose(y, yb, rtol=1e-12, atol=1e-15)


def test_linear_identity_returns_dequantized_weight():
    rng = np.random.default_rng(12)
    N, K, G = 9, 40, 8
    w = (rng.standard_normal((N, K)) * 0.02).astype(F32)
    codes, s, z = O.quantize_pack(w, G, O.ASYM)
    eye = O.f32_to_bf16_bits(np.eye(K, dtype=F32))
    y = O.linear(eye, codes, s, z, None, K, G, O.ASYM)
    wd = O.bf16_bits_to_f32(O.dequantize(codes, s, z, None, K, G, O.ASYM, "bf16"))
    assert np.array_equal(y.T, wd.astype(np.float64))


def test_workload_inputs_are_seeded_and_shaped():
    wl = workload("prefill", N=32, K=256, M=8)
    a, b = generate(wl), generate(wl)
    assert torch.equal(a["w"], b["w"]) and torch.equal(a["x"], b["x"])
    g = a["g_idx"].numpy()
    assert np.array_equal(np.bincount(g), np.full(256 // 128, 128))
    t = generate(workload("codec", N=4, K=33))
    assert t["w"].dtype == torch.bfloat16 and t["x"] is None
    assert bf16_bits(t["w"]).dtype == np.uint16


def test_payload_bytes_matches_format():
    codes = np.zeros((3, 5), np.uint8)
    scales = np.ones((3, 1), F32)
    assert O.payload_bytes(codes, scales) == 15 + 12
    assert O.payload_bytes(codes, scales, np.zeros((3, 1), np.uint8)) == 15 + 12 + 3


def test_validate_rejects_malformed():
    codes = np.zeros((2, 3), np.uint8)
    s = np.ones((2, 1), F32)
    O.validate_packed(codes, s, None, 5, 32, O.SYM)
    bad = codes.copy()
    bad[1, 2] = 0x10                                   # odd width, high nibble set
    with pytest.raises(ValueError):
        O.validate_packed(bad, s, None, 5, 32, O.SYM)
    with pytest.raises(ValueError):
        O.validate_packed(codes, np.zeros((2, 1), F32), None, 5, 32, O.SYM)
    with pytest.raises(ValueError):
        O.validate_packed(codes, np.full((2, 1), np.inf, F32), None, 5, 32, O.SYM)
    with pytest.raises(ValueError):
        O.validate_packed(codes, s, np.full((2, 1), 16, np.uint8), 5, 32, O.ASYM)
    with pytest.raises(ValueError):
        O.validate_packed(codes, s, None, 5, 32, O.SYM, g_idx=np.array([0, 0, 1, 0, 0]))


# --------------------------------------------------------------------------
# LoRA merge ([Keras] Dense._get_kernel_with_merged_lora)
# --------------------------------------------------------------------------
def _nearest_f32_of(fr):
    """fp32 nearest to the rational ``fr`` (checked against both neighbours)."""
    from fractions import Fraction
    c = np.float32(float(fr))
    for nb in (np.nextafter(c, np.float32(np.inf)), np.nextafter(c, np.float32(-np.inf))):
        assert abs(Fraction(float(c)) - fr) <= abs(Fraction(float(nb)) - fr)
    return c


def test_lora_update_is_the_correctly_rounded_product():
    """With all-zero codes (Wd = 0) and c = 1 the merged weight is the update
    itself: every entry must be the fp32 nearest to the exact rational
    sum_j A[k, j] B[j, n] (A is [K, r], B is [r, N]: entry (n, k))."""
    from fractions import Fraction
    rng = np.random.default_rng(21)
    N, K, r = 5, 9, 3
    A = rng.standard_normal((K, r)).astype(F32)
    B = rng.standard_normal((r, N)).astype(F32)
    codes = np.zeros((N, (K + 1) // 2), dtype=np.uint8)
    scales = np.ones((N, 1), dtype=F32)
    got = O.lora_merged_weight(codes, scales, None, None, K, O.PER_CHANNEL, O.SYM, A, B, 1.0)
    for n in range(N):
        for k in range(K):
            exact = sum(Fraction(float(A[k, j])) * Fraction(float(B[j, n])) for j in range(r))
            assert got[n, k] == _nearest_f32_of(exact), (n, k)


@pytest.mark.parametrize("mode", [O.SYM, O.ASYM])
def test_lora_zero_update_requantizes_to_itself(mode):
    """c = 0 leaves the dequantized weight; quantizing it again must give the
    same codes and zero-points (the quantizer is idempotent on its own grid:
    every group reaches its extreme codes), and scales within one fp32 ulp."""
    rng = np.random.default_rng(22)
    N, K, G, r = 48, 320, 64, 4
    w = (rng.standard_normal((N, K)) * 0.02).astype(F32)
    c, s, z = O.quantize_pack(w, G, mode)
    A = rng.standard_normal((K, r)).astype(F32)
    B = rng.standard_normal((r, N)).astype(F32)
    c2, s2, z2 = O.lora_merge(c, s, z, None, K, G, mode, A, B, 0.0)
    assert np.array_equal(c2, c)
    if z is not None:
        assert np.array_equal(z2, z)
    ulps = np.abs(s2.view(np.int32).astype(np.int64) - s.view(np.int32).astype(np.int64))
    assert ulps.max() <= 1


@pytest.mark.parametrize("mode,G,act", [(O.SYM, 32, False), (O.ASYM, 64, False), (O.ASYM, 32, True),
                                        (O.SYM, O.PER_CHANNEL, False)])
def test_lora_merge_is_within_the_quantization_bound(mode, G, act):
    """End to end against real arithmetic: the merged codes dequantize to
    Wd + (alpha / r) A B (exact, fp64 matmul) within half a step of the new
    group scale (plus the fp32 roundings of the merge)."""
    rng = np.random.default_rng(23)
    N, K, r, alpha = 40, 256, 8, 16.0
    w = (rng.standard_normal((N, K)) * 0.02).astype(F32)
    gidx = (rng.permutation(K) // 32).astype(np.int32) if act else None
    c, s, z = O.quantize_pack(w, G, mode, gidx)
    A = (rng.standard_normal((K, r)) * 0.05).astype(F32)    # update ~ 2 quantization steps
    B = (rng.standard_normal((r, N)) * 0.05).astype(F32)
    c2, s2, z2 = O.lora_merge(c, s, z, gidx, K, G, mode, A, B, alpha / r)
    target = O.dequantize(c, s, z, gidx, K, G, mode, out="f32").astype(np.float64) \
        + (alpha / r) * (A.astype(np.float64) @ B.astype(np.float64)).T
    got = O.dequantize(c2, s2, z2, gidx, K, G, mode, out="f32").astype(np.float64)
    step = s2.astype(np.float64)[:, O.group_of_columns(K, G, gidx)]
    slack = 4 * np.finfo(np.float32).eps * (np.abs(target) + step)
    assert np.all(np.abs(got - target) <= 0.5 * step + slack)
    # the update is not lost: at this size it moves many codes
    assert np.mean(c2 != c) > 0.1


# --------------------------------------------------------------------------
# packed zero-points (R10)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("NG", [1, 2, 7, 32, 33])
def test_packed_zeros_layout_and_round_trip(NG):
    rng = np.random.default_rng(31 + NG)
    z = rng.integers(0, 16, size=(5, NG)).astype(np.uint8)
    p = O.pack_zeros(z)
    assert p.shape == (5, (NG + 1) // 2) and p.dtype == np.uint8
    # byte j holds group 2j (low nibble) and group 2j + 1 (high nibble), written out
    for n in range(5):
        for j in range(p.shape[1]):
            hi = int(z[n, 2 * j + 1]) if 2 * j + 1 < NG else 0
            assert int(p[n, j]) == int(z[n, 2 * j]) + 16 * hi
    assert np.array_equal(O.unpack_zeros(p, NG), z)
    with pytest.raises(ValueError):
        O.pack_zeros(np.full((1, 2), 16, dtype=np.uint8))


# --------------------------------------------------------------------------
# GGUF Q4_0 block codec (R11)
# --------------------------------------------------------------------------
def test_q4_0_hand_worked_block():
    """w[i] = (i - 16) * 7/128: amax = 7/8, so d = 1/8 exactly (fp16 0x3000) and
    w/d = (i - 16) * 7/16; i = 8 and 24 are exact ties (-3.5, 3.5 -> -4, 4).
    Expected bytes from exact rationals and Python's half-even round()."""
    from fractions import Fraction
    w = np.array([[(i - 16) * 7 / 128 for i in range(32)]], dtype=F32)
    got = O.q4_0_quantize(w)
    assert got.shape == (1, 1, 18)
    q = [max(-7, min(7, round(Fraction(i - 16) * Fraction(7, 16)))) for i in range(32)]
    assert q[8] == -4 and q[24] == 4
    expect = [0x00, 0x30] + [(q[i] + 8) | ((q[i + 16] + 8) << 4) for i in range(16)]
    assert got[0, 0].tolist() == expect
    # and back: (q - 8) * d with d = 1/8, exact
    assert np.array_equal(O.q4_0_dequantize(got)[0], np.array([qq / 8 for qq in q], dtype=F32))


def test_q4_0_decodes_hand_built_bytes():
    """d = 0.5 (fp16 0x3800); byte 2 + i = low nibble a_i, high nibble b_i gives
    weight i = (a_i - 8) / 2 and weight 16 + i = (b_i - 8) / 2."""
    blk = np.zeros((1, 1, 18), dtype=np.uint8)
    blk[0, 0, 0:2] = [0x00, 0x38]
    lo = [(3 * i) % 16 for i in range(16)]
    hi = [(5 * i + 1) % 16 for i in range(16)]
    blk[0, 0, 2:] = [a | (b << 4) for a, b in zip(lo, hi)]
    want = [(a - 8) / 2 for a in lo] + [(b - 8) / 2 for b in hi]
    assert O.q4_0_dequantize(blk)[0].tolist() == want


def test_q4_0_equals_signed_group32_when_the_scale_is_exact():
    """When amax / 7 is representable in fp16 the Q4_0 block holds exactly the
    signed G = 32 quantization (R3): same codes, same dequantized values."""
    rng = np.random.default_rng(41)
    N, K = 16, 256
    w = (rng.uniform(-1, 1, size=(N, K)) * 0.8).astype(F32)
    blk = w.reshape(N, K // 32, 32)
    pos = rng.integers(0, 32, size=(N, K // 32))
    scale = np.float32(2.0) ** rng.integers(-6, 2, size=(N, K // 32)).astype(F32)
    for n in range(N):
        for b in range(K // 32):
            blk[n, b] *= scale[n, b]
            blk[n, b, pos[n, b]] = 0.875 * scale[n, b] * (1 if (n + b) % 2 else -1)   # amax = 7 * 2^k / 8
    w = blk.reshape(N, K)
    q4 = O.q4_0_quantize(w)
    qs = q4[..., 2:]
    u = np.concatenate([qs & 15, qs >> 4], axis=-1).reshape(N, K).astype(np.int16) - 8
    q, s, _ = O.quantize(w, 32, O.SYM)
    assert np.array_equal(u, q)
    assert np.array_equal(O.q4_0_dequantize(q4), O.dequantize(O.pack_nibbles(q), s, None, None, K, 32, O.SYM, "f32"))


def test_q4_0_scale_is_nearest_fp16_and_error_bound():
    rng = np.random.default_rng(42)
    w = (rng.standard_normal((64, 512)) * 0.02).astype(F32)
    q4 = O.q4_0_quantize(w)
    d = np.ascontiguousarray(q4[..., 0:2]).view("<f2")[..., 0].astype(np.float64)
    amax = np.max(np.abs(w.reshape(64, 16, 32)), axis=2).astype(np.float64)
    ideal = amax / 7
    # nearest fp16: no fp16 neighbour is closer (fp32(amax/7) is within 2^-24 relative)
    for nb in (np.nextafter(d.astype(np.float16), np.float16(np.inf)), np.nextafter(d.astype(np.float16), np.float16(0))):
        assert np.all(np.abs(d - ideal) <= np.abs(nb.astype(np.float64) - ideal) + ideal * 2 ** -23)
    deq = O.q4_0_dequantize(q4).astype(np.float64).reshape(64, 16, 32)
    err = np.abs(deq - w.astype(np.float64).reshape(64, 16, 32))
    bound = d[..., None] / 2 + 7 * np.abs(ideal - d)[..., None] + 1e-12
    assert np.all(err <= bound * (1 + 2 ** -20))
    u = np.concatenate([q4[..., 2:] & 15, q4[..., 2:] >> 4], axis=-1)
    assert u.min() >= 1 and u.max() <= 15          # codes q + 8 with |q| <= 7


def test_q4_0_zero_block_and_shape_check():
    w = np.zeros((2, 64), dtype=F32)
    w[1, 32:] = np.linspace(-1, 1, 32, dtype=F32)
    q4 = O.q4_0_quantize(w)
    assert q4[0].tolist() == [[0, 0] + [0x88] * 16] * 2 and q4[1, 0].tolist() == [0, 0] + [0x88] * 16
    assert np.all(O.q4_0_dequantize(q4)[0] == 0)
    with pytest.raises(ValueError):
        O.q4_0_quantize(np.zeros((1, 48), dtype=F32))


def test_q4_0_quantizes_against_the_stored_scale():
    """The codes are taken against the stored fp16 d, and clamped to [-7, 7].
    amax = 1: d = fp16(1/7) = 1170/1024 * 2^-3, 0.024% below 1/7; the weight
    3.5 d is an exact tie for d (-> 4) but lies below the tie for 1/7 (-> 3).
    A block with amax = 10 * 2^-24 has d = 2^-24 (the smallest fp16
    subnormal), so w / d = 10 clamps to 7."""
    d16 = 1170 / 1024 / 8
    w = np.zeros((2, 32), dtype=F32)
    w[0, 0] = 1.0
    w[0, 1] = 3.5 * d16
    w[1, 0] = 10 * 2.0 ** -24
    q4 = O.q4_0_quantize(w)
    assert np.ascontiguousarray(q4[0, 0, 0:2]).view("<f2")[0] == np.float16(d16)
    assert (q4[0, 0, 2] & 15) == 15 and (q4[0, 0, 3] & 15) == 8 + 4
    assert np.ascontiguousarray(q4[1, 0, 0:2]).view("<f2")[0] == np.float16(2.0 ** -24)
    assert (q4[1, 0, 2] & 15) == 15
