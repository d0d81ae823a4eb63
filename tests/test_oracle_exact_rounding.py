"""Pins for the rounding of every fp32 step of the oracle's quantizer.

The quantizer's steps are IEEE binary32 operations, each rounded once to the
nearest value with ties to even, in the order the readings state (the signed
scale max|w| / 7; the zero-point scale (hi - lo) / 15 and zero-point
rint(-lo / s); the codes rint(w / s), clamped to the code range; the Gemma
``_quantization_utils.py`` page's ``uniform_quantize`` rounds with jnp.round,
half to even; the keras ``dense.py`` diff page's int4 branch of
``Dense.quantize`` quantizes each block of the kernel against its own scale).

Here the expected values come from exact rational arithmetic
(``fractions.Fraction``) and the definition of rounding to the nearest
binary32 number, written from the IEEE 754 definition (53-bit doubles and
numpy are not used for any expected value).  A quantizer that multiplies by
a rounded reciprocal instead of dividing, or that rounds a quotient twice,
disagrees with these values on the inputs below: the tests also check that
each input set would expose that slip, so a pin cannot pass vacuously.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import w4_oracle as O

F32 = np.float32
HALF = Fraction(1, 2)


def rn32(q: Fraction) -> Fraction:
    """The binary32 number nearest to the rational q, ties to the even
    significand; gradual underflow below 2^-126 (spacing 2^-149).  The tests
    never reach the overflow threshold."""
    if q == 0:
        return Fraction(0)
    neg = q < 0
    a = -q if neg else q
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if a < Fraction(2) ** e:
        e -= 1                                  # now 2^e <= a < 2^(e+1)
    spacing = Fraction(2) ** (max(e, -126) - 23)
    m = a / spacing
    n = m.numerator // m.denominator
    r = m - n
    if r > HALF or (r == HALF and n % 2 == 1):
        n += 1
    v = n * spacing
    assert v < Fraction(2) ** 128
    return -v if neg else v


def rint_even(v: Fraction) -> int:
    """Nearest integer, ties to even."""
    n = v.numerator // v.denominator            # floor
    r = v - n
    if r > HALF or (r == HALF and n % 2 == 1):
        n += 1
    return n


def exact_group(vals, mode):
    """(s, z, codes) of one group from its fp32 values (given as Fractions),
    every operation rounded once to binary32."""
    if mode == O.SYM:
        amax = max(abs(v) for v in vals)
        s = rn32(amax / 7)
        if s == 0:
            s = Fraction(1)
        return s, None, [min(7, max(-7, rint_even(rn32(v / s)))) for v in vals]
    lo = min(Fraction(0), min(vals))
    hi = max(Fraction(0), max(vals))
    span = rn32(hi - lo)
    s = rn32(span / 15)
    if s == 0:
        s = Fraction(1)
    z = min(15, max(0, rint_even(rn32(-lo / s))))
    return s, z, [min(15, max(0, rint_even(rn32(v / s)) + z)) for v in vals]


def exact_quantize(w, G, mode, g_idx=None):
    """Exact-rational quantization of fp32 w [N, K]: codes int [N, K],
    scales [N, NG] and zero-points [N, NG] as Python numbers."""
    N, K = w.shape
    NG = O.n_groups(K, G)
    gid = np.arange(K) // G if g_idx is None else np.asarray(g_idx)
    q = [[None] * K for _ in range(N)]
    sc = [[Fraction(1)] * NG for _ in range(N)]
    zp = [[0] * NG for _ in range(N)]
    for n in range(N):
        row = [Fraction(float(v)) for v in w[n]]
        for g in range(NG):
            cols = [k for k in range(K) if gid[k] == g]
            if not cols:
                continue
            s, z, codes = exact_group([row[k] for k in cols], mode)
            sc[n][g] = s
            zp[n][g] = 0 if z is None else z
            for k, c in zip(cols, codes):
                q[n][k] = c
    return q, sc, zp


def assert_oracle_exact(w, G, mode, g_idx=None):
    q, s, z = O.quantize(w, G, mode, g_idx)
    eq, es, ez = exact_quantize(w, G, mode, g_idx)
    N, K = w.shape
    for n in range(N):
        for g in range(s.shape[1]):
            assert Fraction(float(s[n, g])) == es[n][g], f"scale ({n}, {g})"
            if mode == O.ASYM:
                assert int(z[n, g]) == ez[n][g], f"zero-point ({n}, {g})"
        assert q[n].tolist() == eq[n], f"codes of row {n}"


def inverse_form_quantize(w, G, mode):
    """The tempting variant the pins must reject: every division replaced by a
    multiply with the rounded reciprocal (contiguous groups only)."""
    N, K = w.shape
    b = w.reshape(N, K // G, G)
    if mode == O.SYM:
        amax = np.max(np.abs(b), axis=2, keepdims=True)
        s = (amax * (F32(1) / F32(7))).astype(F32)
        s[s == 0] = F32(1)
        return np.clip(np.rint((b * (F32(1) / s).astype(F32)).astype(F32)), -7, 7).reshape(N, K), s, None
    lo = np.minimum(b.min(axis=2, keepdims=True), F32(0))
    hi = np.maximum(b.max(axis=2, keepdims=True), F32(0))
    s = ((hi - lo).astype(F32) * (F32(1) / F32(15))).astype(F32)
    s[s == 0] = F32(1)
    r = (F32(1) / s).astype(F32)
    z = np.clip(np.rint((-lo * r).astype(F32)), 0, 15)
    q = np.clip(np.rint((b * r).astype(F32)) + z, 0, 15)
    return q.reshape(N, K), s, z


def _bf16_weights(N, K, std, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(N, K, generator=g) * std).to(torch.bfloat16).float().numpy()


# --------------------------------------------------------------------------
# random weights: bf16-valued (short significands make exact half-integer
# quotients common, as in the codec workload) and full fp32
# --------------------------------------------------------------------------
@pytest.mark.parametrize("mode", [O.SYM, O.ASYM])
@pytest.mark.parametrize("G", [32, 128])
def test_quantizer_rounds_every_step_once_bf16_weights(mode, G):
    w = _bf16_weights(48, 512, 0.02, 11 + G)
    assert_oracle_exact(w, G, mode)
    # teeth: the reciprocal-multiply variant disagrees on these weights
    q, s, z = O.quantize(w, G, mode)
    qi, si, zi = inverse_form_quantize(w, G, mode)
    assert not np.array_equal(q, qi)


@pytest.mark.parametrize("mode", [O.SYM, O.ASYM])
def test_quantizer_rounds_every_step_once_fp32_weights(mode):
    g = torch.Generator().manual_seed(5)
    w = (torch.randn(24, 256, generator=g) * 0.02).numpy()
    w[3, 7] *= 8.0                                    # an outlier, as in the batched-decode weights
    assert_oracle_exact(w, 32, mode)
    _, s, _ = O.quantize(w, 32, mode)
    _, si, _ = inverse_form_quantize(w, 32, mode)
    assert not np.array_equal(s.ravel(), si.ravel())  # the scale quotient itself has teeth here


@pytest.mark.parametrize("mode", [O.SYM, O.ASYM])
def test_quantizer_exact_with_scattered_groups(mode):
    w = _bf16_weights(16, 256, 0.02, 21)
    perm = torch.randperm(256, generator=torch.Generator().manual_seed(22)).numpy()
    g_idx = (perm // 32).astype(np.int32)
    assert_oracle_exact(w, 32, mode, g_idx)


def test_quantizer_exact_on_degenerate_groups():
    # all-zero group (s = 1), one-signed groups (lo or hi pinned at 0), subnormal
    # magnitudes (the scale quotient underflows or is inexact)
    w = np.zeros((4, 64), F32)
    w[1, :32] = np.linspace(0.5, 3.0, 32, dtype=F32)
    w[1, 32:] = -np.linspace(0.25, 1.0, 32, dtype=F32)
    w[2, :32] = np.float32(3e-44) * np.arange(32, dtype=F32)
    w[3, :32] = F32(1e-39)
    w[3, 5] = F32(-2e-39)
    for mode in (O.SYM, O.ASYM):
        assert_oracle_exact(w, 32, mode)


# --------------------------------------------------------------------------
# constructed groups whose quotients are exact half-integers, where one
# rounding (division) and two roundings (reciprocal, then product) part ways
# --------------------------------------------------------------------------
def _half_integer_cases(halves):
    """Scales s = k / 2^j (odd k < 256) with a half-integer h of `halves` for
    which rint(fp32(h s * fp32(1/s))) differs from rint(fp32(h s / s)) = the
    even neighbour of h.  Deterministic search."""
    found = []
    for k in range(3, 256, 2):
        for j in range(0, 8):
            s = F32(k / 2 ** j)
            for h in halves:
                w = F32(h) * s
                if np.rint(F32(w / s)) != np.rint(F32(w * F32(F32(1) / s))):
                    found.append((s, h))
    return found


def test_constructed_half_integer_quotients_divide_once():
    cases = _half_integer_cases((0.5, 1.5, 2.5, 3.5, 4.5, 5.5, 6.5))
    assert len(cases) > 50
    rows = []
    for s, h in cases[:64]:
        # signed group: max|w| = 7 s gives the scale s exactly; then w = +-h s
        rows.append([F32(7) * s, F32(h) * s, -F32(h) * s, F32(0.5) * s] + [F32(0)] * 4)
    w = np.array(rows, F32)
    assert_oracle_exact(w, 8, O.SYM)
    q, _, _ = O.quantize(w, 8, O.SYM)
    qi, _, _ = inverse_form_quantize(w, 8, O.SYM)
    assert not np.array_equal(q, qi)


def test_constructed_zero_point_quotients_divide_once():
    # zero-point groups: lo = -h s with h = z0 + 1/2, hi = lo + 15 s, so that
    # s = (hi - lo) / 15 exactly and -lo / s is the half-integer h
    cases = _half_integer_cases(tuple(z0 + 0.5 for z0 in range(15)))
    rows = []
    for s, h in cases:
        lo = -F32(h) * s
        hi = F32(15) * s + lo
        if F32(hi - lo) != F32(15) * s or F32(F32(hi - lo) / F32(15)) != s:
            continue
        rows.append([lo, hi, F32(2.5) * s, -F32(1.5) * s] + [F32(0)] * 4)
        if len(rows) == 64:
            break
    assert len(rows) > 10
    w = np.array(rows, F32)
    assert_oracle_exact(w, 8, O.ASYM)
    # teeth: with the same scales, -lo times the rounded reciprocal picks the
    # other neighbour of the half-integer
    _, s, z = O.quantize(w, 8, O.ASYM)
    lo = np.minimum(w.min(axis=1), F32(0))
    zi = np.rint((-lo * (F32(1) / s[:, 0]).astype(F32)).astype(F32))
    assert not np.array_equal(z[:, 0], zi.astype(np.uint8))


def test_exact_rounding_helper_against_known_binary32_values():
    # the helper itself, against values whose binary32 encodings are fixed
    assert rn32(Fraction(1, 3)) == Fraction(11184811, 2 ** 25)        # 0x3EAAAAAB
    assert rn32(Fraction(1, 7)) == Fraction(9586981, 2 ** 26)         # 0x3E124925
    assert rn32(Fraction(1, 10)) == Fraction(13421773, 2 ** 27)       # 0x3DCCCCCD
    assert rn32(Fraction(2 ** 24 + 1)) == 2 ** 24                     # tie to even
    assert rn32(Fraction(2 ** 24 + 3)) == 2 ** 24 + 4                 # tie to even (upward)
    assert rn32(Fraction(3, 2 ** 150)) == Fraction(2, 2 ** 149)       # 1.5 x 2^-149: tie to even 2^-148
    assert rn32(Fraction(1, 2 ** 150)) == 0                           # half the smallest subnormal: to 0
    assert rn32(Fraction(-5, 2)) == Fraction(-5, 2)
    assert [rint_even(Fraction(v, 2)) for v in (-5, -3, -1, 1, 3, 5)] == [-2, -2, 0, 0, 2, 2]
    for bits in (0x3F800001, 0x00000003, 0x7F000000, 0x0080FFFF):
        v = np.array([bits], np.uint32).view(F32)[0]
        assert rn32(Fraction(float(v))) == Fraction(float(v))
