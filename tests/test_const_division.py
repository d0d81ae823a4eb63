"""The constant-divisor quotient used for group scales (div_const in
int4_group_wise_amd/csrc/w4_device.h): q0 = fp32(x * r) with r = fp32(1 / D),
then q = fp32(q0 + fp32(x - q0 * D) * r) with both steps fused multiply-adds.
For D = 7 and D = 15 it must equal the correctly rounded fp32(x / D) for every
finite x >= 0; the scales amax / 7 and (hi - lo) / 15 of the quantizers
depend on it for bit-exact codes.

The fused steps are emulated in fp64: x * r and q0 * D are exact there (24 x 24
and 24 x 4 significant bits), so x - q0 * D is exact and rounds once to fp32
like the device fma; e * r is exact and q0 + e * r is rounded to 53 bits before
fp32, a double rounding that cannot change the result here: the significand
of x / D is a multiple of 1 / D away from an integer, so it stays at least
1 / (2 D) of a unit in the last place (about 2^-28 to 2^-29 relative) from
every fp32 rounding midpoint, far beyond the ~2^-47 by which q0 + e * r
differs from x / D (the residual x - q0 * D is exact in fp32).  By default
four full binades, the whole subnormal range and the top binade are checked
(a few seconds); W4_EXHAUSTIVE=1 checks all 2^31 - 2^23 finite non-negative
values (about a minute per divisor).
"""
import os

import numpy as np
import pytest

EXHAUSTIVE = os.environ.get("W4_EXHAUSTIVE") == "1"


def _emulated(x64, d):
    r32 = np.float32(1.0) / np.float32(d)                  # fp32(1 / D), correctly rounded
    r = np.float64(r32)
    q0 = (x64 * r).astype(np.float32).astype(np.float64)
    e = (x64 - q0 * d).astype(np.float32).astype(np.float64)
    return (q0 + e * r).astype(np.float32)


def _ranges():
    one = int(np.float32(1.0).view(np.uint32))
    if EXHAUSTIVE:
        return [(0, 0x7F800000)]
    return [
        (0, 0x00800000),                                   # zero and all subnormals
        (one, one + 4 * 0x00800000),                       # [1, 16): scales of unit-sized weights
        (0x7F000000, 0x7F800000),                          # the top binade, up to the largest finite
    ]


@pytest.mark.parametrize("d", [7, 15])
def test_constant_division_is_correctly_rounded(d):
    chunk = 1 << 24
    for lo, hi in _ranges():
        for start in range(lo, hi, chunk):
            u = np.arange(start, min(start + chunk, hi), dtype=np.uint32)
            x = u.view(np.float32)
            got = _emulated(x.astype(np.float64), d)
            want = x / np.float32(d)                       # IEEE fp32 division
            bad = np.flatnonzero(got.view(np.uint32) != want.view(np.uint32))
            assert bad.size == 0, f"D={d}: x={float(x[bad[0]]).hex()} gives {float(got[bad[0]]).hex()}, " \
                                  f"not {float(want[bad[0]]).hex()}"


def test_reciprocal_constants():
    """fp32(1 / 7) and fp32(1 / 15) as the kernel's constant expressions give them."""
    assert float(np.float32(1.0) / np.float32(7)).hex() == "0x1.24924a0000000p-3"
    assert float(np.float32(1.0) / np.float32(15)).hex() == "0x1.1111120000000p-4"
