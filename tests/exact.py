"""Exact rational arithmetic for pinning the oracle (test helper, CPU only).

Rounds exact ``fractions.Fraction`` values to binary floating-point formats
with round-to-nearest, ties-to-even, written from the IEEE 754 definition
(significand precision p, minimum normal exponent emin, subnormals, overflow
to infinity).  It uses no numpy float arithmetic, so it can check the
oracle's numpy float32 / float16 / bf16 steps independently.
"""

from fractions import Fraction
import math

import numpy as np

INF = float("inf")

# (precision p incl. hidden bit, emin of normals, emax)
FMT = {
    "f32": (24, -126, 127),
    "f16": (11, -14, 15),
    "bf16": (8, -126, 127),
}


def _floor_log2(a: Fraction) -> int:
    """floor(log2(a)) for a > 0, exactly."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # 2^e <= a < 2^(e+1) may be off by one
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_fmt(x, fmt: str):
    """Round the exact value x (Fraction, int or float) to format fmt; returns Fraction or +/-inf."""
    p, emin, emax = FMT[fmt]
    if isinstance(x, float):
        if math.isinf(x):
            return x
        x = Fraction(x)
    x = Fraction(x)
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = max(_floor_log2(a), emin)
    ulp = Fraction(2) ** (e - (p - 1))
    n = a / ulp
    n0 = n.numerator // n.denominator
    rem = n - n0
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n0 % 2 == 1):
        n0 += 1
    v = n0 * ulp
    max_finite = (2 - Fraction(2) ** (1 - p)) * Fraction(2) ** emax
    if v > max_finite:
        return sign * INF
    return sign * v


def frac(v) -> Fraction:
    """Exact Fraction of a finite numpy / Python float."""
    return Fraction(float(v))


def rint_clamp_0_15(t: Fraction) -> int:
    """The code for t: the nearest integer in [0, 15], ties to the even one (brute force over 16 codes)."""
    best = None
    for c in range(16):
        d = abs(Fraction(c) - t)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1]


def rint_half_even(t: Fraction) -> int:
    """The nearest integer to t, ties to the even one (no clamping)."""
    f = t.numerator // t.denominator  # floor
    rem = t - f
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and f % 2 == 1):
        return f + 1
    return f


def bf16_from_fraction_bits(v) -> int:
    """uint16 bit pattern of a bf16 value given exactly (Fraction or +/-inf)."""
    if isinstance(v, float) and math.isinf(v):
        return 0x7F80 if v > 0 else 0xFF80
    f = float(v)  # exact: bf16 values are representable in float64
    return int(np.array([f], dtype=np.float32).view(np.uint32)[0] >> 16)
