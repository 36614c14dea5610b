"""Exact rational arithmetic used to pin the oracle (no floating point inside).

These helpers round a Fraction to a binary floating-point format by the
IEEE-754 definition (nearest representable value, ties to the even
significand), so the oracle's numpy conversions can be checked against the
definition instead of against themselves.
"""
from fractions import Fraction
import math


def floor_log2(v: Fraction) -> int:
    """floor(log2(v)) for v > 0, exactly."""
    e = v.numerator.bit_length() - v.denominator.bit_length()
    # now 2^(e-1) < v < 2^(e+1); fix up to 2^e <= v < 2^(e+1)
    if Fraction(2) ** e > v:
        e -= 1
    return e


def round_half_even(v: Fraction) -> int:
    f = math.floor(v)
    r = v - f
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and f % 2 == 1):
        return f + 1
    return f


def round_to_format(v: Fraction, mant_bits: int, emin: int, emax: int) -> Fraction:
    """Round v to the format with `mant_bits` significand bits (incl. hidden bit),
    minimum normal exponent `emin` and maximum exponent `emax`; returns the
    rounded value, or +-inf (as a float) on overflow."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = max(floor_log2(a), emin)
    quantum = Fraction(2) ** (e - (mant_bits - 1))
    m = round_half_even(a / quantum)
    r = m * quantum
    largest = (Fraction(2) - Fraction(2) ** (1 - mant_bits)) * Fraction(2) ** emax
    if r > largest:
        return sign * math.inf
    return sign * r


def fp16_exact(v: Fraction):
    return round_to_format(v, 11, -14, 15)


def fp32_exact(v: Fraction):
    return round_to_format(v, 24, -126, 127)


def all_finite_fp16():
    """Every finite float16 value (as Python floats), both signs, one zero."""
    import numpy as np
    bits = np.arange(0, 0x7C00, dtype=np.uint16)          # +0 .. largest finite
    pos = bits.view(np.float16)
    return np.concatenate([-pos[:0:-1], pos])
