"""Exact-rational IEEE 754 rounding, written from the binary16/binary32
definitions (significand p bits, minimum normal exponent emin, largest finite
value), used to pin the oracle's floating-point steps independently of numpy.
"""
from __future__ import annotations

import math
from fractions import Fraction

# (precision p, emin, emax) of the IEEE binary formats
BINARY16 = (11, -14, 15)
BINARY32 = (24, -126, 127)


def round_to_format(v: Fraction, fmt) -> float:
    """Round an exact rational to the nearest value of ``fmt``, ties to an even
    significand; overflow (at or beyond max + half an ulp, tie to even) gives
    +-inf.  Returns a Python float (binary64 holds every binary16/32 value)."""
    p, emin, emax = fmt
    if v == 0:
        return 0.0
    sign = -1 if v < 0 else 1
    a = abs(v)
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, emin)                      # subnormals share emin's spacing
    ulp = Fraction(2) ** (e - (p - 1))
    m = a / ulp                            # scaled significand, exact
    lo = math.floor(m)
    rem = m - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    r = lo * ulp
    maxv = (2 - Fraction(2) ** (1 - p)) * Fraction(2) ** emax
    if r > maxv:
        return sign * math.inf
    return sign * float(r)


def fp16(v) -> float:
    return round_to_format(Fraction(v), BINARY16)


def fp32(v) -> float:
    return round_to_format(Fraction(v), BINARY32)


def round_half_even(t: Fraction) -> int:
    lo = math.floor(t)
    rem = t - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        return lo + 1
    return lo
