"""Exact binary32 rounding of rational numbers, for the CPU pins.

Written from the IEEE 754 definition (round to nearest, ties to even, with
the binary32 precision of 24 bits and smallest normal exponent -126; no
overflow handling: callers stay in range).  Shares nothing with the oracle.
"""

from __future__ import annotations

import math
from fractions import Fraction

import numpy as np


def exp2floor(v: Fraction) -> int:
    """floor(log2(v)) for v > 0."""
    e = v.numerator.bit_length() - v.denominator.bit_length()
    if Fraction(2) ** e > v:
        e -= 1
    elif Fraction(2) ** (e + 1) <= v:
        e += 1
    return e


def round_half_even(v: Fraction) -> int:
    f = math.floor(v)
    r = v - f
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and f % 2 == 1):
        return f + 1
    return f


def rn32(v: Fraction) -> Fraction:
    """The binary32 value nearest to v (ties to even)."""
    if v == 0:
        return Fraction(0)
    a = abs(v)
    e = max(exp2floor(a), -126)
    ulp = Fraction(2) ** (e - 23)
    r = round_half_even(a / ulp) * ulp
    return r if v > 0 else -r


def f32(v: Fraction) -> np.float32:
    """A binary32-representable rational as np.float32 (exact)."""
    return np.float32(float(v))


def rn32_sqrt(v: Fraction) -> Fraction:
    """The binary32 value nearest to sqrt(v), v >= 0, decided with exact squares."""
    if v == 0:
        return Fraction(0)
    c = Fraction(float(np.float32(math.sqrt(float(v)))))
    for _ in range(4):
        e = max(exp2floor(c), -126)
        ulp = Fraction(2) ** (e - 23)
        lo_ulp = ulp / 2 if c == Fraction(2) ** e and e > -126 else ulp
        if (c + ulp / 2) ** 2 < v:
            c += ulp
        elif (c - lo_ulp / 2) ** 2 > v:
            c -= lo_ulp
        else:
            return c
    raise AssertionError("sqrt rounding did not settle")
