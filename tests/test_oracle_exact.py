"""Exact-rational pin of the oracle's weight split (CPU only).

The split is written out again from its definition with Python's Fraction:
theta' = |x| rounded to the nearest value of the 16-bit format, ties away
from zero (the format's spacing below its smallest normal is fixed); the ECC
is the exact offset (|x| - |theta'|) measured in units of 2^-N of the spacing
on the side of theta' that x lies on (below a power of two above the
smallest normal that spacing is halved), rounded half to even and clamped to
the N-bit range.  Thousands of random f32 values (all magnitudes, fp16
subnormals, values within a few f32 spacings of every kind of tie) must give
the oracle's theta' pattern and rho exactly.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle as O

# (precision bits incl. the implicit one, exponent of the smallest normal,
#  exponent bits' bias, largest finite value)
FMT = {"bf16": (8, -126, 127, Fraction(2 ** 127) * (2 - Fraction(1, 2 ** 7))),
       "fp16": (11, -14, 15, Fraction(65504))}


def _exp2floor(v: Fraction) -> int:
    e = v.numerator.bit_length() - v.denominator.bit_length()
    if Fraction(2) ** e > v:
        e -= 1
    elif Fraction(2) ** (e + 1) <= v:
        e += 1
    return e


def _spacing(a: Fraction, p: int, emin: int) -> Fraction:
    """Spacing above |a| in the format (a >= 0, finite)."""
    e = max(_exp2floor(a), emin) if a > 0 else emin
    return Fraction(2) ** (e - p + 1)


def _rna(v: Fraction, p: int, emin: int) -> Fraction:
    s = _spacing(v, p, emin)
    k = v / s
    q = k.numerator // k.denominator
    if k - q >= Fraction(1, 2):
        q += 1
    a = q * s
    return a


def _encode(a: Fraction, fmt: str) -> int:
    """Bit pattern of a non-negative representable value."""
    p, emin, bias, _ = FMT[fmt]
    if a == 0:
        return 0
    e = _exp2floor(a)
    mant_bits = p - 1
    if e < emin:                                   # subnormal
        m = a / Fraction(2) ** (emin - mant_bits)
        assert m.denominator == 1
        return int(m)
    m = a / Fraction(2) ** (e - mant_bits) - 2 ** mant_bits
    assert m.denominator == 1
    return ((e + bias) << mant_bits) | int(m)


def exact_split(x: float, fmt: str, n: int):
    p, emin, bias, amax = FMT[fmt]
    v = Fraction(abs(float(x)))
    sign = 0x8000 if np.signbit(np.float32(x)) else 0
    a = _rna(v, p, emin)
    if a > amax:                                   # saturate, the offset clamps at its top
        return sign | _encode(amax, fmt), 2 ** (n - 1) - 1
    d = v - a
    up = _spacing(a, p, emin)
    if d >= 0:
        ulp = up
    else:
        # spacing below a: half the spacing above when a is a power of two
        # above the smallest normal, the same otherwise
        ulp = up / 2 if (a > Fraction(2) ** emin and a == Fraction(2) ** _exp2floor(a)) else up
    delta = d * 2 ** n / ulp
    q = delta.numerator // delta.denominator       # floor
    r = delta - q
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and q % 2 == 1):
        q += 1
    q = max(-(2 ** (n - 1)), min(2 ** (n - 1) - 1, q))
    return sign | _encode(a, fmt), q


def _samples(fmt, rng):
    p, emin, _, amax = FMT[fmt]
    xs = [rng.standard_normal(600) * 0.02,
          (rng.standard_normal(300) * 10.0 ** rng.uniform(-12, 4, 300)),
          rng.uniform(-2.0 ** emin, 2.0 ** emin, 300)]
    # values near ties: midpoints between neighbouring 16-bit values, +- a few f32 spacings
    k = rng.integers(1, 2 ** 14, 200)
    e = rng.integers(emin, emin + 20, 200)
    mids = (2.0 * k + 1) * 2.0 ** (e.astype(float) - p) * np.where(rng.random(200) < 0.5, 1, -1)
    m32 = mids.astype(np.float32).view(np.uint32).astype(np.int64)
    near = (m32[:, None] + np.arange(-2, 3)[None, :]).ravel().astype(np.uint32).view(np.float32)
    xs.append(near.astype(np.float64))
    # just below powers of two above the smallest normal (the halved inner spacing)
    pe = rng.integers(emin + 1, emin + 40, 100)
    p32 = (2.0 ** pe.astype(float)).astype(np.float32).view(np.uint32).astype(np.int64)
    steps = rng.integers(1, 2 ** (24 - p) + 4, 100)
    below = (p32 - steps).astype(np.uint32).view(np.float32).astype(np.float64)
    xs.append(below * np.where(rng.random(100) < 0.5, 1, -1))
    x = np.concatenate(xs).astype(np.float32)
    return x[np.isfinite(x) & (np.abs(x.astype(np.float64)) < float(amax) * 1.01)]


@pytest.mark.parametrize("fmt,n", [("bf16", 8), ("bf16", 16), ("fp16", 8)])
def test_split_equals_exact_rational_definition(fmt, n):
    rng = np.random.default_rng({"bf16": 11, "fp16": 12}[fmt] + n)
    x = _samples(fmt, rng)
    w, r = O.split_weights(x, fmt, n)
    bad = []
    for i, xi in enumerate(x):
        we, re_ = exact_split(float(xi), fmt, n)
        if int(w[i]) != we or int(r[i]) != re_:
            bad.append((hex(int(np.float32(xi).view(np.uint32))), int(w[i]), we, int(r[i]), re_))
    assert not bad, f"{len(bad)} of {x.size} differ, e.g. {bad[:4]}"
    assert x.size > 2000
