"""Oracle: 16-bit downcast weight + N-bit ULP-normalised ECC (split / reconstruct).

TEST INFRASTRUCTURE ONLY -- see the package docstring for who may import it.

What the pages fix (FlashOptim thread by Davis Blalock, the posts on weight
splitting and on what the ECC bits hold; blog "FlashOptim: Breaking the
Memory Wall with 24-bit Weights and Companded States", Methodology section 1
"ULP-based Weight Splitting"):

* an f32 master weight x32 is stored as a B-bit downcast theta' (the model
  parameter itself) plus an N-bit error-correction code rho;
* all f32 values that downcast to one theta' form a fixed interval
  [val_min, val_max] whose width is bounded by the ULP of theta';
* rho is the position of x32 inside that interval, normalised by the ULP and
  quantised to an N-bit integer; N = 8 with B = 16 gives "24-bit" master
  weights, N = 32 - B is meant to be lossless.

Readings taken where the pages are silent:

R1  The downcast rounds to nearest with ties AWAY from zero (RNA).  Under RNA
    every finite theta' owns exactly 2^(24-p) f32 values on each side
    combined, which is what makes a 16-bit ECC lossless for bf16.
R2  rho is the signed, side-aware, ULP-normalised error in magnitude
    orientation:  a = |theta'|,  ulp_out(a) = spacing just above a,
    ulp_in(a) = spacing just below a (half of ulp_out only when a is a power of
    two above the smallest normal), delta = (|x32| - a) * 2^N / ulp_side,
    rho = clamp(round_half_even(delta), -2^(N-1), 2^(N-1) - 1).
    Reconstruction: |x| = a + rho * ulp_side * 2^-N with the sign of theta'.
R3  Edges: NaN -> quiet NaN (sign kept, payload = quiet bit only), rho = 0;
    +-Inf -> +-Inf, rho = 0; a finite x32 whose RNA result overflows the
    16-bit format saturates to +-max with rho clamped (documented non-exact).
    +-0 keeps its sign.  Zero and 16-bit subnormals use the subnormal spacing.
R4  Supported (format, N): (bf16, 8), (bf16, 16), (fp16, 8).

Everything here is evaluated on float64 VALUES (spacings from frexp, floors,
power-of-two scalings), all of which are exact for these magnitudes; the HIP
path works on IEEE bit patterns instead.

Parity status: pinned (exhaustive theta' sweeps with sampled preimages,
closed-form golden cases, an independent integer RNA for bf16, identity of
bf16+16 over a strided sweep of all f32 patterns; see tests/test_oracle_split.py).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Fmt:
    name: str
    p: int      # significand precision in bits, implicit bit included
    emin: int   # exponent of the smallest normal
    emax: int   # exponent of the largest finite binade

    @property
    def max_finite(self) -> float:
        return (2.0 - 2.0 ** (1 - self.p)) * 2.0 ** self.emax

    @property
    def min_normal(self) -> float:
        return 2.0 ** self.emin


FORMATS = {
    "bf16": Fmt("bf16", p=8, emin=-126, emax=127),
    "fp16": Fmt("fp16", p=11, emin=-14, emax=15),
}

SUPPORTED = {("bf16", 8), ("bf16", 16), ("fp16", 8)}


def _fmt(fmt) -> Fmt:
    return FORMATS[fmt] if isinstance(fmt, str) else fmt


def _check(fmt: Fmt, ecc_bits: int) -> None:
    if (fmt.name, ecc_bits) not in SUPPORTED:
        raise ValueError(f"unsupported format/ECC combination {fmt.name}+{ecc_bits}")


def _exponent(a: np.ndarray, fmt: Fmt) -> np.ndarray:
    """floor(log2(a)) for a > 0, clamped below at the format's emin (so zero and
    subnormals get the subnormal binade)."""
    safe = np.where(a > 0, a, 1.0)
    _, e = np.frexp(safe)          # safe = m * 2^e with m in [0.5, 1)
    e = e.astype(np.int64) - 1
    e = np.where(a > 0, e, fmt.emin)
    return np.maximum(e, fmt.emin)


def spacing_out(a: np.ndarray, fmt) -> np.ndarray:
    """Distance from a (>= 0, representable) to the next larger value of the format."""
    fmt = _fmt(fmt)
    return np.ldexp(1.0, _exponent(a, fmt) - (fmt.p - 1))


def spacing_in(a: np.ndarray, fmt) -> np.ndarray:
    """Distance from a (> 0, representable) to the next smaller value of the format.
    Equal to spacing_out except at a power of two above the smallest normal,
    where the binade below is twice as fine."""
    fmt = _fmt(fmt)
    out = spacing_out(a, fmt)
    m, _ = np.frexp(np.where(a > 0, a, 1.0))
    pow2_above_min = (m == 0.5) & (a > fmt.min_normal)
    return np.where(pow2_above_min, out / 2.0, out)


def rna_downcast(x32: np.ndarray, fmt) -> tuple[np.ndarray, np.ndarray]:
    """Round |x32| to the nearest value of `fmt`, ties away from zero (R1).

    Returns (a, overflow): a = the rounded magnitude as float64 (saturated at the
    format's max for finite inputs that overflow, R3), overflow = where that
    happened.  Non-finite inputs return their own magnitude (inf or nan).
    """
    fmt = _fmt(fmt)
    with np.errstate(invalid="ignore"):
        ax = np.abs(np.asarray(x32, dtype=np.float32).astype(np.float64))
    finite = np.isfinite(ax)
    axf = np.where(finite, ax, 0.0)
    q = spacing_out_from_value(axf, fmt)
    k = axf / q                              # exact: division by a power of two
    kf = np.floor(k)
    a = (kf + (k - kf >= 0.5)) * q           # ties go up in magnitude
    overflow = finite & (a > fmt.max_finite)
    a = np.where(overflow, fmt.max_finite, a)
    a = np.where(finite, a, ax)
    return a, overflow


def spacing_out_from_value(ax: np.ndarray, fmt: Fmt) -> np.ndarray:
    """Spacing of the format in the binade that contains the (not necessarily
    representable) magnitude ax."""
    return np.ldexp(1.0, _exponent(ax, fmt) - (fmt.p - 1))


def _encode_bits(a: np.ndarray, neg: np.ndarray, fmt: Fmt, nan: np.ndarray) -> np.ndarray:
    """Bit pattern of the 16-bit value with magnitude a (exactly representable,
    inf allowed) and sign `neg`; NaN -> quiet NaN with the sign kept."""
    a = np.where(nan, 0.0, a)
    if fmt.name == "bf16":
        f = a.astype(np.float32)
        assert np.array_equal(f.astype(np.float64), a), "bf16 magnitude not exact in f32"
        u = f.view(np.uint32)
        assert not np.any(u & 0xFFFF), "value not representable in bf16"
        bits = (u >> 16).astype(np.uint16)
        qnan = np.uint16(0x7FC0)
        sign = np.uint16(0x8000)
    else:
        with np.errstate(over="ignore"):
            h = a.astype(np.float16)
        assert np.array_equal(h.astype(np.float64), a), "value not representable in fp16"
        bits = h.view(np.uint16).copy()
        qnan = np.uint16(0x7E00)
        sign = np.uint16(0x8000)
    bits = np.where(nan, qnan, bits).astype(np.uint16)
    return np.where(neg, bits | sign, bits).astype(np.uint16)


def bits_to_value(bits: np.ndarray, fmt) -> np.ndarray:
    """16-bit pattern -> its exact value as float64 (sign included)."""
    fmt = _fmt(fmt)
    bits = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        if fmt.name == "bf16":
            return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        return bits.view(np.float16).astype(np.float64)


def split_weights(x32: np.ndarray, fmt="bf16", ecc_bits: int = 8):
    """f32 master weight -> (theta' bits uint16, rho int8/int16)  (R1-R4)."""
    fmt = _fmt(fmt)
    _check(fmt, ecc_bits)
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    neg = np.signbit(x32)
    nan = np.isnan(x32)
    with np.errstate(invalid="ignore"):
        ax = np.abs(x32.astype(np.float64))
    finite = np.isfinite(ax)
    with np.errstate(invalid="ignore"):
        a, _ = rna_downcast(x32, fmt)
        af = np.where(finite, a, 0.0)
        axf = np.where(finite, ax, 0.0)
        above = axf >= af
        ulp = np.where(above, spacing_out(af, fmt), spacing_in(af, fmt))
        delta = (axf - af) * 2.0 ** ecc_bits / ulp     # exact: Sterbenz + powers of two
        lo, hi = -(2 ** (ecc_bits - 1)), 2 ** (ecc_bits - 1) - 1
        rho = np.clip(np.rint(delta), lo, hi)          # np.rint rounds half to even
        rho = np.where(finite, rho, 0.0)
    w16 = _encode_bits(a, neg, fmt, nan)
    rho = rho.astype(np.int8 if ecc_bits == 8 else np.int16)
    return w16, rho


def reconstruct_weights(w16: np.ndarray, rho: np.ndarray, fmt="bf16", ecc_bits: int = 8) -> np.ndarray:
    """(theta' bits, rho) -> f32 master weight (R2).  Non-finite theta' is returned
    as is.  Defined on what split_weights produces (in particular rho >= 0 when
    theta' is +-0)."""
    fmt = _fmt(fmt)
    _check(fmt, ecc_bits)
    val = bits_to_value(w16, fmt)
    a = np.abs(val)
    finite = np.isfinite(a)
    af = np.where(finite, a, 0.0)
    r = np.asarray(rho).astype(np.float64)
    ulp = np.where(r >= 0, spacing_out(af, fmt), spacing_in(af, fmt))
    mag = af + r * ulp * 2.0 ** (-ecc_bits)            # exact in float64
    signed = np.where(np.signbit(val), -mag, mag)
    out = np.where(finite, signed, val)
    f = out.astype(np.float32)
    ok = np.isnan(out) | (f.astype(np.float64) == out)
    assert np.all(ok), "reconstruction not exactly representable in f32"
    return f


def f16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """IEEE binary16 pattern -> float32 (exact widening)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 pattern -> float32 (exact widening)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_f16_bits_exact(x: np.ndarray) -> np.ndarray:
    """float32 values that are exactly representable in binary16 -> their pattern."""
    x = np.asarray(x, dtype=np.float32)
    h = x.astype(np.float16)
    assert np.array_equal(h.astype(np.float32)[~np.isnan(x)], x[~np.isnan(x)])
    return h.view(np.uint16)
