"""Oracle: blockwise 8-bit state codecs (companded and linear).

TEST INFRASTRUCTURE ONLY -- see the package docstring for who may import it.

What the pages fix:

* each optimizer state variable is quantised to 8-bit codes plus one 16-bit
  scale for every 32 consecutive elements (FlashOptim thread, Davis Blalock,
  the post on linear quantisation of state variables);
* plain linear quantisation of that form diverges, so an invertible
  companding function is applied first: a softsign-like one for momentum-like
  states and a square root for variance-like states, mapped onto the 256 bins
  of INT8 / UINT8 (same thread, posts on companding; blog "FlashOptim:
  Breaking the Memory Wall with 24-bit Weights and Companded States",
  Methodology section 2 "Companded Quantization" and "Critical Insight");
* blockwise quantisation quantises independent blocks (summary of
  "8-bit Optimizers via Block-wise Quantization", Block-wise Dynamic
  Quantization) -- prior art for the block structure.

Readings:

C1  Block = 32 consecutive elements of the flattened tensor; the last block
    holds n mod 32 elements.  The absmax ignores NaN (IEEE maxNum), so only a
    block that is NaN throughout has a NaN absmax (and a NaN scale); for a
    short last block it covers only the valid elements (zero padding is
    equivalent because every candidate is >= 0).
C2  Scale format: IEEE binary16.  Momentum: s = RU16(max |m|).  Variance:
    s = RU16(sqrt_rn(max v)) -- the scale lives in the square-root domain, so
    it never underflows where max v would.  RU16 = smallest binary16 >= the
    value; above 65504 it saturates at 65504; NaN -> NaN.
C3  Momentum compander (softsign-like): z = m * R with R = RN32(1/s) per
    block (0 when s = 0); q = sign(z) * round_half_even(127 * phi(min(|z|,1)))
    with phi(a) = 2a / (1 + a), phi(0) = 0, phi(1) = 1.  The rounding is the
    exact one of the real number 127*phi(a) for the float32 a; no ties exist
    (each threshold (2k+1)/(507-2k) has an odd denominator > 1).
    Decode: m = RN32(s * LUT[q]) with LUT[q] = RN32(q / (254 - |q|)), the
    inverse of phi at q/127.  Codes in [-127, 127].
C4  Variance compander (square root): C = RN32(255/s) per block (0 when
    s = 0); q = clamp(round_half_even(RN32(sqrt_rn(v) * C)), 0, 255).
    Decode: t = RN32(RN32(s * K255) * q) with K255 = RN32(1/255); v = RN32(t*t).
    The decoded levels are (k/255)^2 * s^2: a linear-square grid.
C5  Linear ablation (no companding), same scales as C2:
    momentum q = clamp(rint(RN32(m * RN32(127/s))), -127, 127),
             decode RN32(RN32(s * K127) * q), K127 = RN32(1/127);
    variance q = clamp(rint(RN32(v * RN32(255/(s*s)))), 0, 255),
             decode RN32(RN32(RN32(s*s) * K255) * q).
C6  Codes are clamped to range before rounding (IEEE minNum/maxNum, which
    send NaN to the upper bound): a NaN momentum element gets +127 and a NaN
    variance element 255, under either codec.
C7  The one int8 pattern outside the momentum code range, -128, is never
    written by the encoder.  Stored states may still hold it, so decode
    defines it: the companded LUT saturates it to -127 (so every code decodes
    into [-s, s]); the linear decode is the plain product for every int8.

RN32(.) is one IEEE float32 rounding; numpy float32 arithmetic provides it.
Where floating point decides a code, the decision is taken in float32 (the
kernel's precision) except the companded momentum rounding, which is the exact
rounding of 127*phi(a) (float64 evaluation is exact for that decision:
|127*phi(a) - (k+1/2)| >= 2^-35 for every float32 a near a threshold, far
above float64's error).

Parity status: pinned (invertibility, monotone decode, phi(0)=0 and
phi(+-1)=+-1, exhaustive half-step bound over float32 z in [-1, 1] sampled
densely, hand-computed golden codes, RU16 against numpy's binary16 cast,
companded-vs-linear error on heavy-tailed data; tests/test_oracle_codecs.py).
"""

from __future__ import annotations

import numpy as np

from .numerics import FORMATS, _exponent, f16_bits_to_f32

BLOCK = 32
F16 = FORMATS["fp16"]
F16_MAX = 65504.0
K127 = np.float32(1.0) / np.float32(127.0)
K255 = np.float32(1.0) / np.float32(255.0)


def ru_fp16_bits(x32: np.ndarray) -> np.ndarray:
    """Smallest binary16 >= x (x >= 0 or NaN), saturating at 65504 (C2)."""
    x = np.asarray(x32, dtype=np.float32).astype(np.float64)
    nan = np.isnan(x)
    xf = np.where(nan, 0.0, np.minimum(x, F16_MAX))
    q = np.ldexp(1.0, _exponent(xf, F16) - (F16.p - 1))   # spacing of x's binade
    a = np.ceil(xf / q) * q                                # exact: power-of-two scaling
    a = np.minimum(a, F16_MAX)
    bits = a.astype(np.float16).view(np.uint16).copy()
    bits[nan] = 0x7E00
    return bits


def _blocks(x: np.ndarray) -> np.ndarray:
    """(n,) -> (ceil(n/32), 32), zero padded (C1)."""
    x = np.asarray(x, dtype=np.float32).ravel()
    nb = -(-x.size // BLOCK)
    pad = np.zeros(nb * BLOCK, dtype=np.float32)
    pad[: x.size] = x
    return pad.reshape(nb, BLOCK)


def block_scales(x: np.ndarray, kind: str) -> np.ndarray:
    """fp16 scale bits per 32-element block for a momentum ('m') or variance ('v')
    state (C1, C2)."""
    b = _blocks(x)
    if b.shape[0] == 0:
        return np.zeros(0, dtype=np.uint16)
    if kind == "m":
        amax = np.fmax.reduce(np.abs(b), axis=1)
    elif kind == "v":
        amax = np.sqrt(np.fmax.reduce(b, axis=1))          # float32 sqrt: correctly rounded
    else:
        raise ValueError(kind)
    return ru_fp16_bits(amax.astype(np.float32))


def _per_elem(scale_bits: np.ndarray, n: int) -> np.ndarray:
    s = f16_bits_to_f32(scale_bits)
    return np.repeat(s, BLOCK)[:n]


def momentum_lut(codec: str = "companded") -> np.ndarray:
    """LUT[q + 127] = RN32(q / (254 - |q|)) for q in [-127, 127] (C3)."""
    q = np.arange(-127, 128, dtype=np.float32)
    if codec != "companded":
        raise ValueError("the momentum LUT exists for the companded codec only")
    return q / (np.float32(254.0) - np.abs(q))


def _phi_code(a64: np.ndarray) -> np.ndarray:
    """round_half_even(127 * phi(a)), phi(a) = 2a/(1+a), for 0 <= a <= 1 (C3)."""
    return np.rint(254.0 * a64 / (1.0 + a64))


def encode_momentum(m: np.ndarray, scale_bits: np.ndarray, codec: str = "companded") -> np.ndarray:
    m = np.asarray(m, dtype=np.float32).ravel()
    s = _per_elem(scale_bits, m.size)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        if codec == "companded":
            r = np.where(s > 0, np.float32(1.0) / np.where(s > 0, s, np.float32(1)), np.float32(0))
            z = (m * r).astype(np.float32)
            a = np.fmin(np.abs(z), np.float32(1.0)).astype(np.float64)   # NaN -> 1 (C6)
            q = _phi_code(a)
            q = np.where(z < 0, -q, q)
        elif codec == "linear":
            c = np.where(s > 0, np.float32(127.0) / np.where(s > 0, s, np.float32(1)), np.float32(0))
            y = (m * c).astype(np.float32)
            y = np.fmax(np.fmin(y, np.float32(127)), np.float32(-127))     # NaN -> 127 (C6)
            q = np.rint(y)
        else:
            raise ValueError(codec)
    return np.clip(q, -127, 127).astype(np.int8)


def decode_momentum(q: np.ndarray, scale_bits: np.ndarray, codec: str = "companded") -> np.ndarray:
    q = np.asarray(q, dtype=np.int8).ravel()
    s = _per_elem(scale_bits, q.size)
    if codec == "companded":
        lut = momentum_lut("companded")
        return (s * lut[np.maximum(q.astype(np.int64), -127) + 127]).astype(np.float32)   # C7
    if codec == "linear":
        step = (s * K127).astype(np.float32)
        return (step * q.astype(np.float32)).astype(np.float32)
    raise ValueError(codec)


def encode_variance(v: np.ndarray, scale_bits: np.ndarray, codec: str = "companded") -> np.ndarray:
    v = np.asarray(v, dtype=np.float32).ravel()
    s = _per_elem(scale_bits, v.size)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        if codec == "companded":
            c = np.where(s > 0, np.float32(255.0) / np.where(s > 0, s, np.float32(1)), np.float32(0))
            y = (np.sqrt(v) * c).astype(np.float32)
        elif codec == "linear":
            s2 = (s * s).astype(np.float32)
            c = np.where(s2 > 0, np.float32(255.0) / np.where(s2 > 0, s2, np.float32(1)), np.float32(0))
            y = (v * c).astype(np.float32)
        else:
            raise ValueError(codec)
        y = np.fmin(y, np.float32(255))                                    # NaN -> 255 (C6)
        q = np.clip(np.rint(y), 0, 255)
    return q.astype(np.uint8)


def decode_variance(q: np.ndarray, scale_bits: np.ndarray, codec: str = "companded") -> np.ndarray:
    q = np.asarray(q, dtype=np.uint8).ravel()
    s = _per_elem(scale_bits, q.size)
    qf = q.astype(np.float32)
    if codec == "companded":
        step = (s * K255).astype(np.float32)
        t = (step * qf).astype(np.float32)
        return (t * t).astype(np.float32)
    if codec == "linear":
        step = ((s * s).astype(np.float32) * K255).astype(np.float32)
        return (step * qf).astype(np.float32)
    raise ValueError(codec)


def quantize_state(x: np.ndarray, kind: str, codec: str = "companded"):
    """f32 state -> (codes, fp16 scale bits)."""
    s = block_scales(x, kind)
    if kind == "m":
        return encode_momentum(x, s, codec), s
    return encode_variance(x, s, codec), s


def dequantize_state(codes: np.ndarray, scale_bits: np.ndarray, kind: str, codec: str = "companded"):
    if kind == "m":
        return decode_momentum(codes, scale_bits, codec)
    return decode_variance(codes, scale_bits, codec)
