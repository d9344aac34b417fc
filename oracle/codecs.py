"""Oracle: blockwise state codecs (8-bit companded and linear, 4-bit companded,
8-bit companded with bfloat16 block scales).

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
    holds n mod 32 elements and only those count.  The absmax ignores NaN
    (IEEE maxNum), so a block whose valid elements are all NaN -- a short last
    block included -- has a NaN absmax and a NaN scale.  (Padding the short
    block with NaN, which maxNum skips, gives exactly that.)
C2  Scale format: IEEE binary16.  Momentum: s = RU16(max |m|).  Variance:
    s = RU16(sqrt_rn(max v)) -- the scale lives in the square-root domain, so
    it never underflows where max v would.  RU16 = smallest binary16 >= the
    value; above 65504 it saturates at 65504; NaN -> NaN.
C3  Momentum compander (softsign-like).  Normalise, then compand: z = m / s,
    one IEEE float32 division; q = sign(z) * round_half_even(127 * phi(a)),
    a = min(|z|, 1), phi(a) = 2a / (1 + a), phi(0) = 0, phi(1) = 1.  The
    rounding is the exact one of the real number 127*phi(a) for the float32
    a; no ties exist (each threshold (2k+1)/(507-2k) has an odd denominator
    > 1).  Decode: m = RN32(s * LUT[q]), LUT[q] = RN32(q / (254 - |q|)), the
    inverse of phi at q/127.  Codes in [-127, 127].
C4  Variance compander (square root).  Compand, normalise, scale to the code
    range, each step one float32 operation: w = sqrt_rn(v), z = w / s,
    y = 255 * z, q = clamp(round_half_even(y), 0, 255).  Decode with the
    block's level spacing D = RN32(s / 255): t = RN32(D * q), v = RN32(t * t).
    The decoded levels are (k * s/255)^2: a linear-square grid.
C5  Linear ablation (no companding), same scales as C2.  Momentum:
    z = m / s, y = 127 * z, q = clamp(round_half_even(y), -127, 127); decode
    m = RN32(D * q), D = RN32(s / 127).  Variance: s2 = s * s (exact),
    z = v / s2, y = 255 * z, q = clamp(round_half_even(y), 0, 255); decode
    v = RN32(D * q), D = RN32(s2 / 255).
C6  A NaN element has no nearest level: it gets code 0, and values beyond the
    code range (+-Inf, or finite values past a saturated scale) clamp to the
    end codes.  That is the rule of a saturating float-to-integer conversion
    (Java's and Rust's casts, WebAssembly's trunc_sat: out-of-range values
    clamp, NaN gives 0).  A NaN element therefore decodes to 0 on the next
    step, the value of a fresh state; the NaN survives in the state only when
    it fills its block (C1), whose NaN scale decodes every code to NaN.  An
    all-zero block has s = 0, and 0/0 = NaN codes its elements 0 as well.
C7  The one int8 pattern outside the momentum code range, -128, is never
    written by the encoder.  Stored states may still hold it, so decode
    defines it: the companded LUT saturates it to -127 (so every code decodes
    into [-s, s]); the linear decode is the plain product for every int8.

C8  4-bit states.  The pages name lower-bit states only as an outlook (blog,
    Conclusion & Perspective, Future Outlook: 4-bit states might work given
    a more aggressive transform) and define no transform, so the plainest
    reading keeps everything of C1-C7 and narrows the codes: codec
    "companded4".  Momentum: q = sign(z) * round_half_even(7 * phi(a)), codes
    in [-7, 7] (no ties: the thresholds (2k+1)/(27-2k) have odd denominators
    > 1); decode m = RN32(s * LUT4[q]), LUT4[q] = RN32(q / (14 - |q|)), the
    inverse of phi at q/7; the pattern -8 is never written and decodes as -7.
    Variance: w = sqrt_rn(v), z = w / s, y = RN32(15 * z),
    q = clamp(round_half_even(y), 0, 15); decode D = RN32(s / 15),
    t = RN32(D * q), v = RN32(t * t).  Storage: two codes per byte, element
    2i in the low nibble and 2i+1 in the high one, momentum codes as 4-bit
    two's complement; an odd-length tensor's last byte has a zero high
    nibble.  Only the companded codec has a 4-bit form (the pages report
    that plain linear codes diverge already at 8 bits).
C9  bfloat16 block scales (codec "companded_bf16scale").  The pages fix a
    16-bit scale per 32 elements and name no format; C2 reads binary16.  The
    other 16-bit format the method already uses for weights is bfloat16,
    which keeps float32's exponent range at 8 significand bits.  The variant
    keeps everything of C1-C7 and changes only the scale:
    s = RUbf16(max |m|) or RUbf16(sqrt_rn(max v)), RUbf16 = smallest
    bfloat16 >= the value (subnormal bfloat16 values included), saturating
    at the largest finite bfloat16 (0x7F7F); NaN -> 0x7FC0.  Blocks far below
    binary16's smallest subnormal keep nonzero codes, and a block's codes do
    not change when its values are scaled by a power of two (four for v)
    anywhere in the normal range.

RN32(.) is one IEEE float32 rounding; numpy float32 arithmetic provides it
(its division and square root are the correctly rounded IEEE operations).
Every quotient above is such a division: there is no reciprocal-multiply
anywhere.  Where floating point decides a code, the decision is taken on
float32 values; the companded momentum rounding alone is evaluated exactly
for its float32 argument (float64 is exact for that decision:
|127*phi(a) - (k+1/2)| >= 2^-35 for every float32 a near a threshold, far
above float64's error).

Parity status: pinned (C9: RUbf16 against a search of the sorted table of
every bfloat16 value, codes equal to the binary16-scale codec wherever the
two scales coincide, power-of-two scale invariance, tiny blocks;
tests/test_oracle_bf16scale.py; the rest for both code widths: invertibility, monotone decode, phi(0)=0 and
phi(+-1)=+-1, exhaustive half-step bound over float32 z in [-1, 1] sampled
densely, hand-computed golden codes, exact-rational codes for inputs where a
reciprocal-multiply would differ from the division, RU16 against numpy's
binary16 cast, companded-vs-linear error on heavy-tailed data, NaN and
infinity codes, NaN-filled short last blocks, hand-packed nibble bytes;
tests/test_oracle_codecs.py).
"""

from __future__ import annotations

import numpy as np

from .numerics import FORMATS, _exponent, bf16_bits_to_f32, f16_bits_to_f32

BLOCK = 32
F16 = FORMATS["fp16"]
F16_MAX = 65504.0
BF16 = FORMATS["bf16"]
F32 = np.float32

# codecs whose codes come from the companders (C3, C4, C8, C9)
COMPANDED_CODECS = ("companded", "companded4", "companded_bf16scale")
# the format of each codec's block scales (C2, C9)
SCALE_FORMAT = {"companded": "fp16", "linear": "fp16", "companded4": "fp16", "companded_bf16scale": "bf16"}


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


def ru_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Smallest bfloat16 >= x (x >= 0 or NaN), saturating at the largest finite
    bfloat16; NaN -> 0x7FC0 (C9)."""
    x = np.asarray(x32, dtype=np.float32).astype(np.float64)
    nan = np.isnan(x)
    xf = np.where(nan, 0.0, np.minimum(x, BF16.max_finite))
    q = np.ldexp(1.0, _exponent(xf, BF16) - (BF16.p - 1))  # spacing of x's binade (subnormals: 2^-133)
    a = np.ceil(xf / q) * q                                 # exact: power-of-two scaling
    a = np.minimum(a, BF16.max_finite)
    bits = (a.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)   # a is a bfloat16 value
    bits[nan] = 0x7FC0
    return bits


def scale_to_f32(scale_bits: np.ndarray, codec: str = "companded") -> np.ndarray:
    """Stored block-scale patterns -> float32 (exact), in the codec's scale
    format (C2, C9)."""
    if SCALE_FORMAT[codec] == "bf16":
        return bf16_bits_to_f32(scale_bits)
    return f16_bits_to_f32(scale_bits)


def _blocks(x: np.ndarray) -> np.ndarray:
    """(n,) -> (ceil(n/32), 32); the short last block is padded with NaN, which
    the maxNum reductions skip, so only its valid elements count (C1)."""
    x = np.asarray(x, dtype=np.float32).ravel()
    nb = -(-x.size // BLOCK)
    pad = np.full(nb * BLOCK, np.nan, dtype=np.float32)
    pad[: x.size] = x
    return pad.reshape(nb, BLOCK)


def block_scales(x: np.ndarray, kind: str, codec: str = "companded") -> np.ndarray:
    """Scale bits per 32-element block for a momentum ('m') or variance ('v')
    state (C1, C2; binary16, or bfloat16 under C9)."""
    b = _blocks(x)
    if b.shape[0] == 0:
        return np.zeros(0, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        if kind == "m":
            amax = np.fmax.reduce(np.abs(b), axis=1)
        elif kind == "v":
            amax = np.sqrt(np.fmax.reduce(b, axis=1))      # float32 sqrt: correctly rounded
        else:
            raise ValueError(kind)
    ru = ru_bf16_bits if SCALE_FORMAT[codec] == "bf16" else ru_fp16_bits
    return ru(amax.astype(np.float32))


def _per_elem(scale_bits: np.ndarray, n: int, codec: str) -> np.ndarray:
    s = scale_to_f32(scale_bits, codec)
    return np.repeat(s, BLOCK)[:n]


# largest momentum code L and largest variance code of each codec (C3-C5, C8, C9)
CODE_MAX = {"companded": (127, 255), "linear": (127, 255), "companded4": (7, 15),
            "companded_bf16scale": (127, 255)}


def code_bytes(n: int, codec: str) -> int:
    """Bytes of one state's code array for n elements (C8: two 4-bit codes a byte)."""
    return (n + 1) // 2 if codec == "companded4" else n


def momentum_lut(codec: str = "companded") -> np.ndarray:
    """LUT[q + L] = RN32(q / (2L - |q|)) for q in [-L, L], the inverse of phi
    at q/L: L = 127 (C3, C9) or 7 (C8)."""
    if codec not in COMPANDED_CODECS:
        raise ValueError("the momentum LUT exists for the companded codecs only")
    L = CODE_MAX[codec][0]
    q = np.arange(-L, L + 1, dtype=np.float32)
    return q / (F32(2 * L) - np.abs(q))


def pack_nibbles(q: np.ndarray) -> np.ndarray:
    """Codes in [-8, 15] -> bytes, element 2i in the low nibble, 2i+1 in the
    high one (4-bit two's complement for negative codes); an odd count leaves
    the last high nibble 0 (C8)."""
    q = np.asarray(q).astype(np.int64).ravel()
    if q.size % 2:
        q = np.concatenate([q, np.zeros(1, np.int64)])
    nib = q & 0xF
    return (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8)


def unpack_nibbles(b: np.ndarray, n: int, signed: bool) -> np.ndarray:
    """The first n codes of a nibble-packed array (C8): int8 in [-8, 7] when
    signed, else uint8 in [0, 15]."""
    b = np.asarray(b, dtype=np.uint8).ravel().astype(np.int64)
    nib = np.empty(2 * b.size, np.int64)
    nib[0::2] = b & 0xF
    nib[1::2] = b >> 4
    nib = nib[:n]
    if signed:
        return np.where(nib >= 8, nib - 16, nib).astype(np.int8)
    return nib.astype(np.uint8)


def level_spacing(scale_bits: np.ndarray, kind: str, codec: str) -> np.ndarray:
    """The block's level spacing D of the decodes in C4/C5/C8 (float32 per
    block): RN32(s/255) (variance, companded), RN32(s/15) (variance,
    companded4), RN32(s/127) (momentum, linear), RN32(RN32(s*s)/255)
    (variance, linear)."""
    s = scale_to_f32(scale_bits, codec)
    with np.errstate(all="ignore"):
        if kind == "v" and codec in COMPANDED_CODECS:
            return (s / F32(CODE_MAX[codec][1])).astype(F32)
        if kind == "m" and codec == "linear":
            return (s / F32(127.0)).astype(F32)
        if kind == "v" and codec == "linear":
            return ((s * s).astype(F32) / F32(255.0)).astype(F32)
    raise ValueError((kind, codec))


def _phi_code(a64: np.ndarray, L: int = 127) -> np.ndarray:
    """round_half_even(L * phi(a)), phi(a) = 2a/(1+a), for 0 <= a <= 1 (C3, C8).
    float64 decides exactly: a float32 a lies at least 2^-35 (L = 127) or
    2^-31 (L = 7) from every threshold in units of L*phi, far above float64's
    error."""
    return np.rint(2.0 * L * a64 / (1.0 + a64))


def _saturating_code(y: np.ndarray, lo: int, hi: int) -> np.ndarray:
    """round_half_even(y) clamped to [lo, hi]; NaN -> 0 (C6)."""
    nan = np.isnan(y)
    q = np.clip(np.rint(np.where(nan, F32(0), y)), lo, hi)
    return np.where(nan, 0, q)


def encode_momentum(m: np.ndarray, scale_bits: np.ndarray, codec: str = "companded") -> np.ndarray:
    m = np.asarray(m, dtype=np.float32).ravel()
    s = _per_elem(scale_bits, m.size, codec)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        z = (m / s).astype(F32)                                   # one float32 division (C3, C5)
        if codec in COMPANDED_CODECS:
            nan = np.isnan(z)
            a = np.fmin(np.abs(np.where(nan, F32(0), z)), F32(1.0)).astype(np.float64)
            q = _phi_code(a, CODE_MAX[codec][0])
            q = np.where(z < 0, -q, q)
            q = np.where(nan, 0, q)                               # C6
        elif codec == "linear":
            q = _saturating_code((F32(127.0) * z).astype(F32), -127, 127)
        else:
            raise ValueError(codec)
    return q.astype(np.int8)


def decode_momentum(q: np.ndarray, scale_bits: np.ndarray, codec: str = "companded") -> np.ndarray:
    q = np.asarray(q, dtype=np.int8).ravel()
    if codec in COMPANDED_CODECS:
        L = CODE_MAX[codec][0]
        s = _per_elem(scale_bits, q.size, codec)
        lut = momentum_lut(codec)
        return (s * lut[np.maximum(q.astype(np.int64), -L) + L]).astype(F32)   # C7, C8
    if codec == "linear":
        d = np.repeat(level_spacing(scale_bits, "m", "linear"), BLOCK)[: q.size]
        return (d * q.astype(F32)).astype(F32)
    raise ValueError(codec)


def encode_variance(v: np.ndarray, scale_bits: np.ndarray, codec: str = "companded") -> np.ndarray:
    v = np.asarray(v, dtype=np.float32).ravel()
    s = _per_elem(scale_bits, v.size, codec)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        if codec in COMPANDED_CODECS:
            w = np.sqrt(v).astype(F32)                            # correctly rounded (C4, C8)
            z = (w / s).astype(F32)
        elif codec == "linear":
            s2 = (s * s).astype(F32)                              # exact: 11-bit significands
            z = (v / s2).astype(F32)
        else:
            raise ValueError(codec)
        top = CODE_MAX[codec][1]
        y = (F32(top) * z).astype(F32)
        q = _saturating_code(y, 0, top)
    return q.astype(np.uint8)


def decode_variance(q: np.ndarray, scale_bits: np.ndarray, codec: str = "companded") -> np.ndarray:
    q = np.asarray(q, dtype=np.uint8).ravel()
    d = np.repeat(level_spacing(scale_bits, "v", codec), BLOCK)[: q.size]
    qf = q.astype(F32)
    if codec in COMPANDED_CODECS:
        t = (d * qf).astype(F32)
        return (t * t).astype(F32)
    if codec == "linear":
        return (d * qf).astype(F32)
    raise ValueError(codec)


def quantize_state(x: np.ndarray, kind: str, codec: str = "companded"):
    """f32 state -> (codes, scale bits); one code per element (4-bit codes
    unpacked: pack_nibbles gives their stored bytes)."""
    s = block_scales(x, kind, codec)
    if kind == "m":
        return encode_momentum(x, s, codec), s
    return encode_variance(x, s, codec), s


def dequantize_state(codes: np.ndarray, scale_bits: np.ndarray, kind: str, codec: str = "companded"):
    if kind == "m":
        return decode_momentum(codes, scale_bits, codec)
    return decode_variance(codes, scale_bits, codec)
