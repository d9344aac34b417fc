"""Pins for the oracle's blockwise state codecs (CPU only).

Anchors: hand-derived golden codes, exact rational arithmetic near every code
threshold and for the normalising divisions (on inputs where multiplying by a
rounded reciprocal would give another code), numpy's binary16 cast for the
round-up scale, invertibility and monotonicity of the companders, the
half-step bound, the NaN / infinity codes, NaN-filled short last blocks, and
the pages' claim that companding cuts quantisation error on heavy-tailed
states.
"""

import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
from oracle.codecs import momentum_lut

from exact_fp import f32, rn32, rn32_sqrt, round_half_even

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "codec_cases.txt")


def _golden():
    rows = []
    with open(GOLDEN) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            head, vals, codes = [p.strip() for p in line.split("|")]
            kind, codec, scale = head.split()
            rows.append((kind, codec, int(scale, 16),
                         [float(v) for v in vals.split()], [int(c) for c in codes.split()]))
    return rows


@pytest.mark.parametrize("row", _golden(), ids=lambda r: f"{r[0]}-{r[1]}-{r[2]:04x}")
def test_golden_codes(row):
    kind, codec, scale, vals, codes = row
    x = np.zeros(32, np.float32)
    x[: len(vals)] = vals
    q, s = O.quantize_state(x, kind, codec)
    assert int(s[0]) == scale
    assert [int(c) for c in q[: len(codes)]] == codes
    assert np.all(q[len(codes):] == 0)


def test_ru_fp16_against_numpy_cast():
    # RU16(x) = the numpy binary16 cast (RNE) bumped up when it landed below x
    rng = np.random.default_rng(10)
    pats = np.arange(0, 0x7C00, dtype=np.uint16)
    h = pats.view(np.float16).astype(np.float32)
    x = np.concatenate([h, np.nextafter(h, np.float32(np.inf)), np.nextafter(h, np.float32(0)),
                        (rng.random(200_000) * rng.choice([1e-7, 1e-4, 1.0, 6e4], 200_000)).astype(np.float32)])
    x = x[(x >= 0) & (x <= 65504)]
    ref = x.astype(np.float16)
    below = ref.astype(np.float32) < x
    ref[below] = np.nextafter(ref[below], np.float16(np.inf))
    assert np.array_equal(O.ru_fp16_bits(x), ref.view(np.uint16))
    # saturation and NaN
    assert list(O.ru_fp16_bits(np.array([65504.5, 1e9, np.inf, np.nan], np.float32))) == [0x7BFF] * 3 + [0x7E00]


def test_momentum_code_exact_near_thresholds():
    # The exact code of a float32 a is round(127 * 2a/(1+a)).  Compare the
    # oracle with Fraction arithmetic for float32 values within a few ulps of
    # every threshold (2k+1)/(507-2k), where any evaluation error would show.
    zs = []
    for k in range(127):
        t = np.array([float(Fraction(2 * k + 1, 507 - 2 * k))], np.float32).view(np.int32)[0]
        zs.extend(int(t) + d for d in range(-3, 4))
    a32 = np.array(zs, np.int32).view(np.float32)
    a32 = a32[(a32 >= 0) & (a32 <= 1)]
    q = O.encode_momentum(a32, np.full(-(-a32.size // 32), 0x3C00, np.uint16))   # scale 1.0
    for ai, qi in zip(a32, q):
        fa = Fraction(float(ai))
        y = 254 * fa / (1 + fa)
        k = int(y)
        want = k + (1 if y - k > Fraction(1, 2) else 0)
        assert y - k != Fraction(1, 2)          # no exact ties exist
        assert int(qi) == want, (float(ai), int(qi), want)


def test_momentum_invertible_and_monotone():
    lut = momentum_lut()
    assert lut[127] == 0.0 and lut[0] == -1.0 and lut[254] == 1.0      # phi^-1(0)=0, phi^-1(+-1)=+-1
    assert np.all(np.diff(lut) > 0)
    rng = np.random.default_rng(11)
    scales = np.concatenate([np.array([0x0001, 0x03FF, 0x0400, 0x3C00, 0x7BFF], np.uint16),
                             rng.integers(1, 0x7C00, 300).astype(np.uint16)])
    codes = np.arange(-127, 128, dtype=np.int8)
    for s in scales:
        nb = -(-codes.size // 32)
        sb = np.full(nb, s, np.uint16)
        m = O.decode_momentum(codes, sb)
        assert np.all(np.diff(m.astype(np.float64)) > 0)
        assert np.array_equal(O.encode_momentum(m, sb), codes)
        m2 = O.decode_momentum(codes, sb, "linear")
        assert np.array_equal(O.encode_momentum(m2, sb, "linear"), codes)


def test_variance_invertible_and_monotone():
    rng = np.random.default_rng(12)
    scales = np.concatenate([np.array([0x0001, 0x0400, 0x3C00, 0x7BFF], np.uint16),
                             rng.integers(1, 0x7C00, 300).astype(np.uint16)])
    codes = np.arange(0, 256).astype(np.uint8)
    for s in scales:
        sb = np.full(8, s, np.uint16)
        for codec in ("companded", "linear"):
            v = O.decode_variance(codes, sb, codec)
            assert v[0] == 0.0
            assert np.all(np.diff(v.astype(np.float64)) >= 0)
            assert np.array_equal(O.encode_variance(v, sb, codec), codes), (hex(s), codec)


def test_half_step_bound_companded_domain():
    # every float32 z in a dense sweep of [0, 1]: |127*phi(z) - q| <= 1/2, i.e.
    # the code is the nearest level in the companded domain; and the decoded
    # level is within half a level spacing of z in the raw domain.
    z = np.arange(0x00000000, 0x3F800001, 97, dtype=np.int64).astype(np.int32).view(np.float32)
    sb = np.full(-(-z.size // 32), 0x3C00, np.uint16)
    q = O.encode_momentum(z, sb).astype(np.float64)
    zz = z.astype(np.float64)
    y = 254 * zz / (1 + zz)
    assert np.max(np.abs(y - q)) <= 0.5
    dec = O.decode_momentum(q.astype(np.int8), sb).astype(np.float64)
    # raw domain: the error is bounded by the distance from the level to the
    # preimages of the companded half-way points, phi^-1(y) = y / (2 - y)
    inv = lambda y: y / (2 - y)
    lvl = inv(q / 127)
    t_hi = inv(np.minimum(q + 0.5, 127) / 127)
    t_lo = inv(np.maximum(q - 0.5, 0) / 127)
    bound = np.maximum(t_hi - lvl, lvl - t_lo)
    assert np.all(np.abs(dec - zz) <= bound * (1 + 1e-6) + 1e-12)


def test_variance_half_step_bound():
    rng = np.random.default_rng(13)
    v = (rng.standard_t(3, 32 * 20000) * 1e-3).astype(np.float32) ** 2
    q, s = O.quantize_state(v, "v")
    sv = np.repeat(s.view(np.float16).astype(np.float64), 32)
    w = np.sqrt(v.astype(np.float64))
    # in the sqrt domain the code is within half a step (plus float32 rounding)
    assert np.all(np.abs(w / sv * 255 - q) <= 0.5 + 1e-5)


def test_zero_state_roundtrip():
    z = np.zeros(100, np.float32)
    for kind in ("m", "v"):
        for codec in ("companded", "linear"):
            q, s = O.quantize_state(z, kind, codec)
            assert np.all(q == 0) and np.all(s == 0)
            assert np.all(O.dequantize_state(q, s, kind, codec) == 0)


def test_scale_never_zero_for_nonzero_block_and_sqrt_domain():
    # the variance scale lives in the sqrt domain: squared gradients of 1e-3
    # (v ~ 1e-9) would underflow binary16 directly, their square roots do not
    rng = np.random.default_rng(14)
    g = (rng.standard_t(3, 32 * 1000) * 1e-3).astype(np.float32)
    v = np.float32(0.001) * g * g
    s = O.block_scales(v, "v")
    assert np.all(s > 0)
    assert np.mean(v.reshape(-1, 32).max(1).astype(np.float16) == 0) > 0.3   # direct fp16 would underflow often


def test_companding_reduces_error_heavy_tailed():
    # the pages: companding cuts quantisation error versus linear codes
    rng = np.random.default_rng(15)
    g = (rng.standard_t(3, 32 * 50000) * 1e-3).astype(np.float32)
    m = np.float32(0.1) * g
    v = np.float32(0.05) * g * g
    def med_rel(kind, codec, x):
        q, s = O.quantize_state(x, kind, codec)
        d = O.dequantize_state(q, s, kind, codec).astype(np.float64)
        nz = x != 0
        return np.median(np.abs(d[nz] - x[nz]) / np.abs(x[nz]))
    assert med_rel("m", "companded", m) < med_rel("m", "linear", m)
    assert med_rel("v", "companded", v) < 0.5 * med_rel("v", "linear", v)


def test_tail_block_covers_valid_elements_only():
    x = np.zeros(37, np.float32)
    x[33] = 0.5                  # only element of the short last block
    x[0] = 4.0
    q, s = O.quantize_state(x, "m")
    assert s.size == 2 and s[1] == np.float16(0.5).view(np.uint16) and s[0] == np.float16(4.0).view(np.uint16)
    assert q[33] == 127


def test_decode_level_spacing_is_one_division():
    # D = RN32(s/255) (variance), RN32(s/127) (linear momentum),
    # RN32(RN32(s*s)/255) (linear variance), each one correctly rounded
    # division of the block's scale; decode = RN32(D*q) (squared for the
    # companded variance).  Scales where s*RN32(1/255) rounds differently are
    # included, so a reciprocal-multiply fails here.
    pats = np.arange(0x0001, 0x7C00, 7, dtype=np.uint16)
    s = pats.view(np.float16).astype(np.float32)
    d = O.level_spacing(pats, "v", "companded")
    want = np.array([f32(rn32(Fraction(float(x)) / 255)) for x in s], np.float32)
    assert np.array_equal(d.view(np.uint32), want.view(np.uint32))
    recip = (s * (np.float32(1) / np.float32(255))).astype(np.float32)
    assert np.count_nonzero(recip != want) > 100
    dl = O.level_spacing(pats, "m", "linear")
    want = np.array([f32(rn32(Fraction(float(x)) / 127)) for x in s], np.float32)
    assert np.array_equal(dl.view(np.uint32), want.view(np.uint32))
    dv = O.level_spacing(pats, "v", "linear")
    want = np.array([f32(rn32(Fraction(float(x)) ** 2 / 255)) for x in s], np.float32)
    assert np.array_equal(dv.view(np.uint32), want.view(np.uint32))
    # decode by hand for s = 3 (0x4200): t = RN32(D*q), v = RN32(t*t)
    sb = np.array([0x4200], np.uint16)
    q = np.array([0, 1, 200, 255] + [0] * 28, np.uint8)
    v = O.decode_variance(q, sb)
    D = rn32(Fraction(3, 255))
    for qi, vi in zip(q[:4], v[:4]):
        t = rn32(D * int(qi))
        assert vi == f32(rn32(t * t))


def test_momentum_decode_of_minus_128():
    # -128 is never written by the encoder; the companded decode saturates it to
    # -127 (so every int8 decodes into [-s, s]), the linear decode is -128 * step
    sb = np.array([0x4400], np.uint16)                      # s = 4
    q = np.array([-128, -127, 127] + [0] * 29, np.int8)
    m = O.decode_momentum(q, sb)
    assert m[0] == m[1] == np.float32(-4.0) and m[2] == np.float32(4.0)
    ml = O.decode_momentum(q, sb, "linear")
    step = np.float32(4.0) / np.float32(127.0)
    assert ml[0] == step * np.float32(-128.0) and ml[1] == step * np.float32(-127.0)


def _fp16_scales(rng, k):
    return rng.integers(0x0400, 0x7BFF, k).astype(np.uint16)


def _momentum_code_exact(z: Fraction, codec: str) -> int:
    if codec == "companded":
        a = min(abs(z), Fraction(1))
        q = round_half_even(254 * a / (1 + a))
        return -q if z < 0 else q
    return max(-127, min(127, round_half_even(rn32(127 * z))))


def test_momentum_codes_exact_rational():
    # C3/C5: z = m/s is one float32 division, then the code of z.  Written out
    # with exact rationals; the inputs sit a few float32 ulps from a code
    # threshold and are kept where m * RN32(1/s) gives another code, so a
    # reciprocal-multiply in the oracle fails here.
    rng = np.random.default_rng(40)
    k = rng.integers(0, 127, 40000)
    sb = _fp16_scales(rng, k.size)
    s = sb.view(np.float16).astype(np.float32)
    sign = rng.choice([-1.0, 1.0], k.size)
    for codec in ("companded", "linear"):
        thr = (2 * k + 1) / (507.0 - 2 * k) if codec == "companded" else (k + 0.5) / 127.0
        m0 = (sign * thr * s.astype(np.float64)).astype(np.float32)
        m = (m0.view(np.int32) + rng.integers(-4, 5, k.size).astype(np.int32)).view(np.float32)
        m = np.where(np.abs(m) <= s, m, m0).astype(np.float32)
        recip = (m * (np.float32(1) / s)).astype(np.float32)
        div = (m / s).astype(np.float32)
        code_r = np.array([_momentum_code_exact(Fraction(float(z)), codec) for z in recip])
        code_d = np.array([_momentum_code_exact(Fraction(float(z)), codec) for z in div])
        pick = np.nonzero(code_r != code_d)[0][:80]
        assert pick.size >= 20, codec
        blocks = np.zeros((pick.size, 32), np.float32)
        blocks[:, 0] = m[pick]
        got = O.encode_momentum(blocks.ravel(), sb[pick], codec).reshape(-1, 32)[:, 0]
        for i, gi in zip(pick, got):
            want = _momentum_code_exact(rn32(Fraction(float(m[i])) / Fraction(float(s[i]))), codec)
            assert int(gi) == want, (codec, float(m[i]), float(s[i]), int(gi), want)


def test_variance_codes_exact_rational():
    # C4: w = sqrt_rn(v), z = w/s, y = 255*z, code = round_half_even(y), each a
    # float32 operation; C5 linear: z = v/(s*s), y = 255*z.  Inputs chosen where
    # w * RN32(255/s) (or v * RN32(255/s^2)) gives another code.
    rng = np.random.default_rng(41)
    k = rng.integers(0, 255, 20000)
    sb = _fp16_scales(rng, k.size)
    s = sb.view(np.float16).astype(np.float32)
    s64 = s.astype(np.float64)
    for codec in ("companded", "linear"):
        # inputs a few float32 ulps from a code's rounding boundary k + 1/2
        if codec == "companded":
            v0 = (((k + 0.5) / 255 * s64) ** 2).astype(np.float32)
        else:
            v0 = ((k + 0.5) / 255 * s64 * s64).astype(np.float32)
        v = (v0.view(np.int32) + rng.integers(-6, 7, k.size).astype(np.int32)).view(np.float32)
        if codec == "companded":
            wr = np.sqrt(v).astype(np.float32)
            recip = np.rint((wr * (np.float32(255) / s)).astype(np.float32))
            plain = np.rint((np.float32(255) * (wr / s).astype(np.float32)).astype(np.float32))
        else:
            s2 = (s * s).astype(np.float32)
            recip = np.rint((v * (np.float32(255) / s2)).astype(np.float32))
            plain = np.rint((np.float32(255) * (v / s2).astype(np.float32)).astype(np.float32))
        pick = np.nonzero(recip != plain)[0][:60]
        assert pick.size >= 20, codec
        blocks = np.zeros((pick.size, 32), np.float32)
        blocks[:, 0] = v[pick]
        got = O.encode_variance(blocks.ravel(), sb[pick], codec).reshape(-1, 32)[:, 0]
        for i, gi in zip(pick, got):
            fs = Fraction(float(s[i]))
            if codec == "companded":
                z = rn32(rn32_sqrt(Fraction(float(v[i]))) / fs)
            else:
                z = rn32(Fraction(float(v[i])) / (fs * fs))
            want = max(0, min(255, round_half_even(rn32(255 * z))))
            assert int(gi) == want, (codec, float(v[i]), float(s[i]), int(gi), want)


def test_nan_and_infinity_codes():
    # C6: NaN -> code 0 under every codec; +-Inf (scale saturated at 65504)
    # -> the end codes; an all-zero block has s = 0 and codes 0
    x = np.zeros(96, np.float32)
    x[0:4] = [np.nan, 1.0, -0.5, np.nan]
    x[32:35] = [np.inf, 1.0, -np.inf]
    for codec in ("companded", "linear"):
        q, s = O.quantize_state(x, "m", codec)
        assert list(s) == [0x3C00, 0x7BFF, 0x0000]
        assert q[0] == 0 and q[3] == 0 and q[1] == 127
        assert q[32] == 127 and q[34] == -127 and q[33] == 0
        assert np.all(q[64:] == 0)
        v = np.abs(x)
        qv, sv = O.quantize_state(v, "v", codec)
        assert qv[0] == 0 and qv[3] == 0 and qv[1] == 255 and qv[32] == 255 and qv[34] == 255
        assert sv[1] == 0x7BFF and sv[2] == 0 and np.all(qv[64:] == 0)
    # a negative "variance" has no square root: NaN -> 0
    qn, _ = O.quantize_state(np.array([-1.0, 4.0] + [0.0] * 30, np.float32), "v")
    assert qn[0] == 0 and qn[1] == 255


def test_short_last_block_all_nan_keeps_nan_scale():
    # C1: the valid elements of a short last block are all NaN -> NaN scale,
    # under both kinds; one finite element among them sets the scale alone
    x = np.zeros(40, np.float32)
    x[32:] = np.nan
    for kind in ("m", "v"):
        s = O.block_scales(x, kind)
        assert list(s) == [0x0000, 0x7E00]
    x[39] = 0.25
    assert list(O.block_scales(x, "m")) == [0x0000, 0x3400]
    assert list(O.block_scales(x, "v")) == [0x0000, 0x3800]        # sqrt(0.25) = 0.5
    # a NaN scale decodes every code of the block to NaN
    q = np.zeros(40, np.int8)
    s = np.array([0x0000, 0x7E00], np.uint16)
    assert np.all(np.isnan(O.decode_momentum(q, s)[32:]))
    assert np.all(np.isnan(O.decode_variance(q.view(np.uint8), s)[32:]))


def test_block_absmax_ignores_nan_unless_all_nan():
    # maxNum: a NaN element is skipped; a block with nothing but NaN keeps NaN
    x = np.zeros(96, np.float32)
    x[:32] = np.nan
    x[32:64] = np.linspace(-2.0, 1.0, 32, dtype=np.float32)
    x[40] = np.nan
    x[64:96] = np.nan
    x[95] = 0.25
    for kind in ("m", "v"):
        s = O.block_scales(np.abs(x) if kind == "v" else x, kind)
        assert s[0] == 0x7E00
        want1 = 0x4000 if kind == "m" else O.ru_fp16_bits(np.sqrt(np.array([2.0], np.float32)))[0]
        assert s[1] == want1
        want2 = 0x3400 if kind == "m" else 0x3800          # 0.25, and sqrt(0.25) = 0.5
        assert s[2] == want2
