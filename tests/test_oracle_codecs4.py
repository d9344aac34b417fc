"""Pins for the oracle's 4-bit companded state codec and its nibble storage
(CPU only).

The pages name 4-bit states only as an outlook (blog "FlashOptim: Breaking
the Memory Wall ...", Conclusion & Perspective); the oracle's reading keeps
the 8-bit codec's blocks, scales and companders and maps them onto 4-bit
codes.  Anchors: exact rational arithmetic at every code threshold
(2k+1)/(27-2k) and for the normalising division, the inverse of the
compander at the levels, the half-step bound in the companded domain, the
golden rows of codec_cases.txt, hand-packed bytes, and the first step of a
fresh state (whose update cannot depend on the codec)."""

from fractions import Fraction

import numpy as np
import pytest

import oracle as O
from oracle.codecs import momentum_lut
from oracle.optim import fresh_adamw_state, fresh_sgdm_state

from exact_fp import f32, rn32, rn32_sqrt, round_half_even

C4 = "companded4"


def _code4_exact(z: Fraction) -> int:
    a = min(abs(z), Fraction(1))
    q = round_half_even(14 * a / (1 + a))
    return -q if z < 0 else q


def test_momentum_code4_exact_near_thresholds():
    # float32 values within a few ulps of every threshold, where 7*phi(a)
    # crosses k + 1/2: the code is the exact rounding of the real number
    zs = []
    for k in range(7):
        t = np.array([float(Fraction(2 * k + 1, 27 - 2 * k))], np.float32).view(np.int32)[0]
        zs.extend(int(t) + d for d in range(-4, 5))
    a32 = np.array(zs, np.int32).view(np.float32)
    q = O.encode_momentum(a32, np.full(-(-a32.size // 32), 0x3C00, np.uint16), C4)
    for ai, qi in zip(a32, q):
        fa = Fraction(float(ai))
        y = 14 * fa / (1 + fa)
        assert y - int(y) != Fraction(1, 2)                  # no ties
        assert int(qi) == _code4_exact(fa), (float(ai), int(qi))
    # each threshold is crossed: the codes around threshold k are k and k + 1
    for k in range(7):
        around = q[9 * k: 9 * k + 9]
        assert set(int(c) for c in around) == {k, k + 1}


def test_momentum_code4_exact_rational_division():
    # z = m/s is one float32 division; inputs near thresholds where
    # m * RN32(1/s) gives another code
    rng = np.random.default_rng(140)
    k = rng.integers(0, 7, 60000)
    sb = rng.integers(0x0400, 0x7BFF, k.size).astype(np.uint16)
    s = sb.view(np.float16).astype(np.float32)
    sign = rng.choice([-1.0, 1.0], k.size)
    thr = (2 * k + 1) / (27.0 - 2 * k)
    m0 = (sign * thr * s.astype(np.float64)).astype(np.float32)
    m = (m0.view(np.int32) + rng.integers(-3, 4, k.size).astype(np.int32)).view(np.float32)
    m = np.where(np.abs(m) <= s, m, m0).astype(np.float32)
    recip = (m * (np.float32(1) / s)).astype(np.float32)
    div = (m / s).astype(np.float32)
    code_r = np.array([_code4_exact(Fraction(float(z))) for z in recip])
    code_d = np.array([_code4_exact(Fraction(float(z))) for z in div])
    pick = np.nonzero(code_r != code_d)[0][:60]
    assert pick.size >= 5
    blocks = np.zeros((pick.size, 32), np.float32)
    blocks[:, 0] = m[pick]
    got = O.encode_momentum(blocks.ravel(), sb[pick], C4).reshape(-1, 32)[:, 0]
    for i, gi in zip(pick, got):
        assert int(gi) == _code4_exact(rn32(Fraction(float(m[i])) / Fraction(float(s[i]))))


def test_variance_code4_exact_rational():
    # w = sqrt_rn(v), z = RN32(w/s), y = RN32(15*z), code = round_half_even(y)
    # in [0, 15]; inputs near the boundaries k + 1/2
    rng = np.random.default_rng(141)
    k = rng.integers(0, 15, 20000)
    sb = rng.integers(0x0400, 0x7BFF, k.size).astype(np.uint16)
    s = sb.view(np.float16).astype(np.float32)
    v0 = (((k + 0.5) / 15 * s.astype(np.float64)) ** 2).astype(np.float32)
    v = (v0.view(np.int32) + rng.integers(-6, 7, k.size).astype(np.int32)).view(np.float32)
    blocks = np.zeros((400, 32), np.float32)
    blocks[:, 0] = v[:400]
    got = O.encode_variance(blocks.ravel(), sb[:400], C4).reshape(-1, 32)[:, 0]
    for i, gi in enumerate(got):
        z = rn32(rn32_sqrt(Fraction(float(v[i]))) / Fraction(float(s[i])))
        want = max(0, min(15, round_half_even(rn32(15 * z))))
        assert int(gi) == want, (float(v[i]), float(s[i]), int(gi), want)


def test_momentum4_levels_invert_the_compander():
    # LUT4[q] is the inverse of phi at q/7: 7*phi(LUT4[q]) = q up to one
    # float32 rounding of the level; levels are odd-symmetric and increasing
    lut = momentum_lut(C4).astype(np.float64)
    assert lut.size == 15 and lut[7] == 0.0 and lut[0] == -1.0 and lut[14] == 1.0
    assert np.all(np.diff(lut) > 0) and np.array_equal(lut, -lut[::-1])
    q = np.arange(-7, 8)
    assert np.max(np.abs(14 * lut / (1 + np.abs(lut)) - q)) < 1e-5
    # 8-bit and 4-bit levels meet where the grids coincide: q4/7 = q8/127
    # never holds for 0 < |q4| < 7, but the end and middle levels are shared
    lut8 = momentum_lut("companded")
    assert lut[14] == lut8[254] and lut[7] == lut8[127]


def test_momentum4_invertible_and_monotone():
    rng = np.random.default_rng(142)
    scales = np.concatenate([np.array([0x0001, 0x03FF, 0x0400, 0x3C00, 0x7BFF], np.uint16),
                             rng.integers(1, 0x7C00, 300).astype(np.uint16)])
    codes = np.arange(-7, 8, dtype=np.int8)
    for s in scales:
        sb = np.array([s], np.uint16)
        m = O.decode_momentum(codes, sb, C4)
        assert np.all(np.diff(m.astype(np.float64)) > 0)
        assert np.array_equal(O.encode_momentum(m, sb, C4), codes)


def test_variance4_invertible_and_monotone():
    rng = np.random.default_rng(143)
    scales = np.concatenate([np.array([0x0001, 0x0400, 0x3C00, 0x7BFF], np.uint16),
                             rng.integers(1, 0x7C00, 300).astype(np.uint16)])
    codes = np.arange(0, 16).astype(np.uint8)
    for s in scales:
        sb = np.array([s], np.uint16)
        v = O.decode_variance(codes, sb, C4)
        assert v[0] == 0.0 and np.all(np.diff(v.astype(np.float64)) >= 0)
        assert np.array_equal(O.encode_variance(v, sb, C4), codes), hex(s)


def test_momentum4_half_step_bound():
    # every float32 z of a dense sweep of [0, 1]: |7*phi(z) - q| <= 1/2
    z = np.arange(0x00000000, 0x3F800001, 97, dtype=np.int64).astype(np.int32).view(np.float32)
    sb = np.full(-(-z.size // 32), 0x3C00, np.uint16)
    q = O.encode_momentum(z, sb, C4).astype(np.float64)
    zz = z.astype(np.float64)
    assert np.max(np.abs(14 * zz / (1 + zz) - q)) <= 0.5
    assert q.min() == 0 and q.max() == 7


def test_variance4_half_step_bound():
    rng = np.random.default_rng(144)
    v = (rng.standard_t(3, 32 * 20000) * 1e-3).astype(np.float32) ** 2
    q, s = O.quantize_state(v, "v", C4)
    sv = np.repeat(s.view(np.float16).astype(np.float64), 32)
    w = np.sqrt(v.astype(np.float64))
    assert np.all(np.abs(w / sv * 15 - q) <= 0.5 + 1e-5)
    assert q.max() == 15


def test_code_decode_of_minus_8():
    # -8 is never written; it decodes as -7 (every pattern decodes into [-s, s])
    sb = np.array([0x4400], np.uint16)                       # s = 4
    m = O.decode_momentum(np.array([-8, -7, 7], np.int8), sb, C4)
    assert m[0] == m[1] == np.float32(-4.0) and m[2] == np.float32(4.0)


def test_nibble_packing_by_hand():
    # element 2i -> low nibble, 2i+1 -> high nibble; 4-bit two's complement
    assert list(O.pack_nibbles(np.array([1, -1, 7, -7, 0]))) == [0xF1, 0x97, 0x00]
    assert list(O.pack_nibbles(np.array([15, 0, 3, 12, 9]))) == [0x0F, 0xC3, 0x09]
    assert list(O.unpack_nibbles(np.array([0xF1, 0x97, 0x8A], np.uint8), 6, True)) == [1, -1, 7, -7, -6, -8]
    assert list(O.unpack_nibbles(np.array([0x0F, 0xC3, 0x79], np.uint8), 5, False)) == [15, 0, 3, 12, 9]
    rng = np.random.default_rng(145)
    for n in (0, 1, 2, 31, 33, 1000):
        qm = rng.integers(-8, 8, n)
        qv = rng.integers(0, 16, n)
        assert O.pack_nibbles(qm).size == O.code_bytes(n, C4) == (n + 1) // 2
        assert np.array_equal(O.unpack_nibbles(O.pack_nibbles(qm), n, True), qm)
        assert np.array_equal(O.unpack_nibbles(O.pack_nibbles(qv), n, False), qv)


def test_zero_state4():
    z = np.zeros(100, np.float32)
    for kind in ("m", "v"):
        q, s = O.quantize_state(z, kind, C4)
        assert np.all(q == 0) and np.all(s == 0)
        assert np.all(O.dequantize_state(q, s, kind, C4) == 0)


def test_4bit_codes_are_coarser_than_8bit():
    # same blocks and scales: the 4-bit median error on heavy-tailed states
    # lies between 4x and 64x the 8-bit one (a grid 18x coarser), and the
    # momentum codes of the two widths agree on sign and on zero
    rng = np.random.default_rng(146)
    g = (rng.standard_t(3, 32 * 20000) * 1e-3).astype(np.float32)
    m = np.float32(0.1) * g
    def med(codec):
        q, s = O.quantize_state(m, "m", codec)
        d = O.dequantize_state(q, s, "m", codec).astype(np.float64)
        return np.median(np.abs(d - m)), q
    e8, q8 = med("companded")
    e4, q4 = med(C4)
    assert 4 * e8 < e4 < 64 * e8
    assert np.all(np.sign(q4) * np.sign(q8) >= 0) and np.all((q8 == 0) <= (q4 == 0))


@pytest.mark.parametrize("fmt,ecc", [("bf16", 8), ("fp16", 8), ("bf16", 16)])
def test_first_step_update_independent_of_codec(fmt, ecc):
    # from zero states (which decode to 0 under every codec) the first update
    # uses the fresh float32 m and v only: theta', rho and the scales agree
    # with the 8-bit codec; the 4-bit codes are the stored (packed) encoding
    # of the same new states
    rng = np.random.default_rng(147)
    n = 32 * 7 + 13
    x = (rng.standard_normal(n) * 0.02).astype(np.float32)
    gb = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    gbits = gb.astype(np.float16).view(np.uint16) if fmt == "fp16" else (gb.view(np.uint32) >> 16).astype(np.uint16)
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, step=1)
    a8 = O.adamw_step(fresh_adamw_state(x, fmt, ecc), gbits, hp, fmt, ecc, "companded")
    a4 = O.adamw_step(fresh_adamw_state(x, fmt, ecc, C4), gbits, hp, fmt, ecc, C4)
    for k in ("w16", "ecc", "m_s", "v_s"):
        assert np.array_equal(a8[k], a4[k]), k
    assert a4["m_q"].size == a4["v_q"].size == (n + 1) // 2
    assert a4["m_q"][-1] >> 4 == 0 and a4["v_q"][-1] >> 4 == 0          # pad nibble of the odd tail
    theta = O.reconstruct_weights(*O.split_weights(x, fmt, ecc), fmt, ecc)
    g = O.f16_bits_to_f32(gbits) if fmt == "fp16" else (gbits.astype(np.uint32) << 16).view(np.float32)
    S = O.adamw_scalars(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"], 1)
    _, m1, v1, _ = O.adamw_update(theta, g, np.zeros(n, np.float32), np.zeros(n, np.float32), S)
    assert np.array_equal(a4["m_q"], O.pack_nibbles(O.quantize_state(m1, "m", C4)[0]))
    assert np.array_equal(a4["v_q"], O.pack_nibbles(O.quantize_state(v1, "v", C4)[0]))
    s8 = O.sgdm_step(fresh_sgdm_state(x, fmt, ecc), gbits, dict(lr=0.1, momentum=0.9, weight_decay=1e-4, step=1),
                     fmt, ecc, "companded")
    s4 = O.sgdm_step(fresh_sgdm_state(x, fmt, ecc, C4), gbits, dict(lr=0.1, momentum=0.9, weight_decay=1e-4, step=1),
                     fmt, ecc, C4)
    for k in ("w16", "ecc", "b_s"):
        assert np.array_equal(s8[k], s4[k]), k
