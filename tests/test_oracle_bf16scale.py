"""Pins for the oracle's bfloat16 block scales (reading C9, codec
"companded_bf16scale"; CPU only).

Anchors: a search of the sorted table of every non-negative bfloat16 value
for the round-up scale (independent of the oracle's ceil-by-spacing), the
binary16-scale codec wherever the two formats give the same scale value,
power-of-two invariance of codes and scales (a property of any round-up to a
floating-point format in its normal range), the NaN / infinity / saturation
cases, and blocks far below binary16's range keeping their codes.
"""

import numpy as np
import pytest

import oracle as O
from oracle.optim import adamw_step, adamw_update, adamw_scalars, fresh_adamw_state

CODEC = "companded_bf16scale"

# every non-negative finite bfloat16 value, ascending with the pattern
_BF_PATS = np.arange(0, 0x7F80, dtype=np.uint32)
_BF_VALS = (_BF_PATS << 16).view(np.float32).astype(np.float64)


def _ru_bf16_by_search(x):
    """Index of the first bfloat16 value >= x in the sorted table, capped at
    the largest finite one; NaN -> 0x7FC0."""
    x = np.asarray(x, np.float32).astype(np.float64)
    nan = np.isnan(x)
    idx = np.searchsorted(_BF_VALS, np.where(nan, 0.0, x), side="left")
    idx = np.minimum(idx, 0x7F7F)
    return np.where(nan, 0x7FC0, idx).astype(np.uint16)


def test_ru_bf16_against_table_search():
    rng = np.random.default_rng(91)
    v = _BF_VALS.astype(np.float32)
    rand = rng.integers(0, 0x7F800000, 400_000, dtype=np.uint32).view(np.float32)
    x = np.concatenate([v, np.nextafter(v, np.float32(np.inf)), np.nextafter(v, np.float32(0)), rand,
                        np.array([0.0, np.inf, np.nan, np.finfo(np.float32).max,
                                  np.float32(2.0 ** -149)], np.float32)])
    x = x[np.isnan(x) | (x >= 0)]
    got = O.ru_bf16_bits(x)
    ref = _ru_bf16_by_search(x)
    assert np.array_equal(got, ref)


def test_ru_bf16_special_cases():
    got = O.ru_bf16_bits(np.array([0.0, 1.0, 1.0 + 2.0 ** -23, np.inf, np.nan, 3.4e38,
                                   2.0 ** -149, 2.0 ** -133, 2.0 ** -126], np.float32))
    # 1 + 2^-23 rounds up to 1 + 2^-7 (0x3F81); above the largest finite
    # bfloat16 (and +inf) the scale saturates at 0x7F7F; the smallest f32
    # subnormal rounds up to the smallest bfloat16 subnormal 2^-133 (0x0001)
    assert [int(b) for b in got] == [0x0000, 0x3F80, 0x3F81, 0x7F7F, 0x7FC0, 0x7F7F,
                                     0x0001, 0x0001, 0x0080]


def _state(n, rng, kind):
    x = rng.standard_t(3, n) * 1e-3
    x = np.where(np.abs(x) < 1e-7, np.copysign(1e-7, x), x).astype(np.float32)
    return np.abs(x) if kind == "v" else x


@pytest.mark.parametrize("kind", ["m", "v"])
def test_equal_to_binary16_codec_where_scales_coincide(kind):
    # block maxima set to powers of two inside binary16's normal range: both
    # formats hold them exactly, so the scales coincide and so must the codes
    rng = np.random.default_rng(92)
    n = 32 * 512
    x = _state(n, rng, kind)
    e = rng.integers(-12, 14, n // 32)
    top = np.ldexp(1.0, e).astype(np.float32)
    top = top * top if kind == "v" else top                 # v: the scale is sqrt(max v)
    b = x.reshape(-1, 32)
    b *= (top / np.max(np.abs(b), axis=1))[:, None] * np.float32(0.999)
    b[:, 7] = top if kind == "v" else np.where(rng.random(n // 32) < 0.5, -top, top)
    x = b.ravel().astype(np.float32)
    q16, s16 = O.quantize_state(x, kind, "companded")
    qb, sb = O.quantize_state(x, kind, CODEC)
    assert np.array_equal(O.scale_to_f32(s16, "companded"), O.scale_to_f32(sb, CODEC))
    assert np.array_equal(q16, qb)
    assert np.array_equal(O.dequantize_state(q16, s16, kind, "companded"),
                          O.dequantize_state(qb, sb, kind, CODEC))


@pytest.mark.parametrize("kind,k", [("m", -90), ("m", -40), ("m", -17), ("m", 5), ("m", 30), ("m", 90),
                                    ("v", -40), ("v", -17), ("v", 5), ("v", 30), ("v", 45)])
def test_power_of_two_invariance(kind, k):
    # scaling a state by 2^k (v by 4^k) keeps every code and moves every scale
    # exponent by k, anywhere in the normal range (every element stays normal)
    rng = np.random.default_rng(1000 + k)
    n = 32 * 300 + 17
    x = _state(n, rng, kind)
    f = np.float32(2.0 ** (2 * k if kind == "v" else k))
    q0, s0 = O.quantize_state(x, kind, CODEC)
    q1, s1 = O.quantize_state((x * f).astype(np.float32), kind, CODEC)
    assert np.array_equal(q0, q1)
    nz = s0 != 0
    assert np.array_equal((s1[nz] >> 7).astype(np.int64) - (s0[nz] >> 7), np.full(nz.sum(), k))
    d0 = O.dequantize_state(q0, s0, kind, CODEC).astype(np.float64)
    d1 = O.dequantize_state(q1, s1, kind, CODEC).astype(np.float64)
    assert np.array_equal(d0 * float(f), d1)


def test_tiny_blocks_keep_their_codes():
    # momentum around 1e-12: binary16 scales round up to 2^-24 and every code is
    # 0; bfloat16 scales follow the block and the decode stays within the
    # companded grid's resolution (the largest level gap is 2/127 of s)
    rng = np.random.default_rng(94)
    x = (rng.standard_normal(32 * 64) * 1e-12).astype(np.float32)
    q16, s16 = O.quantize_state(x, "m", "companded")
    assert np.all(q16 == 0)
    qb, sb = O.quantize_state(x, "m", CODEC)
    d = O.dequantize_state(qb, sb, "m", CODEC)
    s = np.repeat(O.scale_to_f32(sb, CODEC), 32)
    assert np.all(np.abs(d - x) <= s * (1.0 / 127.0))
    assert np.count_nonzero(qb) > 0.9 * x.size


def test_nan_and_infinity():
    x = np.zeros(32 * 3 + 5, np.float32)
    x[:32] = np.nan                                         # all-NaN block: NaN scale
    x[40] = np.inf                                          # saturated scale, end code
    x[41] = -2.0
    x[96:] = np.nan                                         # all-NaN short last block
    q, s = O.quantize_state(x, "m", CODEC)
    assert [int(b) for b in s] == [0x7FC0, 0x7F7F, 0x0000, 0x7FC0]
    assert q[40] == 127 and q[41] == 0 and np.all(q[:32] == 0)


def test_adamw_step_keeps_small_moments():
    # gradients of 1e-10: after one step the binary16 momentum scale 2^-24
    # codes every m of about 1e-11 as 0, the bfloat16 one keeps m within a level
    rng = np.random.default_rng(95)
    n = 32 * 40 + 9
    x32 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g = (rng.standard_normal(n) * 1e-10).astype(np.float32)
    gb = (g.view(np.uint32) >> 16).astype(np.uint16)        # exact bf16 gradients
    g = (gb.astype(np.uint32) << 16).view(np.float32)
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, step=1)
    st16 = adamw_step(fresh_adamw_state(x32, codec="companded"), gb, hp, codec="companded")
    stb = adamw_step(fresh_adamw_state(x32, codec=CODEC), gb, hp, codec=CODEC)
    assert np.array_equal(st16["w16"], stb["w16"]) and np.array_equal(st16["ecc"], stb["ecc"])
    assert np.all(st16["m_q"] == 0)
    m_true = (np.float32(0.1) * g).astype(np.float32)
    m_b = O.decode_momentum(stb["m_q"], stb["m_s"], CODEC)
    s = np.repeat(O.scale_to_f32(stb["m_s"], CODEC), 32)[:n]
    assert np.all(np.abs(m_b - m_true) <= s / 127.0)
    # the weights follow the unquantised update
    S = adamw_scalars(1e-3, 0.9, 0.999, 1e-8, 0.01, 1)
    st0 = fresh_adamw_state(x32)
    th0 = O.reconstruct_weights(st0["w16"], st0["ecc"])
    th, _, _, _ = adamw_update(th0, g, np.zeros(n, np.float32), np.zeros(n, np.float32), S)
    assert np.array_equal(O.split_weights(th)[0], stb["w16"])
