"""GPU checks of the exact fast arithmetic used by the fused kernels, and of the
table-driven momentum encode, through the C ABI.

fo_selftest compares, on the device, the Newton-refined hardware reciprocal
and the corrected hardware square roots (both neighbours of the estimate, or
one neighbour of the successor's estimate) with the IEEE operations,
and the hardware float-to-u8 conversion with round-half-even + clamp (NaN to
0), over every f32 pattern of the ranges the kernels use them on; and the
residual-corrected division with IEEE division on billions of seeded pairs
from the ranges the kernels admit.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
from precision_optimizer_state_amd import binding as B

pytestmark = pytest.mark.gpu


def test_refined_reciprocal_exact_on_all_positive_normals_below_2_126():
    lo, hi = 0x00800000, 0x7E800000
    assert B.fo_selftest(0, lo, hi - lo) == 0


def test_corrected_sqrt_exact_from_2_minus_96_to_inf():
    lo, hi = 0x0F800000, 0x7F800001
    assert B.fo_selftest(1, lo, hi - lo) == 0
    # zero takes the fast path too
    assert B.fo_selftest(1, 0, 1) == 0


def test_successor_sqrt_exact_on_the_fast_step_domain():
    # every f32 from 2^-96 up to the largest finite one (excluded), and zero;
    # the AdamW step takes it for variances 0 and [2^-96, 2^100]
    lo, hi = 0x0F800000, 0x7F7FFFFF
    assert B.fo_selftest(6, lo, hi - lo) == 0
    assert B.fo_selftest(6, 0, 1) == 0


def test_successor_sqrt_fails_where_it_is_not_used():
    # the largest finite float (its successor is infinite) and the tiny
    # variances below 2^-96, which the gradient range keeps off the fast path
    assert B.fo_selftest(6, 0x7F7FFFFF, 1) == 1
    assert B.fo_selftest(6, 1, 0x0F800000 - 1) > 0


def test_cvt_pk_u8_is_round_half_even_and_saturating_everywhere():
    # every f32 pattern, NaN included (NaN must give 0: the codes of NaN states)
    assert B.fo_selftest(2, 0, 1 << 32) == 0


@pytest.mark.parametrize("seed", [1, 2])
def test_corrected_division_equals_ieee_division(seed):
    # divisors over the whole range of the refined reciprocal, dividends over
    # the range the fast AdamW step admits (and zero), quotients normal
    assert B.fo_selftest(3, seed, 1 << 32) == 0


def test_corrected_division_by_block_scales_equals_ieee_division():
    # fp16 divisors (block scales) with |dividend| <= divisor: the encodes
    assert B.fo_selftest(4, 7, 1 << 32) == 0


def test_selftest_detects_the_range_the_fast_paths_avoid():
    # the fallbacks exist for a reason: the fast forms are wrong on denormals,
    # and the corrected division is wrong for some subnormal quotients (two
    # of the pairs of seed 1, found again by the CPU reproduction of the
    # generator), which the AdamW step's gradient range keeps out
    assert B.fo_selftest(0, 1, 0x00800000 - 1) > 0
    assert B.fo_selftest(1, 1, 0x0F800000 - 1) > 0
    assert B.fo_selftest(5, 1, 1 << 32) > 0


def test_momentum_codes_exact_around_every_threshold():
    """Blocks whose largest magnitude is exactly 1 have scale 1 and R = 1, so
    the kernel encodes z = m itself: sweep every f32 within 64 ulps of each
    code threshold (2k+1)/(507-2k), every key-interval boundary of the
    kernel's table, and a stride through [0, 1], and compare with the exact
    code round(254 z / (1 + z)) of the oracle (spot-checked with Fractions)."""
    pts = []
    for k in range(127):
        t = np.array([float(Fraction(2 * k + 1, 507 - 2 * k))], np.float32).view(np.int32)[0]
        pts.append(np.arange(t - 64, t + 65, dtype=np.int64))
    for key in range(0x3B00, 0x3F81):
        b = key << 16
        pts.append(np.arange(b - 4, b + 5, dtype=np.int64))
    pts.append(np.arange(0, 0x3F800001, 4099, dtype=np.int64))
    u = np.unique(np.concatenate(pts))
    u = u[(u >= 0) & (u <= 0x3F800000)].astype(np.uint32)
    z = u.view(np.float32)
    sign = np.where(np.arange(z.size) % 2 == 0, 1.0, -1.0).astype(np.float32)
    z = z * sign
    # layout: 31 values + one 1.0 per 32-element block
    nb = -(-z.size // 31)
    x = np.zeros(nb * 32, np.float32)
    x.reshape(nb, 32)[:, 0] = 1.0
    body = x.reshape(nb, 32)[:, 1:].reshape(-1)
    body[: z.size] = z
    x.reshape(nb, 32)[:, 1:] = body.reshape(nb, 31)
    q_ref, s_ref = O.quantize_state(x, "m", "companded")
    assert np.all(s_ref == 0x3C00)
    codes = torch.empty(x.size, dtype=torch.int8, device="cuda")
    scales = torch.empty(nb, dtype=torch.float16, device="cuda")
    B.fo_companded_quantize(torch.from_numpy(x).cuda(), codes, scales, "m", "companded")
    torch.cuda.synchronize()
    got = codes.cpu().numpy()
    bad = np.count_nonzero(got != q_ref)
    print(f"momentum codes near thresholds: {x.size} values, {bad} mismatches", flush=True)
    assert bad == 0
    # spot-check the oracle's codes with exact rationals
    rng = np.random.default_rng(0)
    for i in rng.choice(x.size, 2000, replace=False):
        a = Fraction(float(abs(x[i])))
        y = 254 * a / (1 + a)
        k = int(y)
        want = k + (1 if y - k > Fraction(1, 2) else 0)
        assert abs(int(q_ref[i])) == want
