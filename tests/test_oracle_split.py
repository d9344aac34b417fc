"""Pins for the oracle's weight split / reconstruct (CPU only).

Each test checks the oracle against something other than itself: hand-derived
golden cases, an independent integer rounding, numpy's own binary16 cast,
exhaustive sweeps over every 16-bit pattern with the exact interval of f32
preimages, and identities the definition implies (bf16 + 16-bit ECC is
lossless, representable values get rho = 0, sign symmetry).
"""

import os

import numpy as np
import pytest

import oracle as O
from oracle.numerics import FORMATS, bits_to_value, spacing_in, spacing_out

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "split_cases.txt")


def _f32(bits):
    return np.asarray(bits, dtype=np.uint32).view(np.float32)


def _golden():
    rows = []
    with open(GOLDEN) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            fmt, n, x, w, r, *_ = line.split()
            rows.append((fmt, int(n), int(x, 16), int(w, 16), int(r)))
    return rows


@pytest.mark.parametrize("row", _golden(), ids=lambda r: f"{r[0]}+{r[1]}:{r[2]:08x}")
def test_golden_split(row):
    fmt, n, xb, wb, rho = row
    w, r = O.split_weights(_f32([xb]), fmt, n)
    assert int(w[0]) == wb
    assert int(r[0]) == rho


def test_golden_reconstruct_error():
    # reconstruction of every golden case lands within half an ECC step unless
    # the ECC was clamped or the value saturated
    for fmt, n, xb, wb, rho in _golden():
        x = _f32([xb])
        if not np.isfinite(x[0]):
            continue
        xr = O.reconstruct_weights(np.array([wb], np.uint16), np.array([rho]), fmt, n)
        a = abs(bits_to_value(np.array([wb], np.uint16), fmt)[0])
        ulp = spacing_out(np.array([a]), fmt)[0] if rho >= 0 else spacing_in(np.array([a]), fmt)[0]
        step = ulp * 2.0 ** -n
        err = abs(float(xr[0]) - float(x[0]))
        lim = step if abs(rho) >= 2 ** (n - 1) - 1 else step / 2
        assert err <= lim or a == FORMATS[fmt].max_finite


def test_rna_bf16_matches_integer_rounding():
    # independent integer RNA on the magnitude bits: (bits + 0x8000) >> 16
    rng = np.random.default_rng(1)
    u = rng.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    # force a large share of exact ties and near-ties
    u[::4] = (u[::4] & 0xFFFF0000) | 0x8000
    u[1::8] = (u[1::8] & 0xFFFF0000) | 0x7FFF
    x = _f32(u)
    mag = u & 0x7FFFFFFF
    keep = mag < 0x7F7F8000            # finite and no bf16 overflow
    w, _ = O.split_weights(x[keep], "bf16", 8)
    want = ((mag[keep] + 0x8000) >> 16) | ((u[keep] >> 16) & 0x8000)
    assert np.array_equal(w.astype(np.uint32), want)


def test_rna_fp16_vs_numpy_rne():
    # numpy's binary16 cast rounds half to even; off ties it must agree with
    # RNA, on ties RNA must pick the larger magnitude.
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(1_000_000) * rng.choice([1e-6, 1e-3, 1.0, 300.0], 1_000_000)).astype(np.float32)
    x = x[np.abs(x) < 65504]
    w, _ = O.split_weights(x, "fp16", 8)
    ours = w.view(np.float16).astype(np.float64)
    rne = x.astype(np.float16).astype(np.float64)
    lo = np.abs(x.astype(np.float64))
    # a tie is exactly half way between two fp16 neighbours
    a = np.abs(rne)
    sp_o = spacing_out(a, "fp16")
    sp_i = spacing_in(np.where(a > 0, a, 1.0), "fp16")
    tie = (lo - a == sp_o / 2) | (a - lo == sp_i / 2)
    assert np.array_equal(ours[~tie], rne[~tie])
    assert np.all(np.abs(ours[tie]) >= np.abs(rne[tie]))


def _preimage_sweep(fmt, n):
    """For every finite 16-bit pattern (except the max, whose upper edge is the
    overflow), build f32 points at and around both edges of its RNA interval
    [a - ulp_in/2, a + ulp_out/2) plus random interior points, and check that
    split lands in the right pattern with error <= half an ECC step (or < one
    step in the clamped outermost sliver)."""
    F = FORMATS[fmt]
    pats = np.arange(0, 0x8000, dtype=np.uint16)
    a = bits_to_value(pats, fmt)
    ok = np.isfinite(a) & (a < F.max_finite)
    pats, a = pats[ok], a[ok]
    uo = spacing_out(a, fmt)
    ui = np.where(a > 0, spacing_in(np.where(a > 0, a, 1.0), fmt), 0.0)
    lo_edge = a - ui / 2                       # tie below: belongs to a (RNA)
    hi_edge = a + uo / 2                       # tie above: belongs to the next value
    lo32 = lo_edge.astype(np.float32)
    hi32 = hi_edge.astype(np.float32)
    assert np.array_equal(lo32.astype(np.float64), lo_edge)
    assert np.array_equal(hi32.astype(np.float64), hi_edge)
    below_hi = np.nextafter(hi32, np.float32(0))
    above_lo = np.nextafter(lo32, np.float32(np.inf))
    rng = np.random.default_rng(3)
    t = rng.random((64, a.size))
    inner = (lo_edge[None, :] + t * (hi_edge - lo_edge)[None, :]).astype(np.float32)
    inner = np.minimum(inner, below_hi[None, :])
    inner = np.where(inner < lo32[None, :], lo32[None, :], inner)
    pts = np.concatenate([lo32[None], above_lo[None], a.astype(np.float32)[None], below_hi[None], inner])
    pts = np.where(a[None, :] == 0, np.abs(pts), pts)      # zero's interval is [0, ulp/2)
    want = np.broadcast_to(pats[None, :], pts.shape)
    for sgn in (1.0, -1.0):
        x = (pts * np.float32(sgn)).ravel()
        w, r = O.split_weights(x, fmt, n)
        exp_w = want.ravel() | (np.uint16(0x8000) if sgn < 0 else np.uint16(0))
        assert np.array_equal(w, exp_w), fmt
        xr = O.reconstruct_weights(w, r, fmt, n).astype(np.float64)
        aa = np.broadcast_to(a[None, :], pts.shape).ravel()
        step = np.where(r >= 0, spacing_out(aa, fmt), spacing_in(np.where(aa > 0, aa, 1.0), fmt)) * 2.0 ** -n
        err = np.abs(xr - x.astype(np.float64))
        clamped = np.abs(r.astype(np.int64)) >= 2 ** (n - 1) - 1
        assert np.all(err[~clamped] <= step[~clamped] / 2)
        assert np.all(err[clamped] < step[clamped])
    # the upper tie itself goes to the next pattern
    w, _ = O.split_weights(hi32, fmt, n)
    assert np.array_equal(w, pats + 1)


@pytest.mark.parametrize("fmt,n", [("bf16", 8), ("bf16", 16), ("fp16", 8)])
def test_exhaustive_patterns_with_preimages(fmt, n):
    _preimage_sweep(fmt, n)


def _identity_check(u32):
    x = _f32(u32)
    mag = u32 & 0x7FFFFFFF
    keep = mag < 0x7F7F8000              # finite, below the bf16 overflow tie
    x = x[keep]
    w, r = O.split_weights(x, "bf16", 16)
    xr = O.reconstruct_weights(w, r, "bf16", 16)
    assert np.array_equal(xr.view(np.uint32), x.view(np.uint32))


def test_bf16_ecc16_identity_strided():
    """bf16 + 16-bit ECC reconstructs every finite f32 below the bf16 overflow
    tie exactly.  Default: a stride through all 2^32 patterns plus two full
    binades around 1.0 and the normal/subnormal boundary.  Set FO_EXHAUSTIVE=1
    for all 2^32 patterns."""
    if os.environ.get("FO_EXHAUSTIVE") == "1":
        chunk = 1 << 26
        for s in range(0, 1 << 32, chunk):
            _identity_check(np.arange(s, s + chunk, dtype=np.uint64).astype(np.uint32))
        return
    _identity_check(np.arange(0, 1 << 32, 251, dtype=np.uint64).astype(np.uint32))
    _identity_check(np.arange(0x3F000000, 0x3F800000 + (1 << 20), dtype=np.uint64).astype(np.uint32))
    _identity_check(np.arange(0x00700000, 0x00900000, dtype=np.uint64).astype(np.uint32))


@pytest.mark.parametrize("fmt,n", [("bf16", 8), ("bf16", 16), ("fp16", 8)])
def test_representable_values_have_zero_ecc(fmt, n):
    pats = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    v = bits_to_value(pats, fmt)
    ok = np.isfinite(v)
    x = v[ok].astype(np.float32)
    w, r = O.split_weights(x, fmt, n)
    assert np.all(r == 0)
    assert np.array_equal(w, pats[ok])


@pytest.mark.parametrize("fmt,n", [("bf16", 8), ("bf16", 16), ("fp16", 8)])
def test_sign_symmetry(fmt, n):
    rng = np.random.default_rng(4)
    x = (rng.standard_normal(200_000) * 0.02).astype(np.float32)
    w1, r1 = O.split_weights(x, fmt, n)
    w2, r2 = O.split_weights(-x, fmt, n)
    assert np.array_equal(w1 ^ np.uint16(0x8000), w2)
    assert np.array_equal(r1, r2)


def test_specials():
    x = np.array([np.nan, -np.nan, np.inf, -np.inf, 0.0, -0.0, 3.4e38, -3.4e38], np.float32)
    w, r = O.split_weights(x, "bf16", 8)
    assert [int(v) for v in w] == [0x7FC0, 0xFFC0, 0x7F80, 0xFF80, 0x0000, 0x8000, 0x7F7F, 0xFF7F]
    assert list(r[:6]) == [0] * 6 and r[6] == 127 and r[7] == 127
    w, r = O.split_weights(np.array([70000.0, -1e6, np.inf], np.float32), "fp16", 8)
    assert [int(v) for v in w] == [0x7BFF, 0xFBFF, 0x7C00]
    assert list(r) == [127, 127, 0]
    with pytest.raises(ValueError):
        O.split_weights(np.zeros(3, np.float32), "fp16", 16)


def test_error_bound_normal_distribution():
    # the weights the workloads use: N(0, 0.02); bf16+8 error <= half a step
    # except in the clamped sliver; fp16+8 likewise
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(1_000_000) * 0.02).astype(np.float32)
    for fmt in ("bf16", "fp16"):
        w, r = O.split_weights(x, fmt, 8)
        xr = O.reconstruct_weights(w, r, fmt, 8).astype(np.float64)
        a = np.abs(bits_to_value(w, fmt))
        step = np.where(r >= 0, spacing_out(a, fmt), spacing_in(np.where(a > 0, a, 1.0), fmt)) / 256
        err = np.abs(xr - x)
        cl = np.abs(r.astype(int)) >= 127
        assert np.all(err[~cl] <= step[~cl] / 2)
        assert np.all(err[cl] < step[cl])
        # the ECC is a real refinement: 8 more bits cut the mean error ~256x
        err16 = np.abs(x.astype(np.float64) - bits_to_value(w, fmt))
        assert np.mean(err) < np.mean(err16) / 100
