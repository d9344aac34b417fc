"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Sizes are ones the oracle finishes in seconds while spanning many wave tiles
and ragged tails.  Full-size workloads are in test_gpu_configs.py.  The fused
steps run in lock-step (tests/gpu_helpers.py: the oracle steps a host copy of
the device state before each step) and must match bitwise; the device split
of the initial weights is compared with the oracle's split first.
"""

import os

import numpy as np
import pytest
import torch

import oracle as O
from oracle.numerics import FORMATS, bits_to_value, spacing_in, spacing_out
from precision_optimizer_state_amd import binding as B
from precision_optimizer_state_amd.state import alloc_adamw_state, alloc_sgdm_state
from tests.gpu_helpers import (
    check_codes,
    check_weights,
    run_lockstep,
    to_dev,
    to_host,
)
from workloads import host_grad_bits, host_grads, host_weights

pytestmark = pytest.mark.gpu
DT = {"bf16": torch.bfloat16, "fp16": torch.float16}
ECC_DT = {8: torch.int8, 16: torch.int16}
VARIANTS = [("bf16", 8), ("bf16", 16), ("fp16", 8)]


def _split_inputs(fmt, seed=0):
    """Edges and interiors of every 16-bit pattern's rounding interval, both
    signs, plus N(0, 0.02) weights, random f32 bit patterns and specials."""
    F = FORMATS[fmt]
    pats = np.arange(0, 0x8000, dtype=np.uint16)
    a = bits_to_value(pats, fmt)
    ok = np.isfinite(a) & (a < F.max_finite)
    a = a[ok]
    uo = spacing_out(a, fmt)
    ui = np.where(a > 0, spacing_in(np.where(a > 0, a, 1.0), fmt), 0.0)
    lo = (a - ui / 2).astype(np.float32)
    hi = (a + uo / 2).astype(np.float32)
    rng = np.random.default_rng(seed)
    t = rng.random((6, a.size))
    inner = (lo[None].astype(np.float64) + t * (hi - lo)[None]).astype(np.float32)
    pts = np.concatenate([lo, np.nextafter(lo, np.float32(np.inf)), a.astype(np.float32),
                          np.nextafter(hi, np.float32(0)), hi, inner.ravel()])
    pts = np.abs(pts)
    x = np.concatenate([pts, -pts,
                        (rng.standard_normal(1_000_000) * 0.02).astype(np.float32),
                        rng.integers(0, 2 ** 32, 500_000, dtype=np.uint64).astype(np.uint32).view(np.float32),
                        np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 3.4e38, -3.4e38, 70000.0, 1e-45, -1e-45,
                                  65519.0, 65520.0, 6.1e-5, 5.96e-8], np.float32)])
    return x.astype(np.float32)


@pytest.mark.parametrize("fmt,ecc_bits", VARIANTS)
def test_split_matches_oracle_bitwise(fmt, ecc_bits):
    x = _split_inputs(fmt)
    print(f"split {fmt}+{ecc_bits}: n={x.size}", flush=True)
    w_ref, e_ref = O.split_weights(x, fmt, ecc_bits)
    xd = torch.from_numpy(x).cuda()
    w = torch.empty(x.size, dtype=DT[fmt], device="cuda")
    e = torch.empty(x.size, dtype=ECC_DT[ecc_bits], device="cuda")
    B.fo_split_weights(xd, w, e, fmt, ecc_bits)
    torch.cuda.synchronize()
    wg, eg = to_host(w), to_host(e)
    nan = np.isnan(x)
    assert np.array_equal(wg[~nan], w_ref[~nan]), f"theta' differs on {np.count_nonzero(wg[~nan] != w_ref[~nan])}"
    assert np.array_equal(eg, e_ref), f"rho differs on {np.count_nonzero(eg != e_ref)}"
    # NaN inputs: quiet NaN with the input's sign
    assert np.array_equal(wg[nan], w_ref[nan])


@pytest.mark.parametrize("fmt,ecc_bits", VARIANTS)
def test_reconstruct_matches_oracle_bitwise(fmt, ecc_bits):
    x = _split_inputs(fmt, seed=1)
    w_ref, e_ref = O.split_weights(x, fmt, ecc_bits)
    r_ref = O.reconstruct_weights(w_ref, e_ref, fmt, ecc_bits)
    out = torch.empty(x.size, dtype=torch.float32, device="cuda")
    B.fo_reconstruct_weights(to_dev(w_ref, DT[fmt]), to_dev(e_ref, ECC_DT[ecc_bits]), out, fmt, ecc_bits)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    nan = np.isnan(r_ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), r_ref[~nan].view(np.uint32))


@pytest.mark.parametrize("fmt", ["bf16", "fp16"])
def test_reconstruct_every_pattern_and_offset(fmt):
    """ECC decode (the device function the fused steps use) on every finite
    16-bit pattern with every 8-bit offset, against the oracle.  The domain is
    the one reconstruction is defined on: rho >= 0 when theta' is +-0."""
    h = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    h = h[np.isfinite(bits_to_value(h, fmt))]
    rho = np.arange(-128, 128, dtype=np.int64)
    H = np.repeat(h, rho.size)
    R = np.tile(rho, h.size)
    keep = ~(((H & 0x7FFF) == 0) & (R < 0))
    H, R = H[keep], R[keep].astype(np.int8)
    want = O.reconstruct_weights(H, R, fmt, 8)
    out = torch.empty(H.size, dtype=torch.float32, device="cuda")
    B.fo_reconstruct_weights(to_dev(H, DT[fmt]), to_dev(R, torch.int8), out, fmt, 8)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    bad = int(np.count_nonzero(got.view(np.uint32) != want.view(np.uint32)))
    print(f"decode {fmt}+8 over {H.size} (pattern, offset) pairs: {bad} mismatches", flush=True)
    assert bad == 0


@pytest.mark.skipif(os.environ.get("FO_EXHAUSTIVE") != "1",
                    reason="every f32 pattern through the oracle takes ~3 min per format; set FO_EXHAUSTIVE=1")
@pytest.mark.parametrize("fmt", ["bf16", "fp16"])
def test_split_ecc8_every_f32_pattern(fmt):
    """The 8-bit-ECC split of all 2^32 f32 patterns against the oracle: theta'
    for every non-NaN input and rho for every input (NaN theta' is checked in
    test_split_matches_oracle_bitwise)."""
    bad = 0
    for c0 in range(0, 1 << 32, 1 << 28):
        x = np.arange(c0, c0 + (1 << 28), dtype=np.uint64).astype(np.uint32).view(np.float32)
        w = torch.empty(x.size, dtype=DT[fmt], device="cuda")
        e = torch.empty(x.size, dtype=torch.int8, device="cuda")
        B.fo_split_weights(torch.from_numpy(x).cuda(), w, e, fmt, 8)
        torch.cuda.synchronize()
        wg, eg = to_host(w), to_host(e)
        for s0 in range(0, x.size, 1 << 23):
            xs = x[s0:s0 + (1 << 23)]
            wr, er = O.split_weights(xs, fmt, 8)
            bw = (wg[s0:s0 + (1 << 23)] != wr) & ~np.isnan(xs)
            bad += int(np.count_nonzero(bw | (eg[s0:s0 + (1 << 23)] != er)))
        print(f"split {fmt}+8: patterns below {c0 + (1 << 28):#x}: {bad} mismatches", flush=True)
        del w, e
    assert bad == 0


def test_bf16_ecc16_identity_all_f32_patterns_on_device():
    """split -> reconstruct with bf16 + 16-bit ECC is the identity on every
    finite f32 below the bf16 overflow tie: all 2^32 patterns, on the device."""
    chunk = 1 << 28
    w = torch.empty(chunk, dtype=torch.bfloat16, device="cuda")
    e = torch.empty(chunk, dtype=torch.int16, device="cuda")
    r = torch.empty(chunk, dtype=torch.float32, device="cuda")
    bad = 0
    for s in range(0, 1 << 32, chunk):
        u = torch.arange(s, s + chunk, dtype=torch.int64, device="cuda").to(torch.int32)
        x = u.view(torch.float32)
        B.fo_split_weights(x, w, e, "bf16", 16)
        B.fo_reconstruct_weights(w, e, r, "bf16", 16)
        keep = (u & 0x7FFFFFFF) < 0x7F7F8000
        bad += int(((r.view(torch.int32) != u) & keep).sum().item())
        del u, x, keep
    print(f"bf16+16 identity over 2^32 patterns: {bad} mismatches", flush=True)
    assert bad == 0


def _state_inputs(kind, n, seed):
    rng = np.random.default_rng(seed)
    nb = -(-n // 32)
    block_scale = np.repeat(10.0 ** rng.uniform(-9, 4, nb), 32)[:n]
    g = rng.standard_t(3, n)
    if kind == "m":
        x = g * block_scale
    else:
        x = (g * g) * block_scale
    x = x.astype(np.float32)
    x[: 32 * 3] = 0.0                          # all-zero blocks
    x[200:232] = x[200:232] * 1e-30            # underflowing scale
    if kind == "m":
        x[300] = 1e6                           # saturating scale
    return x


@pytest.mark.parametrize("kind", ["m", "v"])
@pytest.mark.parametrize("codec", ["companded", "linear"])
@pytest.mark.parametrize("n", [1 << 20, 1000, 4095 * 7 + 3])
def test_quantize_dequantize_match_oracle(kind, codec, n):
    x = _state_inputs(kind, n, seed=n)
    q_ref, s_ref = O.quantize_state(x, kind, codec)
    nb = -(-n // 32)
    codes = torch.empty(n, dtype=torch.int8 if kind == "m" else torch.uint8, device="cuda")
    scales = torch.empty(nb, dtype=torch.float16, device="cuda")
    B.fo_companded_quantize(torch.from_numpy(x).cuda(), codes, scales, kind, codec)
    out = torch.empty(n, dtype=torch.float32, device="cuda")
    B.fo_dequantize(to_dev(q_ref, codes.dtype), to_dev(s_ref, torch.float16), out, kind, codec)
    torch.cuda.synchronize()
    check_codes(f"quantize {kind}/{codec} codes", to_host(codes), q_ref)
    check_codes(f"quantize {kind}/{codec} scales", to_host(scales), s_ref)
    d_ref = O.dequantize_state(q_ref, s_ref, kind, codec)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), d_ref.view(np.uint32))


@pytest.mark.parametrize("kind", ["m", "v"])
@pytest.mark.parametrize("codec", ["companded", "linear"])
def test_quantize_special_values(kind, codec):
    """NaN, infinities, values that saturate the fp16 scale, signed zeros and
    subnormals, alone and mixed with ordinary values in a block."""
    rng = np.random.default_rng(41)
    sp = np.array([np.nan, np.inf, -np.inf, 3.0e38, -3.0e38, 1.0e6, -1.0e6, 65504.0, 65520.0, -0.0, 0.0,
                   1e-45, -1e-45, 1e-30, 6.0e-8, 1.0], np.float32)
    if kind == "v":
        sp = np.where(np.isnan(sp), sp, np.abs(sp)).astype(np.float32)
    blocks = [np.full(32, v, np.float32) for v in sp]
    for v in sp:
        b = (rng.standard_normal(32) * 0.01).astype(np.float32)
        if kind == "v":
            b = b * b
        b[rng.integers(0, 32)] = v
        blocks.append(b)
    x = np.concatenate(blocks + [sp[:7]])
    q_ref, s_ref = O.quantize_state(x, kind, codec)
    n = x.size
    codes = torch.empty(n, dtype=torch.int8 if kind == "m" else torch.uint8, device="cuda")
    scales = torch.empty(-(-n // 32), dtype=torch.float16, device="cuda")
    B.fo_companded_quantize(torch.from_numpy(x).cuda(), codes, scales, kind, codec)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(scales), s_ref)
    assert np.array_equal(to_host(codes), q_ref)


def _oracle_code_steps():
    """Smallest f32 pattern in [0, 1] whose oracle momentum code (scale 1) is
    at least k + 1, for k = 0..126, by bisection over the patterns (the code
    is non-decreasing in the value)."""
    one = np.full(4, 0x3C00, np.uint16)                  # fp16 1.0 for every block
    code = lambda p: O.encode_momentum(p.astype(np.uint32).view(np.float32), one, "companded").astype(np.int64)
    want = np.arange(1, 128)
    lo = np.zeros(127, np.int64)
    hi = np.full(127, 0x3F800000, np.int64)
    assert np.all(code(lo) < want) and np.all(code(hi) >= want)
    while np.any(hi - lo > 1):
        mid = (lo + hi) // 2
        up = code(mid) >= want
        hi = np.where(up, mid, hi)
        lo = np.where(up, lo, mid)
    return hi


def test_momentum_encode_every_f32_in_unit_interval():
    """The companded momentum code of every f32 value in [0, 1] (and its
    negative) at block scale 1.  Each 32-block is [1.0, 31 consecutive
    patterns], so the scale is fp16 1.0, the reciprocal is exactly 1 and the
    kernel codes z = a itself.  The codes must rise from 0 in 127 unit steps
    placed exactly at the oracle's thresholds, which is the oracle's code on
    all 1,065,353,217 values; negated inputs must give negated codes."""
    N = 0x3F800000 + 1
    nblk = -(-N // 31)
    x = torch.empty(nblk, 32, dtype=torch.int32, device="cuda")
    x[:, 0] = 0x3F800000
    x[:, 1:] = torch.arange(nblk * 31, dtype=torch.int32, device="cuda").view(nblk, 31).clamp_(max=0x3F800000)
    xf = x.view(torch.float32).view(-1)
    codes = torch.empty(nblk * 32, dtype=torch.int8, device="cuda")
    scales = torch.empty(nblk, dtype=torch.float16, device="cuda")
    B.fo_companded_quantize(xf, codes, scales, "m", "companded")
    assert bool((scales.view(torch.int16) == 0x3C00).all())
    cv = codes.view(nblk, 32)[:, 1:].reshape(-1)[:N]
    assert int(cv[0]) == 0
    steps = torch.nonzero(cv[1:] != cv[:-1]).flatten() + 1
    assert steps.numel() == 127, f"{steps.numel()} code changes over [0, 1]"
    assert bool(((cv[steps].to(torch.int32) - cv[steps - 1].to(torch.int32)) == 1).all())
    ref = _oracle_code_steps()
    got = steps.cpu().numpy().astype(np.int64)
    print(f"momentum code steps: {int(np.sum(got != ref))} of 127 misplaced", flush=True)
    assert np.array_equal(got, ref)
    xf.neg_()
    neg = torch.empty_like(codes)
    B.fo_companded_quantize(xf, neg, scales, "m", "companded")
    assert bool((neg == codes.neg()).all())


def _init_states(kind, sizes, fmt, ecc_bits, tag):
    """Device states from seeded f32 weights split on the device; the split
    must equal the oracle's."""
    dev = []
    for i, n in enumerate(sizes):
        x = host_weights(tag, i, n)
        st = (alloc_adamw_state if kind == "adamw" else alloc_sgdm_state)(n, fmt, ecc_bits)
        if n:
            B.fo_split_weights(torch.from_numpy(x).cuda(), st["w16"], st["ecc"], fmt, ecc_bits)
            w_ref, e_ref = O.split_weights(x, fmt, ecc_bits)
            torch.cuda.synchronize()
            check_weights(f"{tag} initial split tensor {i}", to_host(st["w16"]), to_host(st["ecc"]), w_ref, e_ref,
                          fmt, ecc_bits)
        dev.append(st)
    return dev


def _run_adamw(sizes, steps, hp, fmt="bf16", ecc_bits=8, codec="companded", tag="t", inject=None):
    """Lock-step GPU vs oracle over `steps` AdamW steps on a list of tensors."""
    dev = _init_states("adamw", sizes, fmt, ecc_bits, tag)

    def grads(i, step):
        g = host_grads(tag, i, step, sizes[i], "t3")
        if inject is not None:
            g = inject(i, step, g)
        return host_grad_bits(g, fmt)

    return run_lockstep("adamw", dev, steps, grads, hp, fmt, ecc_bits, codec, tag)


HP_C1 = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
HP_LM = dict(lr=6e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)


def test_fused_adamw_flat_1m_10_steps():
    checks = _run_adamw([1 << 20], 10, HP_C1, tag="c1_flat1m")
    print(f"c1 flat 1M: {checks} lock-step checks, all bitwise equal", flush=True)


TAIL_SIZES = list(range(1, 34)) + [63, 64, 65, 1000, 2047, 2048, 2049, 4095, 4096, 4097, 8191, 8193, 20000]


def test_fused_adamw_ragged_tails_multi_tensor():
    rng = np.random.default_rng(7)
    sizes = TAIL_SIZES + [int(v) for v in rng.integers(1, 100_000, 6)]
    checks = _run_adamw(sizes, 3, HP_LM, tag="tails")
    print(f"{len(sizes)} ragged tensors: {checks} lock-step checks, all bitwise equal", flush=True)


@pytest.mark.parametrize("fmt,ecc_bits,codec", [("fp16", 8, "companded"), ("bf16", 16, "companded"),
                                                ("bf16", 8, "linear"), ("fp16", 8, "linear"),
                                                ("bf16", 16, "linear")])
def test_fused_adamw_variants(fmt, ecc_bits, codec):
    sizes = [300_000, 4097, 33, 1]
    _run_adamw(sizes, 4, HP_C1, fmt, ecc_bits, codec, tag=f"var_{fmt}{ecc_bits}{codec}")


def _inject_specials(i, step, g):
    """Isolated NaN/inf gradients, whole 32-element blocks of NaN and of inf
    (an all-NaN block gets a NaN scale, which keeps the state NaN), and a
    short last block (the tensor has 8192 + 5 elements) whose valid elements
    are all NaN, which must keep a NaN scale too."""
    g = g.copy()
    g[5] = np.nan
    g[77] = np.inf
    g[4000] = -np.inf
    g[2048 + 64: 2048 + 96] = np.nan
    g[6144 + 32: 6144 + 64] = np.inf
    if g.size % 32:
        g[g.size - g.size % 32:] = np.nan
    return g


@pytest.mark.parametrize("fmt,ecc_bits,codec", [("bf16", 8, "companded"), ("fp16", 8, "companded"),
                                                ("bf16", 16, "companded"), ("bf16", 8, "linear")])
def test_fused_adamw_nan_inf_grads_propagate(fmt, ecc_bits, codec):
    _run_adamw([8192 + 5], 3, HP_C1, fmt, ecc_bits, codec, tag="nan", inject=_inject_specials)


def _magnitude_band_grads(fmt, n_tiles, step, seed):
    """Gradient bit patterns whose wave tile t (2048 elements) holds values of
    one power-of-two band: |g| in [2^(e0+t), 2^(e0+t+1)) with random signs and
    significands, e0 the smallest exponent of the format's subnormals.  The
    bands run through every exponent of the format, so some tiles lie wholly
    just inside the AdamW fast range, some straddle its edges and take the
    IEEE form, and some overflow to infinity."""
    rng = np.random.default_rng([seed, step])
    e0 = -133 if fmt == "bf16" else -24
    ex = e0 + np.repeat(np.arange(n_tiles), 2048)
    mag = np.ldexp(1.0 + rng.random(ex.size), ex)
    with np.errstate(over="ignore"):                # the top bands overflow to infinity on purpose
        g = (mag * np.where(rng.random(ex.size) < 0.5, -1.0, 1.0)).astype(np.float32)
    g[::97] = 0.0                                   # exact zeros stay on the fast path
    return host_grad_bits(g, fmt)


@pytest.mark.parametrize("fmt,hp", [("bf16", HP_C1), ("bf16", HP_LM), ("fp16", HP_C1),
                                    ("bf16", dict(HP_C1, beta1=0.0, eps=1e-30)),
                                    ("bf16", dict(HP_C1, l2_decay=True)), ("fp16", dict(HP_LM, l2_decay=True))])
def test_fused_adamw_gradient_magnitude_bands(fmt, hp):
    """Lock-step over gradients swept through every exponent, tile by tile:
    the per-tile choice between the exact fast form and the IEEE form must
    never change a result (both must equal the oracle bitwise)."""
    n_tiles = 262 if fmt == "bf16" else 42
    sizes = [n_tiles * 2048 + 5]
    dev = _init_states("adamw", sizes, fmt, 8, f"band_{fmt}")
    checks = run_lockstep("adamw", dev, 3, lambda i, step: np.concatenate(
        [_magnitude_band_grads(fmt, n_tiles, step, 91), host_grad_bits(np.full(5, 1e-3, np.float32), fmt)]),
        hp, fmt, 8, "companded", f"bands {fmt}")
    print(f"magnitude bands {fmt}: {checks} lock-step checks, all bitwise equal", flush=True)


@pytest.mark.parametrize("name,hp", [
    ("beta1_0", dict(lr=1e-3, beta1=0.0, beta2=0.5, eps=1e-8, weight_decay=0.01)),
    ("lr_0", dict(lr=0.0, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)),
    ("large_lr_no_decay", dict(lr=0.5, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.0)),
    ("tiny_eps", dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-30, weight_decay=0.01)),
    ("eps_below_normal", dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-40, weight_decay=0.01)),
])
def test_fused_adamw_degenerate_hyperparameters(name, hp):
    """Hyperparameters at the edges of their ranges take the same path through
    the oracle and the kernel (eps below the smallest normal switches the
    kernel to its IEEE reciprocal)."""
    _run_adamw([20000, 33], 3, hp, tag=f"hp_{name}")


def test_fused_adamw_late_step_and_zero_eps():
    """Bias correction near 1 at step 10^6, and eps = 0, where blocks whose
    variance decodes to zero divide by zero: NaN and Inf must appear at the
    same elements on both sides (NaN weights are compared as NaN)."""
    n = 4096 + 7
    for hp, step0 in ((dict(HP_C1), 10 ** 6), (dict(HP_C1, eps=0.0), 1)):
        dev = _init_states("adamw", [n], "bf16", 8, "late")

        def grads(i, step):
            g = host_grads("late", 0, step, n, "t3")
            g[:64] = 0.0                                    # whole zero blocks: v stays 0
            return host_grad_bits(g, "bf16")

        run_lockstep("adamw", dev, 0, grads, hp, tag=f"late step0={step0} eps={hp['eps']}",
                     step_list=range(step0, step0 + 3))


def _run_sgdm(sizes, steps, hp, fmt="bf16", ecc_bits=8, codec="companded", tag="s", inject=None):
    """Lock-step GPU vs oracle over `steps` SGD-M steps on a list of tensors."""
    dev = _init_states("sgdm", sizes, fmt, ecc_bits, tag)

    def grads(i, step):
        g = host_grads(tag, i, step, sizes[i], "normal_outliers")
        if inject is not None:
            g = inject(i, step, g)
        return host_grad_bits(g, fmt)

    return run_lockstep("sgdm", dev, steps, grads, hp, fmt, ecc_bits, codec, tag)


HP_C4 = dict(lr=0.1, momentum=0.9, weight_decay=1e-4)


@pytest.mark.parametrize("fmt,codec", [("bf16", "companded"), ("fp16", "companded"), ("bf16", "linear")])
def test_fused_sgdm_nan_inf_grads_propagate(fmt, codec):
    _run_sgdm([8192 + 5], 3, HP_C4, fmt, 8, codec, tag="snan", inject=_inject_specials)


@pytest.mark.parametrize("fmt,ecc_bits,codec", [("bf16", 8, "companded"), ("bf16", 16, "companded"),
                                                ("fp16", 8, "companded"), ("bf16", 8, "linear")])
def test_fused_sgdm_matches_oracle(fmt, ecc_bits, codec):
    sizes = [9408, 64, 64, 4096, 36864, 16384, 1000, 2_048_000 // 8, 33, 1]
    _run_sgdm(sizes, 5, HP_C4, fmt, ecc_bits, codec, tag=f"sgdm_{fmt}{ecc_bits}{codec}")


@pytest.mark.parametrize("nesterov,dampening", [(True, 0.0), (False, 0.5), (False, 1.0)])
def test_fused_sgd_nesterov_and_dampening_match_oracle(nesterov, dampening):
    sizes = [9408, 4096, 2049, 33, 1, 100_000]
    hp = dict(HP_C4, nesterov=nesterov, dampening=dampening)
    _run_sgdm(sizes, 4, hp, tag=f"sgd_n{int(nesterov)}_d{dampening}")


@pytest.mark.parametrize("fmt,ecc_bits,codec", [("bf16", 8, "companded"), ("fp16", 8, "companded"),
                                                ("bf16", 16, "linear")])
def test_fused_adam_l2_decay_matches_oracle(fmt, ecc_bits, codec):
    sizes = [300_000, 4097, 33, 1]
    hp = dict(HP_C1, weight_decay=0.05, l2_decay=True)
    _run_adamw(sizes, 4, hp, fmt, ecc_bits, codec, tag=f"adam_l2_{fmt}{ecc_bits}{codec}")


@pytest.mark.parametrize("name,hp", [
    ("momentum_0", dict(lr=0.1, momentum=0.0, weight_decay=1e-4)),
    ("momentum_0_dampening", dict(lr=0.1, momentum=0.0, weight_decay=1e-4, dampening=0.5)),
    ("lr_0", dict(lr=0.0, momentum=0.9, weight_decay=1e-4)),
    ("no_decay", dict(lr=0.1, momentum=0.99, weight_decay=0.0)),
])
def test_fused_sgd_degenerate_hyperparameters(name, hp):
    """Momentum 0 takes the first-step rule at every step (torch keeps no
    buffer then, so dampening has no effect)."""
    _run_sgdm([20000, 33], 3, hp, tag=f"sgd_hp_{name}")


def test_gradient_release_chunks_equal_whole_tensor():
    """Stepping 32-aligned chunks of a tensor in separate calls (as gradients
    arrive) gives bitwise the same state as one call on the whole tensor."""
    n = (1 << 20) + 4096
    x = host_weights("release", 0, n)
    a = alloc_adamw_state(n)
    B.fo_split_weights(torch.from_numpy(x).cuda(), a["w16"], a["ecc"])
    b = {k: (v.clone() if v is not None else None) for k, v in a.items()}
    bounds = [0, 1 << 18, 1 << 19, (1 << 19) + 2048, 1 << 20, n]
    for step in (1, 2, 3):
        gb = host_grad_bits(host_grads("release", 0, step, n, "t3"), "bf16")
        a["grad"].copy_(to_dev(gb, torch.bfloat16))
        b["grad"].copy_(a["grad"])
        hp = B.adamw_hparams(step=step, **HP_C1)
        B.fo_fused_adamw_step([a], hp)
        for lo, hi in zip(bounds[:-1], bounds[1:]):
            chunk = {k: b[k][lo:hi] for k in ("w16", "ecc", "grad", "m_q", "v_q")}
            chunk["m_s"] = b["m_s"][lo // 32: -(-hi // 32)]
            chunk["v_s"] = b["v_s"][lo // 32: -(-hi // 32)]
            B.fo_fused_adamw_step([chunk], hp)
    torch.cuda.synchronize()
    for k in ("w16", "ecc", "m_q", "m_s", "v_q", "v_s"):
        assert torch.equal(a[k].view(torch.uint8), b[k].view(torch.uint8)), k


def test_determinism_two_runs_bitwise_equal():
    n = 3 * (1 << 18) + 17
    x = torch.from_numpy(host_weights("det", 0, n)).cuda()
    outs = []
    for _ in range(2):
        st = alloc_adamw_state(n)
        B.fo_split_weights(x, st["w16"], st["ecc"])
        for step in (1, 2):
            st["grad"].copy_(to_dev(host_grad_bits(host_grads("det", 0, step, n, "t3"), "bf16"), torch.bfloat16))
            B.fo_fused_adamw_step([st], B.adamw_hparams(step=step, **HP_LM))
        outs.append({k: v.clone() for k, v in st.items()})
    for k in ("w16", "ecc", "m_q", "m_s", "v_q", "v_s"):
        assert torch.equal(outs[0][k].view(torch.uint8), outs[1][k].view(torch.uint8)), k


def test_stream_probe_preserves_data_with_zero_key():
    n = 100_003
    st = alloc_adamw_state(n)
    for k in ("w16", "ecc", "m_q", "v_q"):
        st[k].view(torch.uint8).copy_(torch.randint(0, 256, (st[k].numel() * st[k].element_size(),),
                                                    dtype=torch.uint8, device="cuda"))
    before = {k: v.clone() for k, v in st.items()}
    B.fo_stream_probe([st], "bf16", 8, 0)
    torch.cuda.synchronize()
    for k in before:
        assert torch.equal(before[k].view(torch.uint8), st[k].view(torch.uint8)), k


def test_stream_probe_rewrites_every_byte_once():
    """A nonzero key: every ECC, code and scale byte of the list comes back
    XOR-ed with the key's byte at its position in the word (so each was read
    and written exactly once, the ragged tail included), and theta' comes back
    unchanged, because the probe folds the gradient into its key for theta'
    and the gradients here are zero."""
    key = 0x5AC3_961E
    for n in (100_003, 2048 * 4 + 5):
        st = alloc_adamw_state(n)
        for k in ("w16", "ecc", "m_q", "v_q", "m_s", "v_s"):
            st[k].view(torch.uint8).copy_(torch.randint(0, 256, (st[k].numel() * st[k].element_size(),),
                                                        dtype=torch.uint8, device="cuda"))
        st["grad"].zero_()
        before = {k: v.clone() for k, v in st.items()}
        B.fo_stream_probe([st], "bf16", 8, key)
        torch.cuda.synchronize()
        kb = torch.tensor([(key >> (8 * i)) & 0xFF for i in range(4)], dtype=torch.uint8, device="cuda")
        for k in ("ecc", "m_q", "v_q"):
            b = before[k].view(torch.uint8)
            want = b ^ kb.repeat((b.numel() + 3) // 4)[:b.numel()]
            assert torch.equal(st[k].view(torch.uint8), want), f"n={n}: {k}"
        for k in ("m_s", "v_s"):
            want = before[k].view(torch.int16) ^ torch.tensor(key & 0xFFFF, dtype=torch.int32).to(torch.int16).item()
            assert torch.equal(st[k].view(torch.int16), want.to("cuda")), f"n={n}: {k}"
        assert torch.equal(st["w16"].view(torch.uint8), before["w16"].view(torch.uint8)), f"n={n}: w16"


def test_aliasing_list_rejected():
    st = alloc_adamw_state(4096)
    bad = dict(st)
    bad["v_q"] = st["m_q"].view(torch.uint8)
    with pytest.raises(B.FoError) as ei:
        B.fo_fused_adamw_step([bad], B.adamw_hparams(step=1, **HP_C1))
    assert ei.value.code == B.FO_EALIAS
