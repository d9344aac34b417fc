"""bfloat16 block scales (codec "companded_bf16scale") on the GPU, against the oracle.

Reading C9 of the oracle: the companded 8-bit codes of the binary16-scale
codec with each block scale rounded up to bfloat16 instead.  The kernels take
their fast forms while every block scale of a wave lies in binary16's range
(zero or [2^-24, 65504]) and the IEEE forms otherwise, so the tests drive
states through both: ordinary magnitudes, states far below 2^-24 and above
65504, NaN and infinite gradients, and arbitrary stored scale patterns
(subnormal, tiny, huge, NaN).  Every comparison is bitwise; the fused steps
run lock-step (the oracle steps a host copy of the device state before every
GPU step)."""

import numpy as np
import pytest
import torch

import oracle as O
from oracle.numerics import split_weights
from precision_optimizer_state_amd import binding as B
from precision_optimizer_state_amd.state import alloc_adamw_state, alloc_sgdm_state
from workloads import host_grad_bits, host_grads, host_weights

from gpu_helpers import check_codes, run_lockstep, to_dev, to_host

pytestmark = pytest.mark.gpu

CB = "companded_bf16scale"
DT = {"bf16": torch.bfloat16, "fp16": torch.float16}
HP_C1 = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
HP_C4 = dict(lr=0.1, momentum=0.9, weight_decay=1e-4)
SIZES = [1, 7, 31, 33, 1000, 2047, 2048, 2049, 4097, 8193, 100_003]


def _quantize_case(kind, n, mag, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_t(3, n) * mag).astype(np.float32)
    if kind == "v":
        x = (x * x).astype(np.float32)
    return x


@pytest.mark.parametrize("kind", ["m", "v"])
@pytest.mark.parametrize("mag", [1e-3, 1e-12, 1e-25, 1e3, 1e15])
@pytest.mark.parametrize("n", [1, 33, 4097, 100_003])
def test_quantize_dequantize_match_oracle(kind, mag, n):
    # magnitudes inside binary16's scale range, below it (fast forms off) and
    # above it; NaN and infinite elements in the larger cases
    x = _quantize_case(kind, n, mag, [n, int(np.log10(mag)) + 40, kind == "v"])
    if n > 40:
        x[3] = np.nan
        x[n // 2] = np.inf if kind == "v" else -np.inf
        x[n - n % 32:] = np.nan if n % 32 else x[n - n % 32:]
    xd = torch.from_numpy(x).cuda()
    codes = torch.full((n,), 0x55, dtype=torch.int8 if kind == "m" else torch.uint8, device="cuda")
    scales = torch.empty((n + 31) // 32, dtype=torch.float16, device="cuda")
    B.fo_companded_quantize(xd, codes, scales, kind, CB)
    q, s = O.quantize_state(x, kind, CB)
    torch.cuda.synchronize()
    tag = f"{kind} n={n} mag={mag:g}"
    check_codes(f"{tag} scales", to_host(scales), s)
    check_codes(f"{tag} codes", to_host(codes), q)
    back = torch.empty(n, dtype=torch.float32, device="cuda")
    B.fo_dequantize(codes, scales, back, kind, CB)
    want = O.dequantize_state(q, s, kind, CB)
    got = back.cpu().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(want))
    check_codes(f"{tag} decode", np.nan_to_num(got).view(np.uint32), np.nan_to_num(want).view(np.uint32))


@pytest.mark.parametrize("kind", ["m", "v"])
def test_dequantize_every_code_with_assorted_scales(kind):
    # every code under bfloat16 scale patterns from zero and subnormals
    # through tiny and huge normals to the largest finite value and NaN
    rng = np.random.default_rng(97)
    nb = 128
    codes = np.tile(np.arange(256, dtype=np.int64), nb // 8)
    codes = codes.astype(np.int8) if kind == "m" else codes.astype(np.uint8)
    sb = rng.integers(0, 0x7F80, nb).astype(np.uint16)
    sb[:10] = [0x0000, 0x0001, 0x007F, 0x0080, 0x0D00, 0x3380, 0x3C00, 0x477F, 0x7F7F, 0x7FC0]
    out = torch.empty(codes.size, dtype=torch.float32, device="cuda")
    B.fo_dequantize(to_dev(codes, torch.int8 if kind == "m" else torch.uint8), to_dev(sb, torch.float16), out,
                    kind, CB)
    torch.cuda.synchronize()
    want = O.dequantize_state(codes, sb, kind, CB)
    got = out.cpu().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(want))
    check_codes(f"{kind} every code", np.nan_to_num(got).view(np.uint32), np.nan_to_num(want).view(np.uint32))


def _init(kind, sizes, fmt, ecc_bits, tag):
    dev = []
    for i, n in enumerate(sizes):
        st = (alloc_adamw_state if kind == "adamw" else alloc_sgdm_state)(n, fmt, ecc_bits, codec=CB)
        if n:
            B.fo_split_weights(torch.from_numpy(host_weights(tag, i, n)).cuda(), st["w16"], st["ecc"], fmt, ecc_bits)
        dev.append(st)
    return dev


def _grads(tag, sizes, fmt, kind, scale_of=None, inject=None):
    def grads(i, step):
        g = host_grads(tag, i, step, sizes[i], kind)
        if scale_of is not None:
            g = (g * np.float32(scale_of(i, step))).astype(np.float32)
        if inject is not None:
            g = inject(i, step, g)
        return host_grad_bits(g, fmt)
    return grads


def _inject_specials(i, step, g):
    g = g.copy()
    if g.size > 4096:
        g[5] = np.nan
        g[77] = np.inf
        g[4000] = -np.inf
        g[2048 + 64: 2048 + 96] = np.nan
    if g.size % 32 and g.size > 64:
        g[g.size - g.size % 32:] = np.nan
    return g


@pytest.mark.parametrize("fmt,ecc_bits", [("bf16", 8), ("bf16", 16), ("fp16", 8)])
def test_fused_adamw_lockstep(fmt, ecc_bits):
    tag = f"bs_adamw_{fmt}{ecc_bits}"
    n = run_lockstep("adamw", _init("adamw", SIZES, fmt, ecc_bits, tag), 3,
                     _grads(tag, SIZES, fmt, "t3"), HP_C1, fmt, ecc_bits, CB, tag)
    assert n == 3 * len(SIZES)


@pytest.mark.parametrize("l2", [False, True])
def test_fused_adamw_magnitudes_outside_binary16_scales(l2):
    # per tensor and step, gradients scaled by 1e-9 (moments far below 2^-24),
    # by 1e6 (variance roots above 65504) or left alone, so waves alternate
    # between the fast and the IEEE forms from one step to the next
    fmt, ecc_bits = "bf16", 8
    tag = f"bs_mag_l2{int(l2)}"
    factors = (1.0, 1e-9, 1e6, 1e-20, 1.0)
    scale_of = lambda i, step: factors[(i + step) % len(factors)]   # noqa: E731
    run_lockstep("adamw", _init("adamw", SIZES, fmt, ecc_bits, tag), 5,
                 _grads(tag, SIZES, fmt, "t3", scale_of), dict(HP_C1, l2_decay=l2), fmt, ecc_bits, CB, tag)


def test_fused_adamw_nan_inf_grads():
    fmt, ecc_bits = "bf16", 8
    tag = "bs_special"
    run_lockstep("adamw", _init("adamw", SIZES, fmt, ecc_bits, tag), 3,
                 _grads(tag, SIZES, fmt, "t3", inject=_inject_specials), HP_C1, fmt, ecc_bits, CB, tag)


@pytest.mark.parametrize("nesterov,dampening", [(False, 0.0), (True, 0.0), (False, 0.2)])
def test_fused_sgdm_lockstep(nesterov, dampening):
    fmt, ecc_bits = "bf16", 8
    tag = f"bs_sgdm_{int(nesterov)}{dampening}"
    factors = (1.0, 1e-12, 1.0, 1e7)
    scale_of = lambda i, step: factors[(i + step) % len(factors)]   # noqa: E731
    run_lockstep("sgdm", _init("sgdm", SIZES, fmt, ecc_bits, tag), 4,
                 _grads(tag, SIZES, fmt, "normal_outliers", scale_of),
                 dict(HP_C4, nesterov=nesterov, dampening=dampening), fmt, ecc_bits, CB, tag)


def _random_bf16_scales(rng, nb):
    s = rng.integers(0, 0x7F80, nb).astype(np.uint16)
    s[::5] = 0
    s[1::7] = rng.integers(0x3380, 0x4780, s[1::7].size)     # inside binary16's range
    s[2::11] = 0x7FC0
    s[3::13] = rng.integers(1, 0x80, s[3::13].size)           # subnormal
    return s


@pytest.mark.parametrize("fmt,ecc_bits", [("bf16", 8), ("fp16", 8)])
def test_fused_steps_from_arbitrary_states(fmt, ecc_bits):
    # random stored codes with random bfloat16 scale patterns, stepped from a
    # late step count by AdamW and by SGD-M
    rng = np.random.default_rng(98)
    sizes = [1, 31, 33, 2048, 4097, 20000]
    dev_a, dev_s = [], []
    for i, n in enumerate(sizes):
        w16, ecc = split_weights(host_weights("bs_arb", i, n), fmt, ecc_bits)
        nb = -(-n // 32)
        a = alloc_adamw_state(n, fmt, ecc_bits, codec=CB)
        s = alloc_sgdm_state(n, fmt, ecc_bits, codec=CB)
        for d in (a, s):
            d["w16"].copy_(to_dev(w16, DT[fmt]))
            d["ecc"].copy_(to_dev(ecc, d["ecc"].dtype))
        a["m_q"].copy_(to_dev(rng.integers(-128, 128, n).astype(np.int8), torch.int8))
        a["v_q"].copy_(to_dev(rng.integers(0, 256, n).astype(np.uint8), torch.uint8))
        a["m_s"].copy_(to_dev(_random_bf16_scales(rng, nb), torch.float16))
        a["v_s"].copy_(to_dev(_random_bf16_scales(rng, nb), torch.float16))
        s["b_q"].copy_(to_dev(rng.integers(-128, 128, n).astype(np.int8), torch.int8))
        s["b_s"].copy_(to_dev(_random_bf16_scales(rng, nb), torch.float16))
        dev_a.append(a)
        dev_s.append(s)
    grads = lambda i, step: host_grad_bits(host_grads("bs_arb", i, step, sizes[i], "t3"), fmt)   # noqa: E731
    run_lockstep("adamw", dev_a, 0, grads, HP_C1, fmt, ecc_bits, CB, f"arbitrary adamw {fmt}", step_list=(7, 8))
    run_lockstep("sgdm", dev_s, 0, grads, HP_C4, fmt, ecc_bits, CB, f"arbitrary sgdm {fmt}", step_list=(7, 8))
