"""4-bit companded states (codec "companded4") on the GPU, against the oracle.

Reading C8 of the oracle: the 8-bit codec's blocks, fp16 scales and
companders, codes narrowed to [-7, 7] (momentum) and [0, 15] (variance),
two per byte (element 2i in the low nibble).  Every comparison is bitwise on
the stored arrays, nibble padding of odd-length tensors included; the fused
steps run lock-step (the oracle steps a host copy of the device state before
every GPU step)."""

import numpy as np
import pytest
import torch

import oracle as O
from precision_optimizer_state_amd import binding as B
from precision_optimizer_state_amd.state import alloc_adamw_state, alloc_sgdm_state
from workloads import host_grad_bits, host_grads, host_weights

from gpu_helpers import check_codes, check_weights, run_lockstep, to_host

pytestmark = pytest.mark.gpu

C4 = "companded4"
HP_C1 = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
HP_LM = dict(lr=6e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
HP_C4 = dict(lr=0.1, momentum=0.9, weight_decay=1e-4)
TAIL_SIZES = list(range(1, 34)) + [63, 64, 65, 1000, 2047, 2048, 2049, 4095, 4096, 4097, 8191, 8193, 20000]


def _init(kind, sizes, fmt, ecc_bits, tag):
    dev = []
    for i, n in enumerate(sizes):
        x = host_weights(tag, i, n)
        st = (alloc_adamw_state if kind == "adamw" else alloc_sgdm_state)(n, fmt, ecc_bits, codec=C4)
        if n:
            B.fo_split_weights(torch.from_numpy(x).cuda(), st["w16"], st["ecc"], fmt, ecc_bits)
            w_ref, e_ref = O.split_weights(x, fmt, ecc_bits)
            torch.cuda.synchronize()
            check_weights(f"{tag} split {i}", to_host(st["w16"]), to_host(st["ecc"]), w_ref, e_ref, fmt, ecc_bits)
        dev.append(st)
    return dev


def _grads(tag, sizes, fmt, kind, inject=None):
    def grads(i, step):
        g = host_grads(tag, i, step, sizes[i], kind)
        if inject is not None:
            g = inject(i, step, g)
        return host_grad_bits(g, fmt)
    return grads


def _adamw(sizes, steps, hp, fmt="bf16", ecc_bits=8, tag="s4", inject=None):
    dev = _init("adamw", sizes, fmt, ecc_bits, tag)
    return run_lockstep("adamw", dev, steps, _grads(tag, sizes, fmt, "t3", inject), hp, fmt, ecc_bits, C4, tag)


def _sgdm(sizes, steps, hp, fmt="bf16", ecc_bits=8, tag="s4s", inject=None):
    dev = _init("sgdm", sizes, fmt, ecc_bits, tag)
    return run_lockstep("sgdm", dev, steps, _grads(tag, sizes, fmt, "normal_outliers", inject), hp, fmt,
                        ecc_bits, C4, tag)


def _inject_specials(i, step, g):
    g = g.copy()
    g[5] = np.nan
    g[77] = np.inf
    g[4000] = -np.inf
    g[2048 + 64: 2048 + 96] = np.nan
    g[6144 + 32: 6144 + 64] = np.inf
    if g.size % 32:
        g[g.size - g.size % 32:] = np.nan
    return g


@pytest.mark.parametrize("kind", ["m", "v"])
@pytest.mark.parametrize("n", [1, 7, 31, 33, 1000, 4097, 100_003])
def test_quantize_dequantize4_match_oracle(kind, n):
    rng = np.random.default_rng([n, kind == "v"])
    x = (rng.standard_t(3, n) * 1e-3).astype(np.float32)
    if kind == "v":
        x = x * x
    if n > 40:
        x[3] = np.nan
        x[n // 2] = np.inf if kind == "v" else -np.inf
    xd = torch.from_numpy(x).cuda()
    codes = torch.full(((n + 1) // 2,), 0xAA, dtype=torch.uint8, device="cuda")
    scales = torch.empty((n + 31) // 32, dtype=torch.float16, device="cuda")
    B.fo_companded_quantize(xd, codes, scales, kind, C4)
    q, s = O.quantize_state(x, kind, C4)
    torch.cuda.synchronize()
    check_codes(f"{kind} n={n} scales", to_host(scales), s)
    check_codes(f"{kind} n={n} codes", to_host(codes), O.pack_nibbles(q))
    back = torch.empty(n, dtype=torch.float32, device="cuda")
    B.fo_dequantize(codes, scales, back, kind, C4)
    want = O.dequantize_state(q, s, kind, C4)
    got = back.cpu().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(want))
    check_codes(f"{kind} n={n} decode", np.nan_to_num(got).view(np.uint32), np.nan_to_num(want).view(np.uint32))


def test_dequantize4_every_code_and_pattern_minus_8():
    # every byte value (all pairs of nibbles, the never-written -8 included)
    # decodes as the oracle decodes it, for several scales
    b = np.tile(np.arange(256, dtype=np.uint8), 4)                # 1024 bytes = 2048 codes = 64 blocks
    sb = np.array([0x3C00, 0x0001, 0x7BFF, 0x4200] * 16, np.uint16)
    for kind in ("m", "v"):
        out = torch.empty(b.size * 2, dtype=torch.float32, device="cuda")
        B.fo_dequantize(torch.from_numpy(b).cuda(), torch.from_numpy(sb.view(np.float16)).cuda(), out, kind, C4)
        q = O.unpack_nibbles(b, b.size * 2, kind == "m")
        want = O.dequantize_state(q, sb, kind, C4)
        check_codes(f"{kind} all nibbles", out.cpu().numpy().view(np.uint32), want.view(np.uint32))


def test_momentum4_encode_every_f32_in_unit_interval():
    """The 4-bit momentum code of every f32 in [0, 1] at block scale 1 (each
    block is [1.0, 31 consecutive patterns]): 7 unit steps exactly at the
    oracle's thresholds, and negated inputs give negated codes."""
    N = 0x3F800000 + 1
    nblk = -(-N // 31)
    x = torch.empty(nblk, 32, dtype=torch.int32, device="cuda")
    x[:, 0] = 0x3F800000
    x[:, 1:] = torch.arange(nblk * 31, dtype=torch.int32, device="cuda").view(nblk, 31).clamp_(max=0x3F800000)
    xf = x.view(torch.float32).view(-1)
    codes = torch.empty(nblk * 16, dtype=torch.uint8, device="cuda")
    scales = torch.empty(nblk, dtype=torch.float16, device="cuda")

    def unpack(c):
        lo = (c & 15).to(torch.int8)
        hi = (c >> 4).to(torch.int8)
        q = torch.stack([lo, hi], 1).view(-1)
        return torch.where(q >= 8, q - 16, q)

    B.fo_companded_quantize(xf, codes, scales, "m", C4)
    assert bool((scales.view(torch.int16) == 0x3C00).all())
    q = unpack(codes)
    cv = q.view(nblk, 32)[:, 1:].reshape(-1)[:N]
    assert int(cv[0]) == 0 and int(cv[-1]) == 7
    steps = torch.nonzero(cv[1:] != cv[:-1]).flatten() + 1
    assert steps.numel() == 7, f"{steps.numel()} code changes over [0, 1]"
    assert bool(((cv[steps].to(torch.int32) - cv[steps - 1].to(torch.int32)) == 1).all())
    # the oracle's steps: the first f32 a with round(7*phi(a)) = k + 1
    ref = []
    for k in range(7):
        t = np.float32(np.float64(2 * k + 1) / np.float64(27 - 2 * k))
        cand = np.arange(int(np.array([t]).view(np.int32)[0]) - 2, int(np.array([t]).view(np.int32)[0]) + 3,
                         dtype=np.int32)
        codes_c = O.encode_momentum(cand.view(np.float32), np.array([0x3C00], np.uint16), C4)
        ref.append(int(cand[np.argmax(codes_c == k + 1)]))
    got = steps.cpu().numpy().astype(np.int64)
    assert np.array_equal(got, np.array(ref)), (got, ref)
    xf.neg_()
    neg = torch.empty_like(codes)
    B.fo_companded_quantize(xf, neg, scales, "m", C4)
    assert bool((unpack(neg) == -q).all())


def test_fused_adamw4_flat_and_ragged_tails():
    rng = np.random.default_rng(8)
    sizes = [1 << 20] + TAIL_SIZES + [int(v) for v in rng.integers(1, 100_000, 4)]
    checks = _adamw(sizes, 3, HP_LM, tag="s4_tails")
    print(f"4-bit AdamW, {len(sizes)} tensors: {checks} lock-step checks, all bitwise equal", flush=True)


@pytest.mark.parametrize("fmt,ecc_bits", [("fp16", 8), ("bf16", 16)])
def test_fused_adamw4_formats(fmt, ecc_bits):
    _adamw([300_000, 4097, 33, 1], 4, HP_C1, fmt, ecc_bits, tag=f"s4_{fmt}{ecc_bits}")


@pytest.mark.parametrize("fmt,ecc_bits", [("bf16", 8), ("fp16", 8)])
def test_fused_adam4_l2_decay(fmt, ecc_bits):
    _adamw([300_000, 4097, 33, 1], 4, dict(HP_C1, weight_decay=0.05, l2_decay=True), fmt, ecc_bits,
           tag=f"s4_l2_{fmt}")


@pytest.mark.parametrize("fmt,ecc_bits", [("bf16", 8), ("fp16", 8), ("bf16", 16)])
def test_fused_adamw4_nan_inf_grads(fmt, ecc_bits):
    _adamw([8192 + 5], 3, HP_C1, fmt, ecc_bits, tag="s4_nan", inject=_inject_specials)


def test_fused_adamw4_large_values_take_the_ieee_encodes():
    """Gradients of 6e4 and 1e5 with beta2 = 0 make square roots of the
    variance near and past 65504 (saturated scales): the 4-bit variance code
    must clamp at 15 where the 8-bit conversion would saturate at 255."""
    n = 4096 + 9
    dev = _init("adamw", [n], "bf16", 8, "s4_big")

    def grads(i, step):
        g = host_grads("s4_big", 0, step, n, "t3")
        g[:512] = np.where(g[:512] < 0, np.float32(-6.0e4), np.float32(6.0e4))
        g[512:1024] = np.where(g[512:1024] < 0, np.float32(-1.0e5), np.float32(1.0e5))
        return host_grad_bits(g, "bf16")

    run_lockstep("adamw", dev, 3, grads, dict(HP_C1, beta2=0.0), "bf16", 8, C4, "s4_big")


@pytest.mark.parametrize("fmt,ecc_bits", [("bf16", 8), ("fp16", 8), ("bf16", 16)])
def test_fused_sgdm4_matches_oracle(fmt, ecc_bits):
    sizes = [9408, 64, 4096, 36864, 1000, 2_048_000 // 8, 33, 1, 7]
    _sgdm(sizes, 4, HP_C4, fmt, ecc_bits, tag=f"s4_sgd_{fmt}{ecc_bits}")


@pytest.mark.parametrize("nesterov,dampening", [(True, 0.0), (False, 0.5)])
def test_fused_sgd4_nesterov_and_dampening(nesterov, dampening):
    _sgdm([9408, 2049, 33, 1], 3, dict(HP_C4, nesterov=nesterov, dampening=dampening), tag="s4_sgd_nd")


def test_fused_sgdm4_nan_inf_grads():
    _sgdm([8192 + 5], 3, HP_C4, tag="s4_snan", inject=_inject_specials)


def test_one_list_under_two_code_widths_is_validated_per_width():
    """A list validated for 4-bit codes (arrays of ceil(n/2) bytes) is not
    taken as validated for 8-bit codes, whose arrays would overlap: the
    8-bit call on the same addresses must report the overlap."""
    n = 4096
    st = alloc_adamw_state(n, codec=C4)
    st["w16"].zero_()
    st["ecc"].zero_()
    buf = torch.zeros(n, dtype=torch.uint8, device="cuda")
    st["m_q"] = buf[: n // 2]
    st["v_q"] = buf[n // 2:]
    tl = B.AdamWList([st])
    B.fo_fused_adamw_step(tl, B.adamw_hparams(1e-3, 0.9, 0.999, 1e-8, 0.0, 1, codec=C4))
    torch.cuda.synchronize()
    with pytest.raises(B.FoError) as ei:
        B.fo_fused_adamw_step(tl, B.adamw_hparams(1e-3, 0.9, 0.999, 1e-8, 0.0, 1, codec="companded"))
    assert ei.value.code == B.FO_EALIAS


# ---------------------------------------------------------------------------
# drop-in optimizers with 4-bit states
# ---------------------------------------------------------------------------
def _model(seed):
    torch.manual_seed(seed)
    return torch.nn.Sequential(torch.nn.Linear(64, 96), torch.nn.GELU(), torch.nn.Linear(96, 33)).cuda()


def _loss(model, i):
    g = torch.Generator(device="cuda")
    g.manual_seed(2000 + i)
    x = torch.randn(128, 64, generator=g, device="cuda").to(torch.bfloat16)
    y = torch.randn(128, 33, generator=g, device="cuda").to(torch.bfloat16)
    return torch.nn.functional.mse_loss(model(x).float(), y.float())


def _host(opt, p, keys):
    st = opt.state[p]
    out = {"w16": to_host(p.data.view(-1)), "ecc": to_host(st["ecc"].view(-1))}
    out.update({k: to_host(st[k].view(-1)) for k in keys})
    return out


@pytest.mark.parametrize("which", ["adamw", "adam", "sgd", "sgd_nesterov"])
def test_dropin_optimizers4_match_oracle_every_step(which):
    from gpu_helpers import check_state
    from precision_optimizer_state_amd import FlashAdam, FlashAdamW, FlashSGD
    model = _model(5)
    params = list(model.parameters())
    if which in ("adamw", "adam"):
        cls = FlashAdamW if which == "adamw" else FlashAdam
        opt = cls(params, lr=3e-3, betas=(0.9, 0.95), eps=1e-8, weight_decay=0.1, codec=C4)
        hp = dict(lr=3e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, l2_decay=which == "adam")
        keys, step_fn = ("m_q", "m_s", "v_q", "v_s"), O.adamw_step
    else:
        kw = dict(lr=0.05, momentum=0.9, weight_decay=1e-4, nesterov=which == "sgd_nesterov")
        opt = FlashSGD(params, codec=C4, **kw)
        hp = kw
        keys, step_fn = ("b_q", "b_s"), O.sgdm_step
    for p in params:
        assert opt.state[p][keys[0]].numel() == (p.numel() + 1) // 2
    for step in range(1, 5):
        opt.zero_grad(set_to_none=True)
        _loss(model, step).backward()
        grads = [to_host(p.grad.view(-1)) for p in params]
        before = [_host(opt, p, keys) for p in params]
        opt.step()
        torch.cuda.synchronize()
        for i, p in enumerate(params):
            want = step_fn(before[i], grads[i], dict(hp, step=step), "bf16", 8, C4)
            check_state(f"{which} 4-bit step {step} param {i}", _host(opt, p, keys), want)


def test_dropin4_gradient_release_and_state_round_trip():
    from precision_optimizer_state_amd import FlashAdamW
    a, b = _model(6), _model(6)
    oa = FlashAdamW(a.parameters(), lr=3e-3, codec=C4)
    ob = FlashAdamW(b.parameters(), lr=3e-3, codec=C4, grad_release=True, release_bucket=5000)
    for m, o in ((a, oa), (b, ob)):
        for step in range(1, 4):
            o.zero_grad(set_to_none=True)
            _loss(m, step).backward()
            o.step()
    torch.cuda.synchronize()
    for pa, pb in zip(a.parameters(), b.parameters()):
        assert torch.equal(pa.data.view(torch.int16), pb.data.view(torch.int16))
        for k in ("ecc", "m_q", "m_s", "v_q", "v_s"):
            assert torch.equal(oa.state[pa][k].view(torch.uint8), ob.state[pb][k].view(torch.uint8)), k
    # export decodes the stored codes as the oracle does; import encodes f32
    # moments as the oracle does
    for p in a.parameters():
        n = p.numel()
        m, v = oa.export_torch_state(p)
        for got, k, kind in ((m, "m", True), (v, "v", False)):
            q = O.unpack_nibbles(to_host(oa.state[p][k + "_q"]), n, kind)
            want = O.dequantize_state(q, to_host(oa.state[p][k + "_s"]), k, C4)
            assert np.array_equal(got.cpu().numpy().ravel().view(np.uint32), want.view(np.uint32))
        em = torch.randn(p.shape, device="cuda") * 1e-3
        ev = torch.rand(p.shape, device="cuda") * 1e-6
        oa.import_torch_state(p, em, ev, 9)
        for x, k in ((em, "m"), (ev, "v")):
            q, sc = O.quantize_state(x.cpu().numpy().ravel(), k, C4)
            assert np.array_equal(to_host(oa.state[p][k + "_q"]), O.pack_nibbles(q))
            assert np.array_equal(to_host(oa.state[p][k + "_s"]), sc)
