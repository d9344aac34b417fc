"""GPU parity from arbitrary stored states (through the C ABI).

The other parity tests start from zero states and only ever decode codes that
the encoder wrote.  Here the stored codes and block scales are random: every
int8 momentum code (including -128, which the encoder never writes), every
uint8 variance code, and fp16 scales from zero through subnormals to large
normals.  Decoding then covers the whole code space, and the steps run from a
late step count.
"""

import numpy as np
import pytest
import torch

import oracle as O
from oracle.numerics import split_weights
from precision_optimizer_state_amd import binding as B
from precision_optimizer_state_amd.state import alloc_adamw_state, alloc_sgdm_state
from tests.gpu_helpers import run_lockstep, to_dev
from workloads import host_grad_bits, host_grads, host_weights

pytestmark = pytest.mark.gpu
DT = {"bf16": torch.bfloat16, "fp16": torch.float16}
SIZES = [1, 31, 33, 2048, 4097, 20000]


def _random_codes(rng, n):
    nb = -(-n // 32)
    m_q = rng.integers(-128, 128, n).astype(np.int8)
    m_q[: min(n, 256)] = np.arange(-128, 128, dtype=np.int64)[: min(n, 256)].astype(np.int8)
    v_q = rng.integers(0, 256, n).astype(np.uint8)
    m_s = rng.integers(0, 0x5800, nb).astype(np.uint16)
    v_s = rng.integers(0, 0x5000, nb).astype(np.uint16)
    m_s[::7] = 0
    v_s[::5] = 0
    return m_q, m_s, v_q, v_s


@pytest.mark.parametrize("codec", ["companded", "linear"])
def test_dequantize_every_momentum_code(codec):
    rng = np.random.default_rng(5)
    nb = 64
    codes = np.tile(np.arange(-128, 128, dtype=np.int64).astype(np.int8), nb // 8)
    scales = rng.integers(0, 0x7C00, nb).astype(np.uint16)
    scales[:3] = [0x0000, 0x0001, 0x3C00]
    out = torch.empty(codes.size, dtype=torch.float32, device="cuda")
    B.fo_dequantize(to_dev(codes, torch.int8), to_dev(scales, torch.float16), out, "m", codec)
    torch.cuda.synchronize()
    want = O.decode_momentum(codes, scales, codec)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("fmt,ecc_bits,codec", [("bf16", 8, "companded"), ("bf16", 16, "companded"),
                                                ("fp16", 8, "companded"), ("bf16", 8, "linear")])
@pytest.mark.parametrize("l2", [False, True])
def test_fused_adam_from_arbitrary_states(fmt, ecc_bits, codec, l2):
    rng = np.random.default_rng(17)
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    dev = []
    for i, n in enumerate(SIZES):
        w16, ecc = split_weights(host_weights("arb", i, n), fmt, ecc_bits)
        m_q, m_s, v_q, v_s = _random_codes(rng, n)
        d = alloc_adamw_state(n, fmt, ecc_bits)
        d["w16"].copy_(to_dev(w16, DT[fmt]))
        d["ecc"].copy_(to_dev(ecc, d["ecc"].dtype))
        d["m_q"].copy_(to_dev(m_q, torch.int8))
        d["v_q"].copy_(to_dev(v_q, torch.uint8))
        d["m_s"].copy_(to_dev(m_s, torch.float16))
        d["v_s"].copy_(to_dev(v_s, torch.float16))
        dev.append(d)
    run_lockstep("adamw", dev, 0,
                 lambda i, step: host_grad_bits(host_grads("arb", i, step, SIZES[i], "t3"), fmt),
                 dict(hp, l2_decay=l2), fmt, ecc_bits, codec, f"arbitrary {fmt}/{ecc_bits}/{codec} l2={l2}",
                 step_list=(7, 8, 9))


@pytest.mark.parametrize("fmt,ecc_bits,codec", [("bf16", 8, "companded"), ("fp16", 8, "companded"),
                                                ("bf16", 8, "linear")])
@pytest.mark.parametrize("nesterov,dampening", [(False, 0.0), (True, 0.0), (False, 0.3)])
def test_fused_sgd_from_arbitrary_states(fmt, ecc_bits, codec, nesterov, dampening):
    rng = np.random.default_rng(23)
    hp = dict(lr=0.05, momentum=0.9, weight_decay=1e-4, dampening=dampening, nesterov=nesterov)
    dev = []
    for i, n in enumerate(SIZES):
        w16, ecc = split_weights(host_weights("arbs", i, n), fmt, ecc_bits)
        b_q, b_s, _, _ = _random_codes(rng, n)
        d = alloc_sgdm_state(n, fmt, ecc_bits)
        d["w16"].copy_(to_dev(w16, DT[fmt]))
        d["ecc"].copy_(to_dev(ecc, d["ecc"].dtype))
        d["b_q"].copy_(to_dev(b_q, torch.int8))
        d["b_s"].copy_(to_dev(b_s, torch.float16))
        dev.append(d)
    run_lockstep("sgdm", dev, 0,
                 lambda i, step: host_grad_bits(host_grads("arbs", i, step, SIZES[i], "t3"), fmt),
                 hp, fmt, ecc_bits, codec, f"arbitrary sgd {fmt}/{codec} nesterov={nesterov} damp={dampening}",
                 step_list=(4, 5))
