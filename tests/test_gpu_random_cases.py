"""Seeded random cases through the C ABI against the oracle: random tensor
lists (sizes 0 to 200K, ragged tails, empty tensors), every weight format /
ECC / codec combination, AdamW, Adam (L2) and SGD-M (plain, Nesterov,
dampening) with hyperparameters drawn across their ranges, 2-3 free-running
steps each.  Every case must be identical to the oracle on >= 99.99% of
elements and within one LSB / one ECC step on the rest."""

import numpy as np
import pytest
import torch

import oracle as O
from oracle.optim import fresh_adamw_state, fresh_sgdm_state
from precision_optimizer_state_amd import binding as B
from precision_optimizer_state_amd.state import alloc_adamw_state, alloc_sgdm_state
from tests.gpu_helpers import adamw_state_to_host, check_adamw_state, check_sgdm_state, sgdm_state_to_host, to_dev
from workloads import host_grad_bits, host_grads, host_weights

pytestmark = pytest.mark.gpu

DT = {"bf16": torch.bfloat16, "fp16": torch.float16}
FORMATS = [("bf16", 8), ("bf16", 16), ("fp16", 8)]
N_CASES = 120


def _case(i):
    rng = np.random.default_rng([777, i])
    fmt, ecc = FORMATS[rng.integers(len(FORMATS))]
    codec = ["companded", "linear"][int(rng.random() < 0.3)]
    count = int(rng.integers(1, 7))
    sizes = [int(rng.choice([0, 1, 31, 32, 33, 2047, 2048, 2049])) if rng.random() < 0.3
             else int(rng.integers(1, 200_000)) for _ in range(count)]
    if not any(sizes):
        sizes[0] = 4099
    kind = ["adamw", "adam_l2", "sgd"][int(rng.integers(3))]
    if kind == "sgd":
        nest = bool(rng.random() < 0.3)
        hp = dict(lr=float(10 ** rng.uniform(-3, -0.5)), momentum=float(rng.uniform(0.5, 0.99)),
                  weight_decay=float(rng.choice([0.0, 1e-4, 1e-2])),
                  dampening=0.0 if nest else float(rng.choice([0.0, 0.0, 0.1, 0.9])), nesterov=nest)
    else:
        hp = dict(lr=float(10 ** rng.uniform(-4, -2)), beta1=float(rng.choice([0.0, 0.8, 0.9, 0.95])),
                  beta2=float(rng.choice([0.9, 0.95, 0.99, 0.999])), eps=float(10 ** rng.uniform(-10, -6)),
                  weight_decay=float(rng.choice([0.0, 0.01, 0.1])), l2_decay=(kind == "adam_l2"))
    steps = int(rng.integers(2, 4))
    grad_kind = ["t3", "normal_outliers"][int(rng.integers(2))]
    return fmt, ecc, codec, sizes, kind, hp, steps, grad_kind


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case_matches_oracle(i):
    fmt, ecc, codec, sizes, kind, hp, steps, grad_kind = _case(i)
    tag = f"rand{i}"
    print(f"case {i}: {kind} {fmt}+{ecc} {codec} sizes={sizes} steps={steps} hp={hp}", flush=True)
    adam = kind != "sgd"
    xs = [host_weights(tag, j, n) for j, n in enumerate(sizes)]
    dev = [(alloc_adamw_state if adam else alloc_sgdm_state)(n, fmt, ecc) for n in sizes]
    ref = [(fresh_adamw_state if adam else fresh_sgdm_state)(x, fmt, ecc) for x in xs]
    for st, x in zip(dev, xs):
        B.fo_split_weights(torch.from_numpy(x).cuda(), st["w16"], st["ecc"], fmt, ecc)
    tl = B.AdamWList(dev) if adam else B.SGDMList(dev)
    for step in range(1, steps + 1):
        gbs = []
        for j, (st, n) in enumerate(zip(dev, sizes)):
            gb = host_grad_bits(host_grads(tag, j, step, n, grad_kind), fmt)
            gbs.append(gb)
            st["grad"].copy_(to_dev(gb, DT[fmt]))
        if adam:
            B.fo_fused_adamw_step(tl, B.adamw_hparams(step=step, wfmt=fmt, ecc_bits=ecc, codec=codec, **hp))
        else:
            B.fo_fused_sgdm_step(tl, B.sgdm_hparams(step=step, wfmt=fmt, ecc_bits=ecc, codec=codec, **hp))
        for j in range(len(sizes)):
            if sizes[j] == 0:
                continue
            if adam:
                ref[j] = O.adamw_step(ref[j], gbs[j], dict(hp, step=step), fmt, ecc, codec)
            else:
                ref[j] = O.sgdm_step(ref[j], gbs[j], dict(hp, step=step), fmt, ecc, codec)
    torch.cuda.synchronize()
    bad = 0
    for j in range(len(sizes)):
        if sizes[j] == 0:
            continue
        if adam:
            b = check_adamw_state(f"case {i} tensor {j}", adamw_state_to_host(dev[j]), ref[j], fmt, ecc)
        else:
            b = check_sgdm_state(f"case {i} tensor {j}", sgdm_state_to_host(dev[j]), ref[j], fmt, ecc)
        bad += sum(b.values())
    print(f"case {i}: {bad} mismatching elements", flush=True)
