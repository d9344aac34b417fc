"""Shared helpers of the GPU parity tests: host<->device conversion of state
arrays, the lock-step runner and the acceptance checks.

Lock-step: before every GPU step the test copies the device state to the
host, the oracle steps that copy with the same gradient and hyperparameters,
and the result is compared with the device state after its step.  Each step
is therefore checked on its own, from identical inputs, and a difference can
never compound.

Acceptance: the kernels take every decision with the oracle's float32
operations (exact fast arithmetic, verified on the device), so the tests
require bitwise equality of every array: 16-bit weights, ECCs, codes and
block scales.  (The stated bar of the task -- identical on >= 99.99% of
elements, within one unit on the rest -- is implied.)  NaN weights are
compared as NaN: the position must match, the payload may differ.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle as O


def to_host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> NumPy array with the oracle's dtypes (16-bit patterns as uint16)."""
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def to_dev(a: np.ndarray, dtype, device="cuda") -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if dtype in (torch.bfloat16, torch.float16):
        return torch.from_numpy(a.view(np.int16)).to(device).view(dtype)
    return torch.from_numpy(a).to(device)


ADAMW_KEYS = ("w16", "ecc", "m_q", "m_s", "v_q", "v_s")
SGDM_KEYS = ("w16", "ecc", "b_q", "b_s")


def adamw_state_to_host(st: dict) -> dict:
    return {k: to_host(st[k]) for k in ADAMW_KEYS}


def sgdm_state_to_host(st: dict) -> dict:
    return {k: to_host(st[k]) for k in SGDM_KEYS}


def _mismatches(a, b) -> int:
    return int(a.size - np.count_nonzero(a == b)) if a.size else 0


def check_codes(name, got, want):
    bad = _mismatches(got, want)
    if bad:
        idx = np.nonzero(got != want)[0][:8]
        raise AssertionError(f"{name}: {bad} of {got.size} differ; first at {list(idx)}: "
                             f"got {list(got[idx])}, want {list(want[idx])}")
    return 0


def check_weights(name, w_got, e_got, w_want, e_want, fmt, ecc_bits):
    nan = np.isnan(O.reconstruct_weights(w_want, e_want, fmt, ecc_bits))
    nan_got = np.isnan(O.reconstruct_weights(w_got, e_got, fmt, ecc_bits))
    assert np.array_equal(nan, nan_got), f"{name}: NaN weights at different elements"
    check_codes(f"{name} w16", np.where(nan, w_want, w_got), w_want)
    check_codes(f"{name} ecc", e_got, e_want)
    return 0


def check_state(tag, got: dict, want: dict, fmt="bf16", ecc_bits=8):
    check_weights(f"{tag} w16/ecc", got["w16"], got["ecc"], want["w16"], want["ecc"], fmt, ecc_bits)
    for k in got:
        if k not in ("w16", "ecc"):
            check_codes(f"{tag} {k}", got[k], want[k])


def run_lockstep(kind, dev, steps, grads, hp, fmt="bf16", ecc_bits=8, codec="companded", tag="t",
                 step_list=None):
    """Lock-step GPU vs oracle.

    kind: "adamw" (AdamW, or Adam with hp["l2_decay"]) or "sgdm".
    dev: list of device states (dicts of tensors, grads included), initialised.
    grads(i, step) -> the 16-bit gradient bit pattern of tensor i at `step`.
    Runs steps 1..steps (or the steps of step_list) and checks every tensor
    after every step; returns the number of (tensor, step) checks made.
    """
    from precision_optimizer_state_amd import binding as B
    dtype = {"bf16": torch.bfloat16, "fp16": torch.float16}[fmt]
    adam = kind == "adamw"
    host_state = adamw_state_to_host if adam else sgdm_state_to_host
    tl = B.AdamWList(dev) if adam else B.SGDMList(dev)
    checks = 0
    for step in (step_list if step_list is not None else range(1, steps + 1)):
        torch.cuda.synchronize()
        before = [host_state(st) for st in dev]
        gbs = []
        for i, st in enumerate(dev):
            gb = grads(i, step)
            gbs.append(gb)
            if st["w16"].numel():
                st["grad"].copy_(to_dev(gb, dtype))
        if adam:
            B.fo_fused_adamw_step(tl, B.adamw_hparams(step=step, wfmt=fmt, ecc_bits=ecc_bits, codec=codec, **hp))
        else:
            B.fo_fused_sgdm_step(tl, B.sgdm_hparams(step=step, wfmt=fmt, ecc_bits=ecc_bits, codec=codec, **hp))
        torch.cuda.synchronize()
        for i, st in enumerate(dev):
            if not st["w16"].numel():
                continue
            if adam:
                want = O.adamw_step(before[i], gbs[i], dict(hp, step=step), fmt, ecc_bits, codec)
            else:
                want = O.sgdm_step(before[i], gbs[i], dict(hp, step=step), fmt, ecc_bits, codec)
            check_state(f"{tag} step {step} tensor {i} (n={st['w16'].numel()})", host_state(st), want,
                        fmt, ecc_bits)
            checks += 1
    return checks
