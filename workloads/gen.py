"""Seeded input generators (host NumPy and device torch).

Recipe (per tensor of a config, per step):
  * weights: float32 ~ N(0, 0.02);
  * gradients: "t3" Student-t(3) * 1e-3; "t3_lognormal" the same times a
    per-tensor lognormal(0, 1) scale drawn once from the config seed;
    "normal_outliers" N(0, 1e-2) with 1% Bernoulli outliers * 100;
    a new seed every step; cast to the 16-bit format with torch's
    round-to-nearest-even conversion.
Seeds derive from numpy.random.SeedSequence(20261203) keyed by (config,
tensor index, step, stream kind).  The host and device generators draw
different streams from the same seeds; a test compares a host-generated run
with the oracle on host inputs, or copies device-generated inputs back.
"""

from __future__ import annotations

import zlib

import numpy as np
import torch

ROOT_SEED = 20261203
_KINDS = {"w": 1, "g": 2, "scale": 3, "misc": 4}


def seed_for(config: str, tensor: int, step: int, kind: str) -> int:
    ss = np.random.SeedSequence([ROOT_SEED, zlib.crc32(config.encode()), tensor, step, _KINDS[kind]])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & np.uint64(2 ** 62 - 1))


def _tensor_scale(config: str, tensor: int, grad_kind: str) -> float:
    if grad_kind != "t3_lognormal":
        return 1.0
    return float(np.random.default_rng(seed_for(config, tensor, 0, "scale")).lognormal(0.0, 1.0))


def host_weights(config: str, tensor: int, n: int) -> np.ndarray:
    rng = np.random.default_rng(seed_for(config, tensor, 0, "w"))
    return (rng.standard_normal(n, dtype=np.float32) * np.float32(0.02)).astype(np.float32)


def host_grads(config: str, tensor: int, step: int, n: int, grad_kind: str) -> np.ndarray:
    rng = np.random.default_rng(seed_for(config, tensor, step, "g"))
    if grad_kind in ("t3", "t3_lognormal"):
        g = rng.standard_t(3, n) * 1e-3 * _tensor_scale(config, tensor, grad_kind)
    elif grad_kind == "normal_outliers":
        g = rng.normal(0.0, 1e-2, n)
        g = np.where(rng.random(n) < 0.01, g * 100.0, g)
    else:
        raise ValueError(grad_kind)
    return g.astype(np.float32)


def host_grad_bits(g32: np.ndarray, wfmt: str) -> np.ndarray:
    """16-bit pattern of the gradient (torch's RNE cast, as a backward pass)."""
    dt = torch.bfloat16 if wfmt == "bf16" else torch.float16
    return torch.from_numpy(np.ascontiguousarray(g32)).to(dt).view(torch.int16).numpy().view(np.uint16)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def device_weights(config: str, tensor: int, n: int, device="cuda", out=None) -> torch.Tensor:
    gen = _gen(seed_for(config, tensor, 0, "w"), device)
    w = torch.randn(n, generator=gen, device=device, dtype=torch.float32) if out is None else \
        torch.randn(n, generator=gen, device=device, dtype=torch.float32, out=out)
    return w.mul_(0.02)


def device_grads(config: str, tensor: int, step: int, n: int, grad_kind: str, wfmt: str,
                 device="cuda", out=None, chunk: int = 1 << 27) -> torch.Tensor:
    """16-bit gradients generated on the device in chunks (bounded scratch)."""
    dt = torch.bfloat16 if wfmt == "bf16" else torch.float16
    if out is None:
        out = torch.empty(n, dtype=dt, device=device)
    gen = _gen(seed_for(config, tensor, step, "g"), device)
    scale = _tensor_scale(config, tensor, grad_kind)
    for s in range(0, n, chunk):
        m = min(chunk, n - s)
        if grad_kind in ("t3", "t3_lognormal"):
            z = torch.randn(4, m, generator=gen, device=device, dtype=torch.float32)
            chi2 = (z[1:] * z[1:]).sum(0)
            g = z[0] / torch.sqrt(chi2 / 3.0) * (1e-3 * scale)
        else:
            g = torch.randn(m, generator=gen, device=device, dtype=torch.float32) * 1e-2
            u = torch.rand(m, generator=gen, device=device)
            g = torch.where(u < 0.01, g * 100.0, g)
        out[s:s + m] = g.to(dt)
    return out
