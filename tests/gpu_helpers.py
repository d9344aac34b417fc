"""Shared helpers of the GPU parity tests: host<->device conversion of state
arrays and the acceptance bar.

Acceptance bar (per step, per array): codes, ECCs and 16-bit weights
identical on >= 99.99% of elements and within one unit on the rest
(for (theta', rho) pairs: adjacent in the ordered (theta', rho) sequence,
i.e. reconstructed masters within one ECC step); block scales identical on
>= 99.99% of blocks.  The kernels take every decision in the same float32
operations as the oracle, so the expected mismatch count is zero; the
tests print it.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle as O

FRACTION = 0.9999


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


def adamw_state_to_host(st: dict) -> dict:
    return {k: to_host(st[k]) for k in ("w16", "ecc", "m_q", "m_s", "v_q", "v_s")}


def sgdm_state_to_host(st: dict) -> dict:
    return {k: to_host(st[k]) for k in ("w16", "ecc", "b_q", "b_s")}


def _frac_equal(a, b):
    if a.size == 0:
        return 1.0, 0
    eq = a == b
    return float(np.mean(eq)), int(a.size - np.count_nonzero(eq))


def check_codes(name, got, want, lsb=1):
    f, bad = _frac_equal(got, want)
    assert f >= FRACTION, f"{name}: identical on {f:.6f} ({bad} differ)"
    if bad:
        d = np.abs(got.astype(np.int64) - want.astype(np.int64))
        assert d.max() <= lsb, f"{name}: max code difference {d.max()}"
    return bad


def check_weights(name, w_got, e_got, w_want, e_want, fmt, ecc_bits):
    eq = (w_got == w_want) & (e_got == e_want)
    f = float(np.mean(eq)) if eq.size else 1.0
    bad = int(eq.size - np.count_nonzero(eq))
    assert f >= FRACTION, f"{name}: (theta', rho) identical on {f:.6f} ({bad} differ)"
    if bad:
        idx = ~eq
        xg = O.reconstruct_weights(w_got[idx], e_got[idx], fmt, ecc_bits).astype(np.float64)
        xw = O.reconstruct_weights(w_want[idx], e_want[idx], fmt, ecc_bits).astype(np.float64)
        from oracle.numerics import bits_to_value, spacing_out
        a = np.abs(bits_to_value(w_want[idx], fmt))
        step = spacing_out(a, fmt) * 2.0 ** -ecc_bits
        assert np.all(np.abs(xg - xw) <= step * (1 + 1e-9)), f"{name}: differing masters more than one ECC step apart"
    return bad


def check_adamw_state(tag, got: dict, want: dict, fmt="bf16", ecc_bits=8):
    bad = {}
    bad["w"] = check_weights(f"{tag} w16/ecc", got["w16"], got["ecc"], want["w16"], want["ecc"], fmt, ecc_bits)
    bad["m_q"] = check_codes(f"{tag} m_q", got["m_q"], want["m_q"])
    bad["v_q"] = check_codes(f"{tag} v_q", got["v_q"], want["v_q"])
    bad["m_s"] = check_codes(f"{tag} m_s", got["m_s"], want["m_s"], lsb=1)
    bad["v_s"] = check_codes(f"{tag} v_s", got["v_s"], want["v_s"], lsb=1)
    return bad


def check_sgdm_state(tag, got: dict, want: dict, fmt="bf16", ecc_bits=8):
    bad = {}
    bad["w"] = check_weights(f"{tag} w16/ecc", got["w16"], got["ecc"], want["w16"], want["ecc"], fmt, ecc_bits)
    bad["b_q"] = check_codes(f"{tag} b_q", got["b_q"], want["b_q"])
    bad["b_s"] = check_codes(f"{tag} b_s", got["b_s"], want["b_s"], lsb=1)
    return bad
