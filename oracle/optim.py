"""Oracle: the fused optimizer step (AdamW and momentum SGD) over split weights
and companded states.

TEST INFRASTRUCTURE ONLY -- see the package docstring for who may import it.

What the pages fix: FlashOptim's optimizers compute the same updates as the
usual torch.optim ones while storing less (FlashOptim thread, Davis Blalock,
the launch post and the post on doing the same updates; blog "FlashOptim:
Breaking the Memory Wall ...", Conclusion & Perspective: drop-in replacements
for torch.optim).  Gradients stay in the backward pass's 16-bit precision
(thread, the post on gradients).  The pages print no update equations, so the
textbook AdamW / SGD-with-momentum definitions are used.

Readings:

U1  AdamW = torch.optim.AdamW defaults: decoupled weight decay, bias
    correction, step t counted from 1, amsgrad off.  The update uses the fresh
    float32 m and v (before they are re-quantised).
U2  Host scalars are computed in float64 and rounded once to float32:
    b1, b2, 1-b1, 1-b2, decay = 1 - lr*wd, step_size = lr / (1 - b1^t),
    ibc2 = 1 / sqrt(1 - b2^t), eps.
U3  Per-element float32 operation order, every operation rounded once (no
    fused multiply-add; the division and the square root are the correctly
    rounded IEEE operations):
        m = b1*m + (1-b1)*g
        v = b2*v + (1-b2)*(g*g)
        theta = theta*decay
        d = sqrt(v)*ibc2 + eps
        theta = theta - step_size*(m/d)
    The quotient m/d of the textbook update is one IEEE division (rounded
    once), then scaled by the bias-corrected step size and subtracted.
U4  SGD-M = torch.optim.SGD: coupled L2 weight decay, optional dampening and
    Nesterov:  d = g + wd*theta;  b = d at step 1, else b = mu*b + (1-damp)*d;
    u = d + mu*b (Nesterov) or u = b;  theta = theta - lr*u.  With dampening 0
    (1 - damp = 1 exactly) the buffer update is mu*b + d.  With momentum 0
    torch keeps no buffer and steps theta -= lr*d at every step, dampening
    unused; here every step then takes the step-1 rule b = d (so u = d), and
    the stored buffer holds d, which the next step ignores.
U5  The momentum buffer of SGD-M uses the momentum codec.
U6  Adam with coupled L2 weight decay (torch.optim.Adam): g = g + wd*theta
    (theta = the reconstructed master) before the moments; no decoupled
    decay (decay = 1); otherwise as U3.

Parity status: pinned (unquantised update against torch.optim.AdamW, Adam
with weight decay (U6) and SGD (plain, Nesterov, dampening, momentum 0 with
dampening) in float64 and a float64 textbook loop; the update's quotient
against the exact rational m/d rounded once, on inputs where a
reciprocal-multiply rounds differently; bf16+16 ECC reproduces a plain
float32 master bit for bit; first-step closed form;
tests/test_oracle_optim.py).
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

from .codecs import (
    block_scales,
    code_bytes,
    decode_momentum,
    decode_variance,
    encode_momentum,
    encode_variance,
    pack_nibbles,
    unpack_nibbles,
)
from .numerics import bf16_bits_to_f32, f16_bits_to_f32, reconstruct_weights, split_weights

F32 = np.float32


@dataclass(frozen=True)
class AdamWScalars:
    b1: np.float32
    b2: np.float32
    omb1: np.float32
    omb2: np.float32
    decay: np.float32
    step_size: np.float32
    ibc2: np.float32
    eps: np.float32
    wd: np.float32 = F32(0.0)      # coupled decay (U6); 0 for AdamW
    l2: bool = False


@dataclass(frozen=True)
class SGDMScalars:
    lr: np.float32
    mu: np.float32
    wd: np.float32
    damp1: np.float32 = F32(1.0)   # 1 - dampening
    nesterov: bool = False


def adamw_scalars(lr: float, beta1: float, beta2: float, eps: float, weight_decay: float, step: int,
                  l2: bool = False) -> AdamWScalars:
    """U2: float64 -> one float32 rounding each.  l2 selects U6 (Adam)."""
    if step < 1:
        raise ValueError("step counts from 1")
    bc1 = 1.0 - beta1 ** step
    bc2 = 1.0 - beta2 ** step
    return AdamWScalars(
        b1=F32(beta1), b2=F32(beta2), omb1=F32(1.0 - beta1), omb2=F32(1.0 - beta2),
        decay=F32(1.0) if l2 else F32(1.0 - lr * weight_decay), step_size=F32(lr / bc1),
        ibc2=F32(1.0 / math.sqrt(bc2)), eps=F32(eps), wd=F32(weight_decay) if l2 else F32(0.0), l2=l2,
    )


def sgdm_scalars(lr: float, momentum: float, weight_decay: float, dampening: float = 0.0,
                 nesterov: bool = False) -> SGDMScalars:
    return SGDMScalars(lr=F32(lr), mu=F32(momentum), wd=F32(weight_decay), damp1=F32(1.0 - dampening),
                       nesterov=bool(nesterov))


def adamw_update(theta, g, m, v, S: AdamWScalars):
    """U3 on float32 arrays.  Returns (theta, m, v, sqrt(v))."""
    theta = np.asarray(theta, F32); g = np.asarray(g, F32)
    m = np.asarray(m, F32); v = np.asarray(v, F32)
    with np.errstate(all="ignore"):
        if S.l2:
            g = g + S.wd * theta
        m1 = S.b1 * m + S.omb1 * g
        v1 = S.b2 * v + S.omb2 * (g * g)
        th = theta * S.decay
        w = np.sqrt(v1)
        d = w * S.ibc2 + S.eps
        th = th - S.step_size * (m1 / d)
    return th.astype(F32), m1.astype(F32), v1.astype(F32), w.astype(F32)


def sgdm_first(step: int, momentum: float) -> bool:
    """U4: the buffer is set to d at step 1 and, with momentum 0, at every step."""
    return step == 1 or momentum == 0.0


def sgdm_update(theta, g, b, S: SGDMScalars, first: bool = False):
    """U4 on float32 arrays.  Returns (theta, b)."""
    theta = np.asarray(theta, F32); g = np.asarray(g, F32); b = np.asarray(b, F32)
    with np.errstate(all="ignore"):
        d = g + S.wd * theta
        b1 = d if first else S.mu * b + S.damp1 * d
        u = d + S.mu * b1 if S.nesterov else b1
        th = theta - S.lr * u
    return th.astype(F32), b1.astype(F32)


def widen_grad(grad_bits: np.ndarray, fmt: str) -> np.ndarray:
    """16-bit gradient pattern -> float32 (exact)."""
    return bf16_bits_to_f32(grad_bits) if fmt == "bf16" else f16_bits_to_f32(grad_bits)


def _stored_codes(stored: np.ndarray, n: int, codec: str, signed: bool) -> np.ndarray:
    """A state's code array as stored -> one code per element (C8 packs two
    4-bit codes a byte)."""
    if codec == "companded4":
        return unpack_nibbles(stored, n, signed)
    return np.asarray(stored).ravel()


def _stored_form(q: np.ndarray, codec: str) -> np.ndarray:
    """One code per element -> the state's code array as stored."""
    if codec == "companded4":
        return pack_nibbles(q)
    return q


def adamw_step(state: dict, grad_bits: np.ndarray, hp: dict, fmt: str = "bf16",
               ecc_bits: int = 8, codec: str = "companded") -> dict:
    """One fused AdamW step on one tensor.

    state: {"w16": uint16, "ecc": int8|int16, "m_q": int8, "m_s": uint16 (fp16 bits),
            "v_q": uint8, "v_s": uint16}; hp: lr, beta1, beta2, eps, weight_decay, step.
    With codec "companded4" m_q and v_q are the nibble-packed uint8 arrays.
    Returns the new state (same keys).  Steps: widen grad, reconstruct master,
    decode states, update (U3), split, block scales, encode.
    """
    S = adamw_scalars(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"], hp["step"],
                      l2=hp.get("l2_decay", False))
    theta = reconstruct_weights(state["w16"], state["ecc"], fmt, ecc_bits)
    n = theta.size
    g = widen_grad(grad_bits, fmt)
    m = decode_momentum(_stored_codes(state["m_q"], n, codec, True), state["m_s"], codec)
    v = decode_variance(_stored_codes(state["v_q"], n, codec, False), state["v_s"], codec)
    th, m1, v1, _ = adamw_update(theta, g, m, v, S)
    w16, ecc = split_weights(th, fmt, ecc_bits)
    m_s = block_scales(m1, "m", codec)
    v_s = block_scales(v1, "v", codec)
    return {
        "w16": w16, "ecc": ecc,
        "m_q": _stored_form(encode_momentum(m1, m_s, codec), codec), "m_s": m_s,
        "v_q": _stored_form(encode_variance(v1, v_s, codec), codec), "v_s": v_s,
    }


def sgdm_step(state: dict, grad_bits: np.ndarray, hp: dict, fmt: str = "bf16",
              ecc_bits: int = 8, codec: str = "companded") -> dict:
    """One fused SGD-with-momentum step on one tensor.

    state: {"w16", "ecc", "b_q": int8, "b_s": uint16}; hp: lr, momentum, weight_decay,
    optional dampening, nesterov and step (step 1 sets the buffer to d).
    """
    S = sgdm_scalars(hp["lr"], hp["momentum"], hp["weight_decay"], hp.get("dampening", 0.0),
                     hp.get("nesterov", False))
    theta = reconstruct_weights(state["w16"], state["ecc"], fmt, ecc_bits)
    g = widen_grad(grad_bits, fmt)
    b = decode_momentum(_stored_codes(state["b_q"], theta.size, codec, True), state["b_s"], codec)
    th, b1 = sgdm_update(theta, g, b, S, first=sgdm_first(hp["step"], hp["momentum"]))
    w16, ecc = split_weights(th, fmt, ecc_bits)
    b_s = block_scales(b1, "m", codec)
    return {"w16": w16, "ecc": ecc, "b_q": _stored_form(encode_momentum(b1, b_s, codec), codec), "b_s": b_s}


def fresh_adamw_state(x32: np.ndarray, fmt: str = "bf16", ecc_bits: int = 8, codec: str = "companded") -> dict:
    """Split an f32 weight and attach zero states (zero codes and zero scales
    decode to exactly 0)."""
    w16, ecc = split_weights(x32, fmt, ecc_bits)
    n = w16.size
    nb = -(-n // 32)
    qt = np.uint8 if codec == "companded4" else np.int8
    return {"w16": w16, "ecc": ecc,
            "m_q": np.zeros(code_bytes(n, codec), qt), "m_s": np.zeros(nb, np.uint16),
            "v_q": np.zeros(code_bytes(n, codec), np.uint8), "v_s": np.zeros(nb, np.uint16)}


def fresh_sgdm_state(x32: np.ndarray, fmt: str = "bf16", ecc_bits: int = 8, codec: str = "companded") -> dict:
    w16, ecc = split_weights(x32, fmt, ecc_bits)
    n = w16.size
    qt = np.uint8 if codec == "companded4" else np.int8
    return {"w16": w16, "ecc": ecc,
            "b_q": np.zeros(code_bytes(n, codec), qt), "b_s": np.zeros(-(-n // 32), np.uint16)}
