"""Device storage for split weights and 8-bit (or 4-bit) optimizer states.

Per parameter of n elements (AdamW, bf16/fp16 + 8-bit ECC):
    w16 n*2 B, ecc n*1 B, grad n*2 B, m_q n B, v_q n B, m_s and v_s 2*ceil(n/32) B
= 7.125 bytes per parameter (the pages' 16 -> 7 bytes per parameter, plus the
16-bit scales of the 32-element blocks).  With 4-bit codes (codec
"companded4") m_q and v_q hold ceil(n/2) bytes each: 6.125 bytes per
parameter.  Codes and scales start at zero, which decodes to exactly zero
states.
"""

from __future__ import annotations

import torch

_W16 = {"bf16": torch.bfloat16, "fp16": torch.float16}
_ECC = {8: torch.int8, 16: torch.int16}


def nblocks(n: int) -> int:
    return (n + 31) // 32


def code_bytes(n: int, codec: str = "companded") -> int:
    """Bytes of one state's code array: n, or ceil(n/2) for 4-bit codes."""
    return (n + 1) // 2 if codec == "companded4" else n


def alloc_adamw_state(n: int, wfmt: str = "bf16", ecc_bits: int = 8, device="cuda", with_grad: bool = True,
                      codec: str = "companded") -> dict:
    nb = nblocks(n)
    nq = code_bytes(n, codec)
    st = {
        "w16": torch.empty(n, dtype=_W16[wfmt], device=device),
        "ecc": torch.empty(n, dtype=_ECC[ecc_bits], device=device),
        "m_q": torch.zeros(nq, dtype=torch.uint8 if codec == "companded4" else torch.int8, device=device),
        "m_s": torch.zeros(nb, dtype=torch.float16, device=device),
        "v_q": torch.zeros(nq, dtype=torch.uint8, device=device),
        "v_s": torch.zeros(nb, dtype=torch.float16, device=device),
    }
    st["grad"] = torch.zeros(n, dtype=_W16[wfmt], device=device) if with_grad else None
    return st


def alloc_sgdm_state(n: int, wfmt: str = "bf16", ecc_bits: int = 8, device="cuda", with_grad: bool = True,
                     codec: str = "companded") -> dict:
    nb = nblocks(n)
    st = {
        "w16": torch.empty(n, dtype=_W16[wfmt], device=device),
        "ecc": torch.empty(n, dtype=_ECC[ecc_bits], device=device),
        "b_q": torch.zeros(code_bytes(n, codec), dtype=torch.uint8 if codec == "companded4" else torch.int8,
                           device=device),
        "b_s": torch.zeros(nb, dtype=torch.float16, device=device),
    }
    st["grad"] = torch.zeros(n, dtype=_W16[wfmt], device=device) if with_grad else None
    return st
