"""The five workload configurations (shapes, optimizer, hyperparameters)."""

from __future__ import annotations

from dataclasses import dataclass, field

from .shapes import gpt2_small_shapes, llama31_8b_shapes, numel, resnet50_shapes


@dataclass(frozen=True)
class Config:
    name: str
    optimizer: str                 # "adamw" | "sgdm"
    shapes: tuple                  # ((name, shape), ...)
    hp: dict = field(hash=False)
    steps: int = 10
    grad_kind: str = "t3"          # "t3" | "t3_lognormal" | "normal_outliers"
    wfmt: str = "bf16"
    ecc_bits: int = 8
    codec: str = "companded"

    @property
    def numels(self):
        return [numel(s) for _, s in self.shapes]

    @property
    def params(self) -> int:
        return sum(self.numels)

    def bytes_per_param(self) -> float:
        """Algorithmic HBM bytes moved per parameter by one fused step."""
        if self.optimizer == "adamw":
            # read: grad 2, w16 2, ecc E, m 1, v 1, scales 4/32; write: w16 2, ecc E, m 1, v 1, scales 4/32
            e = self.ecc_bits // 8
            return (2 + 2 + e + 1 + 1 + 4 / 32) + (2 + e + 1 + 1 + 4 / 32)
        e = self.ecc_bits // 8
        return (2 + 2 + e + 1 + 2 / 32) + (2 + e + 1 + 2 / 32)


ADAMW_C1 = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
ADAMW_LM = dict(lr=6e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
SGDM_C4 = dict(lr=0.1, momentum=0.9, weight_decay=1e-4)

FLAT_1G = 1 << 30
# gradient-release chunks of the 2^30 tensor: 18 x (4096 x 14336) + 1 x (4096 x 4096)
RELEASE_CHUNKS = tuple([4096 * 14336] * 18 + [4096 * 4096])
assert sum(RELEASE_CHUNKS) == FLAT_1G

CONFIGS = {
    "c1_flat1m": Config("c1_flat1m", "adamw", (("flat", (1 << 20,)),), ADAMW_C1, steps=10, grad_kind="t3"),
    "c2_gpt2": Config("c2_gpt2", "adamw", tuple(gpt2_small_shapes()), ADAMW_LM, steps=20, grad_kind="t3_lognormal"),
    "c3_llama8b": Config("c3_llama8b", "adamw", tuple(llama31_8b_shapes()), ADAMW_LM, steps=3, grad_kind="t3_lognormal"),
    "c4_resnet50": Config("c4_resnet50", "sgdm", tuple(resnet50_shapes()), SGDM_C4, steps=20, grad_kind="normal_outliers"),
    "c5_flat1g_bf16e8": Config("c5_flat1g_bf16e8", "adamw", (("flat", (FLAT_1G,)),), ADAMW_C1, steps=2),
    "c5_flat1g_fp16e8": Config("c5_flat1g_fp16e8", "adamw", (("flat", (FLAT_1G,)),), ADAMW_C1, steps=2, wfmt="fp16"),
    "c5_flat1g_bf16e16": Config("c5_flat1g_bf16e16", "adamw", (("flat", (FLAT_1G,)),), ADAMW_C1, steps=2, ecc_bits=16),
    "c5_flat1g_linear": Config("c5_flat1g_linear", "adamw", (("flat", (FLAT_1G,)),), ADAMW_C1, steps=2, codec="linear"),
}


def config(name: str) -> Config:
    return CONFIGS[name]
