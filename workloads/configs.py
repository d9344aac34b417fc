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

    def read_write_bytes_per_param(self):
        """Algorithmic HBM bytes (read, written) per parameter by one fused step."""
        e = self.ecc_bits // 8
        q = 0.5 if self.codec == "companded4" else 1      # bytes per state code
        if self.optimizer == "adamw":
            # read: grad 2, w16 2, ecc E, m q, v q, scales 4/32; write: w16 2, ecc E, m q, v q, scales 4/32
            return (2 + 2 + e + 2 * q + 4 / 32), (2 + e + 2 * q + 4 / 32)
        return (2 + 2 + e + q + 2 / 32), (2 + e + q + 2 / 32)

    def bytes_per_param(self) -> float:
        """Algorithmic HBM bytes moved per parameter by one fused step."""
        r, w = self.read_write_bytes_per_param()
        return r + w


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
    # 4-bit companded states on the same lists
    "c3_llama8b_s4": Config("c3_llama8b_s4", "adamw", tuple(llama31_8b_shapes()), ADAMW_LM, steps=3,
                            grad_kind="t3_lognormal", codec="companded4"),
    "c4_resnet50_s4": Config("c4_resnet50_s4", "sgdm", tuple(resnet50_shapes()), SGDM_C4, steps=20,
                             grad_kind="normal_outliers", codec="companded4"),
    "c5_flat1g_s4": Config("c5_flat1g_s4", "adamw", (("flat", (FLAT_1G,)),), ADAMW_C1, steps=2, codec="companded4"),
    # bfloat16 block scales on the 8B list
    "c3_llama8b_bs": Config("c3_llama8b_bs", "adamw", tuple(llama31_8b_shapes()), ADAMW_LM, steps=3,
                            grad_kind="t3_lognormal", codec="companded_bf16scale"),
}


def config(name: str) -> Config:
    """A named configuration, or a flat single-tensor list of 2^k elements for
    size sweeps: "flat_2p<k>" (AdamW, bf16 + ECC8, companded, the c5 recipe)
    or "flat_sgd_2p<k>" (SGD-M with the c4 hyperparameters), 10 <= k <= 30."""
    if name in CONFIGS:
        return CONFIGS[name]
    for prefix, opt, hp in (("flat_sgd_2p", "sgdm", SGDM_C4), ("flat_2p", "adamw", ADAMW_C1)):
        if name.startswith(prefix) and name[len(prefix):].isdigit():
            k = int(name[len(prefix):])
            if not 10 <= k <= 30:
                raise KeyError(f"{name}: flat sweep sizes are 2^10 .. 2^30")
            return Config(name, opt, (("flat", (1 << k,)),), hp, steps=2,
                          grad_kind="normal_outliers" if opt == "sgdm" else "t3")
    raise KeyError(name)
