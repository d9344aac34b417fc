"""MI355X (gfx950) fused low-precision optimizer step: 16-bit weights with an
ULP-normalised error-correction code, companded 8-bit optimizer states, fused
AdamW / Adam and momentum SGD over tensor lists.  The compute lives in the HIP
library csrc/ -> lib/libfoamd.so; binding.py marshals torch tensors into its
C ABI (include/foamd.h)."""

from . import binding  # noqa: F401
from .binding import (  # noqa: F401
    AdamWList,
    SGDMList,
    FoError,
    adamw_hparams,
    sgdm_hparams,
    fo_abi_version,
    fo_companded_quantize,
    fo_dequantize,
    fo_fused_adamw_step,
    fo_fused_adamw_step_noalloc,
    fo_fused_sgdm_step,
    fo_reconstruct_weights,
    fo_split_weights,
    fo_stream_probe,
)
from .state import alloc_adamw_state, alloc_sgdm_state  # noqa: F401
from .optim import FlashAdam, FlashAdamW, FlashSGD  # noqa: F401
