"""CPU oracle for the fused low-precision optimizer step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.
The product path (the HIP library and its Python binding) never imports, links
or calls it, and fails loudly when the HIP library is missing instead of
falling back here.

The oracle is a plain, slow, obviously-correct NumPy rendering of what the
method computes, written from the pages that describe FlashOptim:

* "FlashOptim: Breaking the Memory Wall with 24-bit Weights and Companded
  States" (blog summary) -- Methodology section 1 "ULP-based Weight
  Splitting", section 2 "Companded Quantization", TL;DR and "The Problem"
  (byte accounting), "Critical Insight" (linear quantisation ablation).
* Davis Blalock's FlashOptim release thread -- the posts on weight splitting
  and ECC bits, on blockwise 8-bit state quantisation with a 16-bit scale per
  32 elements, on companding for momentum-like and variance-like states, on
  keeping gradients in backward precision, and on gradient release.

It shares no code with the HIP path: the HIP kernels use integer bit tricks on
IEEE encodings, the oracle uses float64 arithmetic on values (spacings,
floors, exact rationals).  Where the pages leave a step open the oracle takes
the reading listed at the top of each module.  Parity status of each function
is stated in its module header.
"""

from .numerics import (  # noqa: F401
    FORMATS,
    rna_downcast,
    split_weights,
    reconstruct_weights,
    f16_bits_to_f32,
    f32_to_f16_bits_exact,
)
from .codecs import (  # noqa: F401
    ru_fp16_bits,
    ru_bf16_bits,
    scale_to_f32,
    block_scales,
    encode_momentum,
    decode_momentum,
    encode_variance,
    decode_variance,
    quantize_state,
    dequantize_state,
    momentum_lut,
    level_spacing,
    code_bytes,
    pack_nibbles,
    unpack_nibbles,
)
from .optim import (  # noqa: F401
    adamw_scalars,
    sgdm_scalars,
    adamw_update,
    sgdm_update,
    adamw_step,
    sgdm_step,
    sgdm_first,
)
