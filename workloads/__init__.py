"""Seeded synthetic workloads shared by the tests, the bench and the smoke run.

This module holds no arithmetic of the optimizer method: only parameter-list
shapes, hyperparameters and seeded random inputs (f32 weights, 16-bit
gradients cast round-to-nearest-even by torch, as a backward pass would
produce them).  The pages measure on ResNet-50 / ImageNet and GPT-2 /
Llama-3.1-8B training (blog "FlashOptim: Breaking the Memory Wall ...",
Performance); no dataset or trained weight is used: these model-shaped
parameter lists with random inputs stand in for them.
"""

from .shapes import gpt2_small_shapes, llama31_8b_shapes, resnet50_shapes  # noqa: F401
from .configs import CONFIGS, Config, config  # noqa: F401
from .gen import (  # noqa: F401
    seed_for,
    host_weights,
    host_grads,
    host_grad_bits,
    device_weights,
    device_grads,
)
