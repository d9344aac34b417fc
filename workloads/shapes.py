"""Parameter-list shapes of the model families the pages train on."""

from __future__ import annotations


def gpt2_small_shapes():
    """GPT-2 small (124,439,808 parameters, head tied to wte): 148 tensors."""
    d, v, ctx, L = 768, 50257, 1024, 12
    out = [("wte", (v, d)), ("wpe", (ctx, d))]
    for i in range(L):
        p = f"h.{i}."
        out += [
            (p + "ln_1.weight", (d,)), (p + "ln_1.bias", (d,)),
            (p + "attn.c_attn.weight", (d, 3 * d)), (p + "attn.c_attn.bias", (3 * d,)),
            (p + "attn.c_proj.weight", (d, d)), (p + "attn.c_proj.bias", (d,)),
            (p + "ln_2.weight", (d,)), (p + "ln_2.bias", (d,)),
            (p + "mlp.c_fc.weight", (d, 4 * d)), (p + "mlp.c_fc.bias", (4 * d,)),
            (p + "mlp.c_proj.weight", (4 * d, d)), (p + "mlp.c_proj.bias", (d,)),
        ]
    out += [("ln_f.weight", (d,)), ("ln_f.bias", (d,))]
    return out


def llama31_8b_shapes():
    """Llama-3.1-8B (8,030,261,248 parameters, untied head, GQA 8 KV heads): 291 tensors."""
    d, ff, kv, v, L = 4096, 14336, 1024, 128256, 32
    out = [("embed_tokens", (v, d))]
    for i in range(L):
        p = f"layers.{i}."
        out += [
            (p + "self_attn.q_proj", (d, d)), (p + "self_attn.k_proj", (kv, d)),
            (p + "self_attn.v_proj", (kv, d)), (p + "self_attn.o_proj", (d, d)),
            (p + "mlp.gate_proj", (ff, d)), (p + "mlp.up_proj", (ff, d)), (p + "mlp.down_proj", (d, ff)),
            (p + "input_layernorm", (d,)), (p + "post_attention_layernorm", (d,)),
        ]
    out += [("norm", (d,)), ("lm_head", (v, d))]
    return out


def resnet50_shapes():
    """torchvision-style ResNet-50 (25,557,032 parameters): 161 tensors."""
    out = [("conv1", (64, 3, 7, 7)), ("bn1.weight", (64,)), ("bn1.bias", (64,))]
    cin = 64
    for li, (blocks, width) in enumerate(zip([3, 4, 6, 3], [64, 128, 256, 512])):
        for b in range(blocks):
            p = f"layer{li + 1}.{b}."
            out += [
                (p + "conv1", (width, cin, 1, 1)), (p + "bn1.weight", (width,)), (p + "bn1.bias", (width,)),
                (p + "conv2", (width, width, 3, 3)), (p + "bn2.weight", (width,)), (p + "bn2.bias", (width,)),
                (p + "conv3", (4 * width, width, 1, 1)), (p + "bn3.weight", (4 * width,)), (p + "bn3.bias", (4 * width,)),
            ]
            if b == 0:
                out += [(p + "downsample.0", (4 * width, cin, 1, 1)),
                        (p + "downsample.1.weight", (4 * width,)), (p + "downsample.1.bias", (4 * width,))]
            cin = 4 * width
    out += [("fc.weight", (1000, 2048)), ("fc.bias", (1000,))]
    return out


def numel(shape) -> int:
    n = 1
    for s in shape:
        n *= s
    return n
