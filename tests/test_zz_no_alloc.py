"""The allocation-free AdamW entry point (fo_fused_adamw_step_noalloc) through
the C ABI: bitwise equal to fo_fused_adamw_step on a copy of the same state,
on two calls in a row, the second with a smaller list (the fixed device
array then holds the first call's larger table beyond the second's), and
when captured into a HIP graph and replayed between calls on another list;
lists over the limit are rejected before any device work."""

import pytest
import torch

from precision_optimizer_state_amd import binding as B
from precision_optimizer_state_amd.state import alloc_adamw_state
from workloads import device_grads, device_weights

pytestmark = pytest.mark.gpu

KEYS = ("w16", "ecc", "m_q", "m_s", "v_q", "v_s")
HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def _states(sizes, tag, codec="companded"):
    out = []
    for i, n in enumerate(sizes):
        st = alloc_adamw_state(n, codec=codec)
        B.fo_split_weights(device_weights(tag, i, n), st["w16"], st["ecc"], "bf16", 8)
        device_grads(tag, i, 1, n, "t3", "bf16", out=st["grad"])
        out.append(st)
    return out


def _clone(states):
    return [{k: (v.clone() if v is not None else None) for k, v in st.items()} for st in states]


@pytest.mark.parametrize("sizes_a,sizes_b", [
    # many tensors and ragged tails, then fewer and smaller ones
    ([(1 << 20) + 77, 33, 0, 4096, 2049, 300_000], [5000, 31]),
    # more than 2^18 wave tiles (two launches), then one small tensor
    ([(1 << 29) + 4097], [70_001]),
])
def test_noalloc_step_equals_cached_step(sizes_a, sizes_b):
    for call, sizes in enumerate((sizes_a, sizes_b)):
        print(f"no-alloc call {call}: sizes {sizes}", flush=True)
        a = _states(sizes, f"noalloc{call}")
        b = _clone(a)
        for step in (1, 2):
            hp = dict(HP, step=step)
            B.fo_fused_adamw_step(a, hp)
            B.fo_fused_adamw_step_noalloc(b, hp)
        torch.cuda.synchronize()
        for i, (sa, sb) in enumerate(zip(a, b)):
            for k in KEYS:
                assert torch.equal(sa[k].view(torch.uint8), sb[k].view(torch.uint8)), (call, i, k)
        del a, b
        torch.cuda.empty_cache()


@pytest.mark.parametrize("codec", ["companded4", "companded_bf16scale"])
def test_noalloc_step_equals_cached_step_other_codecs(codec):
    """The same with 4-bit state codes (two per byte, odd lengths included)
    and with bfloat16 block scales."""
    for call, sizes in enumerate(([(1 << 20) + 77, 33, 4097, 2049], [5001, 31])):
        print(f"no-alloc {codec} call {call}: sizes {sizes}", flush=True)
        a = _states(sizes, f"noalloc_{codec}_{call}", codec)
        b = _clone(a)
        for step in (1, 2):
            hp = dict(HP, step=step, codec=codec)
            B.fo_fused_adamw_step(a, hp)
            B.fo_fused_adamw_step_noalloc(b, hp)
        torch.cuda.synchronize()
        for i, (sa, sb) in enumerate(zip(a, b)):
            for k in KEYS:
                assert torch.equal(sa[k].view(torch.uint8), sb[k].view(torch.uint8)), (call, i, k)


def test_noalloc_rejects_lists_over_the_limit():
    st = alloc_adamw_state(64)
    with pytest.raises(B.FoError) as ei:
        B.fo_fused_adamw_step_noalloc([st] * 2049, dict(HP, step=1))
    assert ei.value.code == B.FO_EINVAL and "2048" in str(ei.value)


def test_noalloc_captured_call_replays_its_own_table():
    """A captured allocation-free call carries its launch table in the graph
    (kernel arguments): eager allocation-free calls on another list rewrite
    the shared device array between replays, and every replay still equals
    the cached entry point's step on a copy of the state."""
    hp = dict(HP, step=3)
    a = _states([300_000 + 77, 4099], "nacap_a")
    ref = _clone(a)
    other = _states([70_001, 33, 5000], "nacap_b")
    tl_a, tl_other = B.AdamWList(a), B.AdamWList(other)
    B.fo_fused_adamw_step_noalloc(tl_other, hp)            # codec tables built outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.fo_fused_adamw_step_noalloc(tl_a, hp)
    for r in range(3):
        B.fo_fused_adamw_step_noalloc(tl_other, hp)        # another table in the shared array
        g.replay()
        B.fo_fused_adamw_step(ref, hp)
        torch.cuda.synchronize()
        for i, (sa, sb) in enumerate(zip(a, ref)):
            for k in KEYS:
                assert torch.equal(sa[k].view(torch.uint8), sb[k].view(torch.uint8)), (r, i, k)
    print("captured no-alloc call: 3 replays bitwise equal to cached eager calls", flush=True)


def test_noalloc_full_list_of_2048_tensors():
    """The largest list the allocation-free step takes: 2048 tensors (54
    kernel-argument chunks of descriptors, ragged sizes), bitwise equal to the
    cached step."""
    import numpy as np
    rng = np.random.default_rng(2048)
    sizes = [int(s) for s in rng.integers(1, 6000, 2048)]
    a = _states(sizes, "nafull")
    b = _clone(a)
    hp = dict(HP, step=1)
    B.fo_fused_adamw_step(a, hp)
    B.fo_fused_adamw_step_noalloc(b, hp)
    torch.cuda.synchronize()
    for i, (sa, sb) in enumerate(zip(a, b)):
        for k in KEYS:
            assert torch.equal(sa[k].view(torch.uint8), sb[k].view(torch.uint8)), (i, k)
    print("no-alloc step over 2048 tensors bitwise equal to the cached step", flush=True)
