"""fo_fused_adamw_step captured in a HIP graph (torch.cuda.graph) after one
warm-up call with the same list: every replay, with eager work and
synchronisation between replays, is bitwise equal to the same call made
eagerly on a copy of the state (the step constants are those captured)."""

import pytest
import torch

from precision_optimizer_state_amd import binding as B
from precision_optimizer_state_amd.state import alloc_adamw_state
from workloads import device_grads, device_weights

pytestmark = pytest.mark.gpu

KEYS = ("w16", "ecc", "m_q", "m_s", "v_q", "v_s")


def _state(n, tag):
    st = alloc_adamw_state(n)
    w = device_weights(tag, 0, n)
    B.fo_split_weights(w, st["w16"], st["ecc"], "bf16", 8)
    device_grads(tag, 0, 1, n, "t3", "bf16", out=st["grad"])
    return st


@pytest.mark.parametrize("sizes", [[300_000 + 77],
                                   # two tensors over more than 2^18 wave tiles: the step is
                                   # two launches (two kernel nodes in the graph)
                                   [(1 << 29) - 5000, 3 * (1 << 20) + 77]],
                         ids=["one_launch", "two_launches"])
def test_captured_step_replays_match_eager_calls(sizes):
    hp = B.adamw_hparams(1e-3, 0.9, 0.999, 1e-8, 0.01, 5)
    al = [_state(n, f"graph{i}") for i, n in enumerate(sizes)]
    tl_a = B.AdamWList(al)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        B.fo_fused_adamw_step(tl_a, hp)              # warm-up: codec tables and launch table exist
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    bl = [{k: v.clone() for k, v in a.items()} for a in al]   # eager twins of the states
    tl_b = B.AdamWList(bl)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.fo_fused_adamw_step(tl_a, hp)
    for r in range(4):
        g.replay()
        B.fo_fused_adamw_step(tl_b, hp)
        junk = torch.randn(1 << 20, device="cuda").sum()    # unrelated eager work between replays
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        for i, (a, b) in enumerate(zip(al, bl)):
            for k in KEYS:
                assert torch.equal(a[k].view(torch.uint8), b[k].view(torch.uint8)), f"replay {r}: tensor {i} {k} differs"
    print(f"graph replays ({len(sizes)} tensors): 4 replays bitwise equal to eager calls", flush=True)
