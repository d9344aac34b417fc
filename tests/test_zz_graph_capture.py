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


def test_captured_step_replays_match_eager_calls():
    n = 300_000 + 77
    hp = B.adamw_hparams(1e-3, 0.9, 0.999, 1e-8, 0.01, 5)
    a = _state(n, "graph")
    tl_a = B.AdamWList([a])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        B.fo_fused_adamw_step(tl_a, hp)              # warm-up: codec tables and launch table exist
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    b = {k: v.clone() for k, v in a.items()}         # eager twin of the state
    tl_b = B.AdamWList([b])
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.fo_fused_adamw_step(tl_a, hp)
    for r in range(4):
        g.replay()
        B.fo_fused_adamw_step(tl_b, hp)
        junk = torch.randn(1 << 20, device="cuda").sum()    # unrelated eager work between replays
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        for k in KEYS:
            assert torch.equal(a[k].view(torch.uint8), b[k].view(torch.uint8)), f"replay {r}: {k} differs"
    print("graph replays: 4 replays bitwise equal to eager calls", flush=True)
