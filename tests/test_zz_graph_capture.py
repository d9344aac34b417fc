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


def _state(n, tag, codec="companded"):
    st = alloc_adamw_state(n, codec=codec)
    w = device_weights(tag, 0, n)
    B.fo_split_weights(w, st["w16"], st["ecc"], "bf16", 8)
    device_grads(tag, 0, 1, n, "t3", "bf16", out=st["grad"])
    return st


@pytest.mark.parametrize("sizes,codec", [([300_000 + 77], "companded"),
                                         # two tensors over more than 2^18 wave tiles: the step is
                                         # two launches (two kernel nodes in the graph)
                                         ([(1 << 29) - 5000, 3 * (1 << 20) + 77], "companded"),
                                         # 4-bit state codes, odd length
                                         ([300_000 + 77, 4097], "companded4")],
                         ids=["one_launch", "two_launches", "one_launch_4bit"])
def test_captured_step_replays_match_eager_calls(sizes, codec):
    hp = B.adamw_hparams(1e-3, 0.9, 0.999, 1e-8, 0.01, 5, codec=codec)
    al = [_state(n, f"graph{i}", codec) for i, n in enumerate(sizes)]
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


def test_captured_table_survives_eviction_by_other_lists():
    """The launch table a graph captured stays valid after more distinct lists
    than the cache holds have been stepped eagerly (its slot is pinned)."""
    hp = B.adamw_hparams(1e-3, 0.9, 0.999, 1e-8, 0.01, 3)
    n = 200_000 + 33
    a = _state(n, "pin_a")
    tl_a = B.AdamWList([a])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        B.fo_fused_adamw_step(tl_a, hp)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    b = {k: v.clone() for k, v in a.items()}
    tl_b = B.AdamWList([b])
    pinned = B.load().fo_cache_pinned()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.fo_fused_adamw_step(tl_a, hp)
    # the captured call pinned its slot (checked before any eviction happens)
    assert B.load().fo_cache_pinned() == pinned + 1
    # 1100 distinct one-block lists, views into one state: more lists than cache slots
    many = _state(1100 * 32, "pin_many")
    for i in range(1100):
        sl = {k: v[i * 32:(i + 1) * 32] if k not in ("m_s", "v_s") else v[i:i + 1] for k, v in many.items()}
        B.fo_fused_adamw_step(B.AdamWList([sl]), hp)
    torch.cuda.synchronize()
    for r in range(2):
        g.replay()
        B.fo_fused_adamw_step(tl_b, hp)
        torch.cuda.synchronize()
        for k in KEYS:
            assert torch.equal(a[k].view(torch.uint8), b[k].view(torch.uint8)), f"replay {r}: {k} differs"
    print("captured table pinned: replays after 1100 other lists bitwise equal to eager calls", flush=True)


def test_captured_sgdm_step_replays_match_eager_calls():
    """fo_fused_sgdm_step captured after a warm-up call: every replay equals
    an eager call on a copy of the state, and the capture pins the list's
    launch table."""
    from precision_optimizer_state_amd.state import alloc_sgdm_state
    sizes = [250_000 + 13, 4097, 33]
    sl = []
    for i, n in enumerate(sizes):
        st = alloc_sgdm_state(n)
        B.fo_split_weights(device_weights(f"sgdcap{i}", 0, n), st["w16"], st["ecc"], "bf16", 8)
        device_grads(f"sgdcap{i}", 0, 1, n, "normal_outliers", "bf16", out=st["grad"])
        sl.append(st)
    hp = B.sgdm_hparams(0.1, 0.9, 1e-4, 2, nesterov=True)
    tl_a = B.SGDMList(sl)
    B.fo_fused_sgdm_step(tl_a, hp)                          # warm-up: the launch table exists
    torch.cuda.synchronize()
    twin = [{k: (v.clone() if v is not None else None) for k, v in st.items()} for st in sl]
    tl_b = B.SGDMList(twin)
    pinned = B.load().fo_cache_pinned()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.fo_fused_sgdm_step(tl_a, hp)
    assert B.load().fo_cache_pinned() == pinned + 1
    for r in range(3):
        g.replay()
        B.fo_fused_sgdm_step(tl_b, hp)
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(sl, twin)):
            for k in ("w16", "ecc", "b_q", "b_s"):
                assert torch.equal(a[k].view(torch.uint8), b[k].view(torch.uint8)), f"replay {r}: tensor {i} {k} differs"
    print("captured SGD-M step: 3 replays bitwise equal to eager calls", flush=True)


def test_capture_of_a_list_never_stepped_is_refused():
    """A captured call whose list has no launch table yet fails before it
    launches anything (filling a slot needs a copy and may need a wait, which
    a capture cannot hold); the list then steps normally outside capture."""
    hp = B.adamw_hparams(1e-3, 0.9, 0.999, 1e-8, 0.01, 1)
    st = _state(50_000 + 3, "cold_capture")
    before = {k: v.clone() for k, v in st.items()}
    tl = B.AdamWList([st])
    pinned = B.load().fo_cache_pinned()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with pytest.raises(B.FoError, match="outside HIP graph capture"):
        with torch.cuda.graph(g):
            B.fo_fused_adamw_step(tl, hp)
    torch.cuda.synchronize()
    assert B.load().fo_cache_pinned() == pinned
    for k in KEYS:
        assert torch.equal(st[k].view(torch.uint8), before[k].view(torch.uint8)), f"{k} changed"
    ref = {k: v.clone() for k, v in st.items()}
    B.fo_fused_adamw_step(tl, hp)
    B.fo_fused_adamw_step(B.AdamWList([ref]), hp)
    torch.cuda.synchronize()
    for k in KEYS:
        assert torch.equal(st[k].view(torch.uint8), ref[k].view(torch.uint8)), f"{k} differs after the refusal"
    print("captured call on a cold list refused; the list steps normally afterwards", flush=True)
