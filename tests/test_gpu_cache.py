"""The launch-table cache's refills, on the GPU.  A call records no event per
use; a refill of a slot waits for the slot's earlier launches by stream order
(same stream, memory rewritten in place), by synchronising the stream (same
stream, memory replaced by a larger table) or by synchronising the device (a
use on another stream).  Each test queues steps of a large list, forces its
slot to be refilled while they may still run, and checks that the queued
steps end bitwise equal to the same steps on an untouched copy, and that the
small lists that forced the refill stepped as one list of their blocks would
(blocks are independent, so one-block lists and the whole array agree)."""

import pytest
import torch

from precision_optimizer_state_amd import binding as B
from precision_optimizer_state_amd.state import alloc_adamw_state
from workloads import device_grads, device_weights

pytestmark = pytest.mark.gpu

KEYS = ("w16", "ecc", "m_q", "m_s", "v_q", "v_s")
SLOTS = 1024


def _state(n, tag):
    st = alloc_adamw_state(n)
    w = device_weights(tag, 0, n)
    B.fo_split_weights(w, st["w16"], st["ecc"], "bf16", 8)
    device_grads(tag, 0, 1, n, "t3", "bf16", out=st["grad"])
    return st


def _hp(t):
    return B.adamw_hparams(1e-3, 0.9, 0.999, 1e-8, 0.01, t)


def _block_lists(st, count, per_list):
    """`count` lists of `per_list` one-block (32-element) tensors, views into st."""
    out = []
    for i in range(count):
        tens = []
        for j in range(per_list):
            b = i * per_list + j
            tens.append({k: (v[b:b + 1] if k in ("m_s", "v_s") else v[b * 32:(b + 1) * 32]) for k, v in st.items()})
        out.append(B.AdamWList(tens))
    return out


def _assert_equal(got, want, what):
    for k in KEYS:
        assert torch.equal(got[k].view(torch.uint8), want[k].view(torch.uint8)), f"{what}: {k} differs"


def _queued_list_and_copy(tag, n=(1 << 26) + 77):
    x = _state(n, tag)
    ref = {k: v.clone() for k, v in x.items()}
    return x, ref, B.AdamWList([x]), B.AdamWList([ref])


def test_refill_from_another_stream_waits_for_the_queued_steps():
    steps = 30
    x, ref, tl_x, tl_ref = _queued_list_and_copy("cache_xs")
    many = _state(1100 * 32, "cache_xs_many")
    whole = {k: v.clone() for k, v in many.items()}
    small = _block_lists(many, 1100, 1)
    a, b = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(a):
        for t in range(1, steps + 1):
            B.fo_fused_adamw_step(tl_x, _hp(t))
    # more distinct lists than slots, from stream b: x's slot is refilled while
    # the steps queued on stream a may still run
    with torch.cuda.stream(b):
        for tl in small:
            B.fo_fused_adamw_step(tl, _hp(1))
    torch.cuda.synchronize()
    for t in range(1, steps + 1):
        B.fo_fused_adamw_step(tl_ref, _hp(t))
    B.fo_fused_adamw_step(B.AdamWList([whole]), _hp(1))
    torch.cuda.synchronize()
    _assert_equal(x, ref, "list stepped on stream a")
    _assert_equal(many, whole, "one-block lists stepped on stream b")
    print(f"refill from another stream: {steps} queued steps and 1100 one-block lists bitwise as expected",
          flush=True)


def test_refill_with_a_larger_table_on_the_same_stream():
    """x's slot (sized for a small table) is refilled by a 200-tensor list on
    the stream x's steps are queued on: the slot's memory is replaced, which
    waits for the stream."""
    steps = 30
    x, ref, tl_x, tl_ref = _queued_list_and_copy("cache_ss")
    pinned = B.load().fo_cache_pinned()
    fill = SLOTS - pinned - 1                 # then x's slot is the least recently used
    many = _state(fill * 32, "cache_ss_many")
    big = _state(200 * 32, "cache_ss_big")
    whole_many = {k: v.clone() for k, v in many.items()}
    whole_big = {k: v.clone() for k, v in big.items()}
    small = _block_lists(many, fill, 1)
    big_list = _block_lists(big, 1, 200)[0]
    a = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(a):
        for t in range(1, steps + 1):
            B.fo_fused_adamw_step(tl_x, _hp(t))
        for tl in small:
            B.fo_fused_adamw_step(tl, _hp(1))
        B.fo_fused_adamw_step(big_list, _hp(1))
    torch.cuda.synchronize()
    for t in range(1, steps + 1):
        B.fo_fused_adamw_step(tl_ref, _hp(t))
    B.fo_fused_adamw_step(B.AdamWList([whole_many]), _hp(1))
    B.fo_fused_adamw_step(B.AdamWList([whole_big]), _hp(1))
    torch.cuda.synchronize()
    _assert_equal(x, ref, "list stepped before the refill")
    _assert_equal(many, whole_many, "one-block lists")
    _assert_equal(big, whole_big, "200-tensor list")
    print(f"refill with a larger table on the same stream ({fill} one-block lists, {pinned} pinned slots): "
          "bitwise as expected", flush=True)


def test_alternating_streams_keep_every_step():
    """One list stepped alternately on two streams (ordered by waits) while
    other lists churn the cache from a third: every step lands."""
    steps = 12
    x, ref, tl_x, tl_ref = _queued_list_and_copy("cache_alt", n=(1 << 24) + 5)
    many = _state(1100 * 32, "cache_alt_many")
    whole = {k: v.clone() for k, v in many.items()}
    small = _block_lists(many, 1100, 1)
    s = [torch.cuda.Stream(), torch.cuda.Stream()]
    c = torch.cuda.Stream()
    torch.cuda.synchronize()
    for t in range(1, steps + 1):
        cur, other = s[t % 2], s[(t + 1) % 2]
        cur.wait_stream(other)                 # the steps of x stay in order
        with torch.cuda.stream(cur):
            B.fo_fused_adamw_step(tl_x, _hp(t))
        with torch.cuda.stream(c):
            for tl in small[(t - 1) * 90:t * 90]:
                B.fo_fused_adamw_step(tl, _hp(1))
    with torch.cuda.stream(c):
        for tl in small[steps * 90:]:
            B.fo_fused_adamw_step(tl, _hp(1))
    torch.cuda.synchronize()
    for t in range(1, steps + 1):
        B.fo_fused_adamw_step(tl_ref, _hp(t))
    B.fo_fused_adamw_step(B.AdamWList([whole]), _hp(1))
    torch.cuda.synchronize()
    _assert_equal(x, ref, "list stepped on alternating streams")
    _assert_equal(many, whole, "one-block lists")
    print("alternating streams: every step bitwise as expected", flush=True)


def test_sgdm_refill_from_another_stream_waits_for_the_queued_steps():
    """The SGD-M entry point shares the cache: its list's slot refilled from
    another stream while its steps may still run on the first."""
    from precision_optimizer_state_amd.state import alloc_sgdm_state

    def sgd_state(n, tag):
        st = alloc_sgdm_state(n)
        w = device_weights(tag, 0, n)
        B.fo_split_weights(w, st["w16"], st["ecc"], "bf16", 8)
        device_grads(tag, 0, 1, n, "normal_outliers", "bf16", out=st["grad"])
        return st

    def hp(t):
        return B.sgdm_hparams(0.1, 0.9, 1e-4, t)

    keys = ("w16", "ecc", "b_q", "b_s")
    steps = 30
    x = sgd_state((1 << 26) + 77, "cache_sgd_x")
    ref = {k: v.clone() for k, v in x.items()}
    many = sgd_state(1100 * 32, "cache_sgd_many")
    whole = {k: v.clone() for k, v in many.items()}
    small = [B.SGDMList([{k: (v[i:i + 1] if k == "b_s" else v[i * 32:(i + 1) * 32]) for k, v in many.items()}])
             for i in range(1100)]
    a, b = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(a):
        for t in range(1, steps + 1):
            B.fo_fused_sgdm_step(B.SGDMList([x]), hp(t))
    with torch.cuda.stream(b):
        for tl in small:
            B.fo_fused_sgdm_step(tl, hp(1))
    torch.cuda.synchronize()
    for t in range(1, steps + 1):
        B.fo_fused_sgdm_step(B.SGDMList([ref]), hp(t))
    B.fo_fused_sgdm_step(B.SGDMList([whole]), hp(1))
    torch.cuda.synchronize()
    for k in keys:
        assert torch.equal(x[k].view(torch.uint8), ref[k].view(torch.uint8)), f"SGD-M list: {k} differs"
        assert torch.equal(many[k].view(torch.uint8), whole[k].view(torch.uint8)), f"one-block SGD-M lists: {k} differs"
    print(f"SGD-M refill from another stream: {steps} queued steps and 1100 one-block lists bitwise as expected",
          flush=True)
