"""Full-size parity of every workload configuration, in the launch
configuration bench.py times (one fused call over the whole parameter list;
19 chunked calls per step in gradient-release mode).

The oracle cannot run 8 billion elements, but 32-element blocks are
independent: for a seeded sample of blocks of every tensor (always including
the tensor's last, possibly partial, block) the test runs in lock-step on
those blocks.  Before every step it gathers the sampled blocks' device state
and gradients, the oracle steps them alone, and after the device step the
same blocks must be bitwise equal.  The initial split of the sampled weights
is compared with the oracle's split first.
"""

import numpy as np
import pytest
import torch

import oracle as O
from precision_optimizer_state_amd import binding as B
from precision_optimizer_state_amd.state import alloc_adamw_state, alloc_sgdm_state
from tests.gpu_helpers import check_state, check_weights, to_host
from workloads import config, device_grads, device_weights
from workloads.configs import Config
from workloads.configs import RELEASE_CHUNKS

pytestmark = pytest.mark.gpu


def _sample_blocks(n, k, rng, forced=()):
    nb = -(-n // 32)
    if nb == 0:
        return np.zeros(0, np.int64), np.zeros(0, np.int64)
    pick = rng.choice(nb, size=min(nb, k), replace=False)
    extra = [b for b in forced if 0 <= b < nb]
    pick = np.unique(np.concatenate([pick, [nb - 1], np.asarray(extra, dtype=np.int64)])).astype(np.int64)
    idx = (pick[:, None] * 32 + np.arange(32)[None, :]).ravel()
    return pick, idx[idx < n]


def _gather(t, idx_dev):
    return to_host(t[idx_dev])


def _sampled_state(st, bdev, idev, adam):
    got = {"w16": _gather(st["w16"], idev), "ecc": _gather(st["ecc"], idev)}
    if adam:
        got.update(m_q=_gather(st["m_q"], idev), m_s=_gather(st["m_s"], bdev),
                   v_q=_gather(st["v_q"], idev), v_s=_gather(st["v_s"], bdev))
    else:
        got.update(b_q=_gather(st["b_q"], idev), b_s=_gather(st["b_s"], bdev))
    return got


def _run(cfg_name, steps, blocks_per_tensor, release=False, cfg=None, forced=()):
    cfg = cfg or config(cfg_name)
    rng = np.random.default_rng(7)
    adam = cfg.optimizer == "adamw"
    states, samples = [], []
    print(f"{cfg_name}: {len(cfg.numels)} tensors, {cfg.params} params, {steps} steps", flush=True)
    for i, n in enumerate(cfg.numels):
        st = (alloc_adamw_state if adam else alloc_sgdm_state)(n, cfg.wfmt, cfg.ecc_bits)
        w = device_weights(cfg.name, i, n)
        blocks, idx = _sample_blocks(n, blocks_per_tensor, rng, forced)
        idx_dev = torch.from_numpy(idx).cuda()
        x0 = w[idx_dev].cpu().numpy()
        B.fo_split_weights(w, st["w16"], st["ecc"], cfg.wfmt, cfg.ecc_bits)
        del w
        if n:
            w_ref, e_ref = O.split_weights(x0, cfg.wfmt, cfg.ecc_bits)
            check_weights(f"{cfg_name} split {i}", _gather(st["w16"], idx_dev), _gather(st["ecc"], idx_dev),
                          w_ref, e_ref, cfg.wfmt, cfg.ecc_bits)
        states.append(st)
        samples.append((torch.from_numpy(blocks).cuda(), idx_dev))
    if adam and release:
        st = states[0]
        lists, lo = [], 0
        for m in RELEASE_CHUNKS:
            hi = lo + m
            c = {k: st[k][lo:hi] for k in ("w16", "ecc", "grad", "m_q", "v_q")}
            c["m_s"] = st["m_s"][lo // 32: -(-hi // 32)]
            c["v_s"] = st["v_s"][lo // 32: -(-hi // 32)]
            lists.append(B.AdamWList([c]))
            lo = hi
    else:
        lists = [B.AdamWList(states) if adam else B.SGDMList(states)]
    total = 0
    for step in range(1, steps + 1):
        before, gsamp = [], []
        for i, (st, n) in enumerate(zip(states, cfg.numels)):
            device_grads(cfg.name, i, step, n, cfg.grad_kind, cfg.wfmt, out=st["grad"])
            gsamp.append(_gather(st["grad"], samples[i][1]))
            before.append(_sampled_state(st, *samples[i], adam) if n else None)
        for tl in lists:
            if adam:
                B.fo_fused_adamw_step(tl, B.adamw_hparams(step=step, wfmt=cfg.wfmt, ecc_bits=cfg.ecc_bits,
                                                          codec=cfg.codec, **cfg.hp))
            else:
                B.fo_fused_sgdm_step(tl, B.sgdm_hparams(step=step, wfmt=cfg.wfmt, ecc_bits=cfg.ecc_bits,
                                                        codec=cfg.codec, **cfg.hp))
        torch.cuda.synchronize()
        for i, st in enumerate(states):
            if cfg.numels[i] == 0:
                continue
            if adam:
                want = O.adamw_step(before[i], gsamp[i], dict(cfg.hp, step=step), cfg.wfmt, cfg.ecc_bits, cfg.codec)
            else:
                want = O.sgdm_step(before[i], gsamp[i], dict(cfg.hp, step=step), cfg.wfmt, cfg.ecc_bits, cfg.codec)
            check_state(f"{cfg_name} step {step} tensor {i}", _sampled_state(st, *samples[i], adam), want,
                        cfg.wfmt, cfg.ecc_bits)
            total += samples[i][1].numel()
    print(f"{cfg_name}{' release' if release else ''}: {total} sampled element-steps over {steps} lock-steps, "
          f"all bitwise equal", flush=True)
    del states, lists
    torch.cuda.empty_cache()


def test_config_c1_flat_1m_full():
    _run("c1_flat1m", 10, 1 << 15)          # every block of the 1M tensor


def test_config_c2_gpt2_small_full():
    _run("c2_gpt2", 20, 96)


def test_config_c3_llama31_8b_full():
    _run("c3_llama8b", 3, 64)


def test_config_c4_resnet50_sgdm_full():
    _run("c4_resnet50", 20, 128)


@pytest.mark.parametrize("name", ["c5_flat1g_bf16e8", "c5_flat1g_fp16e8", "c5_flat1g_bf16e16", "c5_flat1g_linear"])
def test_config_c5_flat_2_30_variants(name):
    _run(name, 2, 20000)


def test_config_c5_gradient_release_chunks():
    _run("c5_flat1g_bf16e8", 2, 20000, release=True)


@pytest.mark.parametrize("opt,wfmt,ecc", [("adamw", "bf16", 8), ("adamw", "bf16", 16), ("sgdm", "fp16", 8)])
def test_tensor_beyond_2_31_elements_next_to_empty_and_tiny_tensors(opt, wfmt, ecc):
    """64-bit indexing at the largest sizes: one tensor of 2^31 + 2^11 + 45
    elements (its 16-bit byte offsets pass 2^31 at element 2^30 and 2^32 at
    element 2^31; its byte-stream offsets pass 2^31 at element 2^31), listed
    after a 33-element and an empty tensor, 2 steps; AdamW with 8- and 16-bit
    ECC and SGD-M on fp16.  Sampled blocks include those around both
    boundaries and the ragged tail."""
    big = (1 << 31) + (1 << 11) + 45
    hp = config("c5_flat1g_bf16e8").hp if opt == "adamw" else config("c4_resnet50").hp
    cfg = Config(f"huge_2_31_{opt}_{wfmt}{ecc}", opt, (("tiny", (33,)), ("empty", (0,)), ("huge", (big,))), hp,
                 steps=2, grad_kind="t3", wfmt=wfmt, ecc_bits=ecc)
    forced = [b + d for b in ((1 << 30) // 32, (1 << 31) // 32) for d in range(-3, 3)]
    _run(cfg.name, 2, 4000, cfg=cfg, forced=forced)
