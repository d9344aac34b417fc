"""Benchmark of the fused low-precision optimizer step on one MI355X.

Default: one fused AdamW step over the Llama-3.1-8B-shaped parameter list
(291 tensors, 8,030,261,248 parameters), bf16 weights + 8-bit ECC, companded
int8/uint8 states with one fp16 scale per 32 elements.  Prints one JSON line.

A "step" is one fused optimizer step over the whole parameter list: one
kernel launch that reads gradients, weights, ECCs, codes and scales and
writes weights, ECCs, codes and scales back.  Inputs are synthetic (seeded
N(0, 0.02) weights, heavy-tailed bf16 gradients) and resident in HBM before
the timed region.  The same gradient buffer is used by every timed step.
"""

from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
KERNEL_SOURCES = ("precision_optimizer_state_amd/csrc/fo_device.hpp",
                  "precision_optimizer_state_amd/csrc/fo_kernels.hpp")


def _code_only(text: str) -> str:
    """C++ source with comments removed and whitespace collapsed, so that an
    edit of comments alone keeps the hash (the kernels it names are the same)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


# the library launches a list as consecutive ranges of at most this many
# 2048-element wave tiles (one kernel each)
LAUNCH_TILES = 1 << 18


def launches_per_call(numels) -> int:
    tiles = sum(-(-n // 2048) for n in numels)
    return -(-tiles // LAUNCH_TILES)


def read_traffic(config_name: str):
    """HBM bytes of one step (all of its launches) from committed rocprofv3
    counter runs, if they were taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{config_name}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_src_sha") != kernel_source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_step"])
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------------------
# device setup
# ---------------------------------------------------------------------------
def build_states(cfg, log):
    import torch

    from precision_optimizer_state_amd import binding as B
    from precision_optimizer_state_amd.state import alloc_adamw_state, alloc_sgdm_state
    from workloads import device_grads, device_weights

    states = []
    t0 = time.perf_counter()
    for i, n in enumerate(cfg.numels):
        if cfg.optimizer == "adamw":
            st = alloc_adamw_state(n, cfg.wfmt, cfg.ecc_bits)
        else:
            st = alloc_sgdm_state(n, cfg.wfmt, cfg.ecc_bits)
        w = device_weights(cfg.name, i, n)
        B.fo_split_weights(w, st["w16"], st["ecc"], cfg.wfmt, cfg.ecc_bits)
        del w
        device_grads(cfg.name, i, 1, n, cfg.grad_kind, cfg.wfmt, out=st["grad"])
        states.append(st)
        if i % 64 == 0:
            log(f"setup: tensor {i}/{len(cfg.numels)}")
    torch.cuda.synchronize()
    log(f"setup: {cfg.params} params in {time.perf_counter() - t0:.1f}s")
    return states


def make_launch(cfg, states, release_chunks=None):
    from precision_optimizer_state_amd import binding as B

    if cfg.optimizer == "adamw":
        if release_chunks:
            st = states[0]
            lists, lo = [], 0
            for m in release_chunks:
                hi = lo + m
                c = {k: st[k][lo:hi] for k in ("w16", "ecc", "grad", "m_q", "v_q")}
                c["m_s"] = st["m_s"][lo // 32: -(-hi // 32)]
                c["v_s"] = st["v_s"][lo // 32: -(-hi // 32)]
                lists.append(B.AdamWList([c]))
                lo = hi
        else:
            lists = [B.AdamWList(states)]

        def launch(step):
            hp = B.adamw_hparams(step=step, wfmt=cfg.wfmt, ecc_bits=cfg.ecc_bits, codec=cfg.codec, **cfg.hp)
            for tl in lists:
                B.fo_fused_adamw_step(tl, hp)
        return launch, lists
    tl = B.SGDMList(states)

    def launch(step):
        B.fo_fused_sgdm_step(tl, B.sgdm_hparams(step=step, wfmt=cfg.wfmt, ecc_bits=cfg.ecc_bits,
                                                 codec=cfg.codec, **cfg.hp))
    return launch, [tl]


# ---------------------------------------------------------------------------
# CPU baseline: the oracle, unchanged, on a bounded sample of the workload
# ---------------------------------------------------------------------------
def _oracle_task(args):
    cfg_name, t_idx, lo, m = args
    import numpy as np

    import oracle as O
    from oracle.optim import fresh_adamw_state, fresh_sgdm_state
    from workloads import config, host_grad_bits, host_grads

    cfg = config(cfg_name)
    rng = np.random.default_rng([t_idx, lo])
    x = (rng.standard_normal(m, dtype=np.float32) * np.float32(0.02)).astype(np.float32)
    gb = host_grad_bits(host_grads(cfg_name, t_idx, 1, m, cfg.grad_kind), cfg.wfmt)
    if cfg.optimizer == "adamw":
        st = fresh_adamw_state(x, cfg.wfmt, cfg.ecc_bits)
        t0 = time.perf_counter()
        O.adamw_step(st, gb, dict(cfg.hp, step=1), cfg.wfmt, cfg.ecc_bits, cfg.codec)
    else:
        st = fresh_sgdm_state(x, cfg.wfmt, cfg.ecc_bits)
        t0 = time.perf_counter()
        O.sgdm_step(st, gb, dict(cfg.hp, step=2), cfg.wfmt, cfg.ecc_bits, cfg.codec)
    return m, time.perf_counter() - t0


def cpu_baseline(cfg, segments=96, seg=1 << 20, log=print):
    import multiprocessing as mp

    import numpy as np

    sizes = np.array(cfg.numels, dtype=np.int64)
    rng = np.random.default_rng(20261203)
    tasks = []
    for _ in range(segments):
        t = int(rng.choice(len(sizes), p=sizes / sizes.sum()))
        m = int(min(seg, sizes[t]))
        lo = int(rng.integers(0, (sizes[t] - m) // 32 + 1)) * 32
        tasks.append((cfg.name, t, lo, m))
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    ctx = mp.get_context("spawn")
    t0 = time.perf_counter()
    with ctx.Pool(cores) as pool:
        res = pool.map(_oracle_task, tasks, chunksize=1)
    wall = time.perf_counter() - t0
    elems = sum(r[0] for r in res)
    cpu_s = sum(r[1] for r in res)
    # the step computations of all workers run concurrently: throughput is the
    # summed element count over the summed compute time, times the worker count
    value = elems / cpu_s * cores
    log(f"cpu baseline: {elems} elements, {cpu_s:.1f} s of oracle compute on {cores} workers (wall {wall:.1f}s)")
    return {"value": value, "unit": "params/s", "cores": cores, "kind": "oracle",
            "sample": f"{segments} segments of up to {seg} consecutive elements at seeded 32-aligned offsets "
                      f"across the parameter list (one optimizer step each, inputs from the same generators); "
                      f"{cpu_s:.1f} s of oracle compute"}


# ---------------------------------------------------------------------------
# optimizer variants on the same byte streams (hyperparameter additions)
VARIANTS = {
    "adam_l2": ("adamw", {"l2_decay": True}),
    "sgd_nesterov": ("sgdm", {"nesterov": True}),
    "sgd_dampening": ("sgdm", {"dampening": 0.1}),
}


def run_dropin(args, cfg, log):
    """FlashAdamW / FlashSGD .step() end to end on the workload's parameter list:
    the drop-in optimizer groups the parameters, marshals them and calls the
    fused step (one launch per step; with --release the post-accumulate-grad
    hooks run in backward order and step buckets of parameters, then the
    end-of-backward flush steps the rest)."""
    import torch

    from precision_optimizer_state_amd import FlashAdamW, FlashSGD
    from workloads import device_grads, device_weights

    params, grads = [], []
    for i, n in enumerate(cfg.numels):
        params.append(torch.nn.Parameter(device_weights(cfg.name, i, n)))
    kw = dict(wfmt=cfg.wfmt, ecc_bits=cfg.ecc_bits, codec=cfg.codec)
    if cfg.optimizer == "adamw":
        hp = cfg.hp
        opt = FlashAdamW(params, lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                         weight_decay=hp["weight_decay"], **kw)
    else:
        opt = FlashSGD(params, lr=cfg.hp["lr"], momentum=cfg.hp["momentum"], weight_decay=cfg.hp["weight_decay"], **kw)
    for i, (p, n) in enumerate(zip(params, cfg.numels)):
        grads.append(device_grads(cfg.name, i, 1, n, cfg.grad_kind, cfg.wfmt).view(p.shape))
    torch.cuda.synchronize()
    log(f"drop-in setup: {len(params)} parameters")

    def one_step():
        if args.release:
            for p, g in zip(reversed(params), reversed(grads)):   # backward order
                p.grad = g
                opt._release_hook(p)
            opt.flush_released()                                   # what the end of backward does
        else:
            for p, g in zip(params, grads):
                p.grad = g
            opt.step()

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    K = args.steps
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    host = 0.0
    t0 = time.perf_counter()
    a.record(stream)
    for _ in range(K):
        h0 = time.perf_counter()
        one_step()
        host += time.perf_counter() - h0
    b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / K
    gpu_ms = a.elapsed_time(b) / K
    bpp = cfg.bytes_per_param()
    achieved = bpp * cfg.params / (gpu_ms * 1e-3) / 1e9
    log(f"drop-in: {ms_per_step:.3f} ms/step wall, {gpu_ms:.3f} ms GPU, {host * 1e3 / K:.3f} ms host enqueue")
    cls = "FlashAdamW" if cfg.optimizer == "adamw" else "FlashSGD"
    return {
        "metric": "optimizer params/sec and achieved HBM GB/s (% of peak), fused AdamW step",
        "value": cfg.params / (ms_per_step * 1e-3),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded N(0,0.02) weights, heavy-tailed 16-bit gradients; no dataset, no trained weights)",
        "config": {"workload": f"{cls}.step() drop-in on the {cfg.name} parameter list"
                               + (", gradient release (buckets of 2^26 elements)" if args.release else ""),
                   "name": cfg.name, "optimizer": cfg.optimizer, "tensors": len(cfg.numels), "params": cfg.params,
                   "format": f"{cfg.wfmt}+ecc{cfg.ecc_bits}", "codec": cfg.codec, "bytes_per_param_moved": bpp},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": None},
        "gpu_ms_per_step": gpu_ms,
        "host_ms_per_step": host * 1e3 / K,
        "kernel_src_sha": kernel_source_hash(),
        "cpu_baseline": None,
    }


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="c3_llama8b")
    ap.add_argument("--release", action="store_true", help="gradient-release mode: one call per chunk (c5 shapes)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true")
    ap.add_argument("--copy-calib", action="store_true", help="also run a plain device copy of 4 GiB (counter calibration)")
    ap.add_argument("--variant", default=None, choices=sorted(VARIANTS),
                    help="optimizer variant: Adam with L2 decay (AdamW lists) or SGD with "
                         "Nesterov momentum / dampening (SGD-M lists)")
    ap.add_argument("--dropin", action="store_true",
                    help="time FlashAdamW/FlashSGD.step() end to end instead of the raw fused call "
                         "(with --release: the gradient-release hooks in backward order)")
    ap.add_argument("--quiet", action="store_true")
    args = ap.parse_args(argv)

    def log(msg):
        if not args.quiet:
            print(f"[bench] {msg}", file=sys.stderr, flush=True)

    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (the step needs no "
              "communication; on several GPUs each would step its own shard of the parameter list)", file=sys.stderr)
        return 2

    import torch

    from precision_optimizer_state_amd import binding as B
    from workloads import config
    from workloads.configs import FLAT_1G, RELEASE_CHUNKS

    cfg = config(args.config)
    if args.variant:
        opt, extra = VARIANTS[args.variant]
        if cfg.optimizer != opt:
            print(f"--variant {args.variant} needs a {opt} workload", file=sys.stderr)
            return 2
        cfg = dataclasses.replace(cfg, hp=dict(cfg.hp, **extra))
    torch.cuda.set_device(0)
    B.load()
    if args.dropin:
        print(json.dumps(run_dropin(args, cfg, log)), flush=True)
        return 0
    states = build_states(cfg, log)
    release = None
    if args.release:
        assert cfg.params == FLAT_1G and len(cfg.numels) == 1, "release mode runs on the 2^30-element tensor"
        release = RELEASE_CHUNKS
    launch, lists = make_launch(cfg, states, release)
    stream = torch.cuda.current_stream()

    step = 0
    for _ in range(args.warmup):
        step += 1
        launch(step)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")

    K = args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(K):
        step += 1
        ev[k][0].record(stream)
        launch(step)
        ev[k][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = [a.elapsed_time(b) for a, b in ev]
    avg_ms = sum(launch_ms) / K
    ms_per_step = wall * 1e3 / K
    params = cfg.params
    bpp = cfg.bytes_per_param()
    alg_bytes = bpp * params
    achieved = alg_bytes / (avg_ms * 1e-3) / 1e9
    log(f"timed {K} steps: {ms_per_step:.3f} ms/step wall, {avg_ms:.3f} ms per step (events), "
        f"{achieved:.0f} GB/s algorithmic")

    probe_gbs = None
    if not args.no_probe and cfg.optimizer == "adamw":
        pe = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
        for tl in lists:
            B.fo_stream_probe(tl, cfg.wfmt, cfg.ecc_bits, 0)
        torch.cuda.synchronize()
        for k in range(K):
            pe[k][0].record(stream)
            for tl in lists:
                B.fo_stream_probe(tl, cfg.wfmt, cfg.ecc_bits, 0)
            pe[k][1].record(stream)
        torch.cuda.synchronize()
        pms = sum(a.elapsed_time(b) for a, b in pe) / K
        probe_gbs = alg_bytes / (pms * 1e-3) / 1e9
        log(f"stream probe (same bytes, no arithmetic): {pms:.3f} ms, {probe_gbs:.0f} GB/s")

    if args.copy_calib:
        src = torch.empty(1 << 30, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 3 x 4 GiB device copies done")
        del src, dst

    line = {
        "metric": "optimizer params/sec and achieved HBM GB/s (% of peak), fused AdamW step",
        "value": params / (ms_per_step * 1e-3),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded N(0,0.02) weights split to 16-bit + ECC, heavy-tailed 16-bit gradients; "
                "no dataset, no trained weights)",
        "config": {
            "workload": {
                "c3_llama8b": "Llama-3.1-8B-shaped parameter list, fused AdamW, bf16 + 8-bit ECC, companded 8-bit states",
            }.get(cfg.name, cfg.name),
            "name": cfg.name,
            "optimizer": cfg.optimizer,
            "tensors": len(cfg.numels),
            "params": params,
            "format": f"{cfg.wfmt}+ecc{cfg.ecc_bits}",
            "codec": cfg.codec,
            "bytes_per_param_moved": bpp,
            "release_chunks": len(release) if release else None,
            "variant": args.variant,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS,
            "traffic": read_traffic(cfg.name + ("_release" if release else "")
                                    + (f"_{args.variant}" if args.variant else "")),
        },
        "kernel_ms_avg": avg_ms,
        # dispatches of the fused kernel per step (the list is launched in
        # ranges of 2^18 tiles); kernel_ms_avg and roofline cover all of them
        "launches_per_step": (sum(launches_per_call([m]) for m in release) if release
                              else launches_per_call(cfg.numels)),
        "stream_probe_gbs": probe_gbs,
        # the fused kernel against the same byte streams moved with no arithmetic
        "vs_stream_probe": (achieved / probe_gbs) if probe_gbs else None,
        "kernel_src_sha": kernel_source_hash(),
    }
    if not args.no_cpu_baseline:
        del states, lists
        torch.cuda.empty_cache()
        line["cpu_baseline"] = cpu_baseline(cfg, log=log)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
