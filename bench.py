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
            st = alloc_adamw_state(n, cfg.wfmt, cfg.ecc_bits, codec=cfg.codec)
        else:
            st = alloc_sgdm_state(n, cfg.wfmt, cfg.ecc_bits, codec=cfg.codec)
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
def _oracle_worker(cfg_name, tasks, barrier, out):
    """One worker process: generate the inputs of its segments, wait for every
    worker to be ready, then run the oracle's step on them and report the
    compute phase's monotonic clock interval (system-wide on Linux)."""
    import numpy as np

    import oracle as O
    from oracle.optim import fresh_adamw_state, fresh_sgdm_state
    from workloads import config, host_grad_bits, host_grads

    cfg = config(cfg_name)
    inputs = []
    for t_idx, lo, m in tasks:
        rng = np.random.default_rng([t_idx, lo])
        x = (rng.standard_normal(m, dtype=np.float32) * np.float32(0.02)).astype(np.float32)
        gb = host_grad_bits(host_grads(cfg_name, t_idx, 1, m, cfg.grad_kind), cfg.wfmt)
        fresh = fresh_adamw_state if cfg.optimizer == "adamw" else fresh_sgdm_state
        inputs.append((fresh(x, cfg.wfmt, cfg.ecc_bits, cfg.codec), gb))
    barrier.wait()
    t0 = time.perf_counter()
    elems = 0
    for st, gb in inputs:
        if cfg.optimizer == "adamw":
            O.adamw_step(st, gb, dict(cfg.hp, step=1), cfg.wfmt, cfg.ecc_bits, cfg.codec)
        else:
            O.sgdm_step(st, gb, dict(cfg.hp, step=2), cfg.wfmt, cfg.ecc_bits, cfg.codec)
        elems += gb.size
    out.put((elems, t0, time.perf_counter()))


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, segments=96, seg=1 << 20, log=print):
    """The oracle, unchanged, on `segments` seeded segments of the workload,
    in worker processes on this host's cores (at most 16, the host share of
    one GPU).  value = elements / wall time of the compute phase: from the
    first worker's start to the last worker's end, all workers released
    together after generating their inputs."""
    import multiprocessing as mp

    import numpy as np

    sizes = np.array(cfg.numels, dtype=np.int64)
    rng = np.random.default_rng(20261203)
    tasks = []
    for _ in range(segments):
        t = int(rng.choice(len(sizes), p=sizes / sizes.sum()))
        m = int(min(seg, sizes[t]))
        lo = int(rng.integers(0, (sizes[t] - m) // 32 + 1)) * 32
        tasks.append((t, lo, m))
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    ctx = mp.get_context("spawn")
    barrier = ctx.Barrier(cores)
    out = ctx.Queue()
    procs = [ctx.Process(target=_oracle_worker, args=(cfg.name, tasks[w::cores], barrier, out)) for w in range(cores)]
    for p in procs:
        p.start()
    res = [out.get() for _ in procs]
    for p in procs:
        p.join()
    elems = sum(r[0] for r in res)
    wall = max(r[2] for r in res) - min(r[1] for r in res)
    value = elems / wall
    model = _cpu_model()
    log(f"cpu baseline: {elems} elements in {wall:.2f} s of wall time on {cores} worker processes ({model})")
    return {"value": value, "unit": "params/s", "cores": cores, "kind": "oracle",
            "sample": f"{segments} segments of up to {seg} consecutive elements at seeded 32-aligned offsets "
                      f"across the parameter list, one optimizer step each; {elems} elements in {wall:.2f} s "
                      f"wall (compute phase) on {cores} processes, {model}"}


# ---------------------------------------------------------------------------
# HBM ceilings on this device: plain streams next to the fused step
# ---------------------------------------------------------------------------
def hbm_ceiling(read_bytes_per_elem, write_bytes_per_elem, steps=10, gib=16, log=print):
    """Plain HBM streams (fo_hbm_probe) over `gib` GiB buffers: read-only,
    write-only, copy and in-place update, each with one wave per 1, 2, 4 and
    8 KiB, timed with HIP events on the launch stream.  From the best rates a
    stream model of the fused step: its written streams are updated in place
    (each written byte is read first), the rest is read only, and the two
    kinds of traffic share the time:
        estimate = (I + R) / (I / inplace + R / read),
    I = 2 * written bytes, R = read bytes - written bytes (per element)."""
    import torch

    from precision_optimizer_state_amd import binding as B

    n = gib << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    B.fo_hbm_probe(src, None, n, "write", 0x5A5A5A5A)        # defined contents
    B.fo_hbm_probe(dst, None, n, "write", 0x3C3C3C3C)
    stream = torch.cuda.current_stream()
    out = {"buffer_gib": gib, "chunks": {}}
    for kib in (1, 2, 4, 8):
        row = {}
        for mode, moved in (("read", n), ("write", n), ("copy", 2 * n), ("inplace", 2 * n)):
            for _ in range(2):
                B.fo_hbm_probe(dst, src, n, mode, 0xFFFFFFFF, chunk_kib=kib)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(steps):
                B.fo_hbm_probe(dst, src, n, mode, 0xFFFFFFFF, chunk_kib=kib)
            b.record(stream)
            torch.cuda.synchronize()
            row[f"{mode}_gbs"] = moved * steps / (a.elapsed_time(b) * 1e-3) / 1e9
        out["chunks"][f"{kib}k"] = row
        log("hbm ceiling, {} KiB per wave: read {read_gbs:.0f}, write {write_gbs:.0f}, copy {copy_gbs:.0f}, "
            "in place {inplace_gbs:.0f} GB/s".format(kib, **row))
    del src, dst
    torch.cuda.empty_cache()
    for mode in ("read", "write", "copy", "inplace"):
        out[f"best_{mode}_gbs"] = max(r[f"{mode}_gbs"] for r in out["chunks"].values())
    inplace = 2.0 * write_bytes_per_elem
    read_only = read_bytes_per_elem - write_bytes_per_elem
    out["stream_model_gbs"] = (inplace + read_only) / (inplace / out["best_inplace_gbs"] +
                                                       read_only / out["best_read_gbs"])
    log("hbm ceiling: best read {best_read_gbs:.0f}, write {best_write_gbs:.0f}, copy {best_copy_gbs:.0f}, "
        "in place {best_inplace_gbs:.0f} GB/s; stream model of the step {stream_model_gbs:.0f} GB/s".format(**out))
    return out


# ---------------------------------------------------------------------------
# rocprofv3 output -> short text summaries (the files under profiles/)
# ---------------------------------------------------------------------------
def rocprof_summary(d, kernel="k_fused_adamw", launches_per_step=0, timed_steps=0, window=0):
    """Summary of the rocprofv3 CSV files in directory d: the kernel
    statistics (top entries), the trace of `kernel` (dispatches, average
    duration, and with launches_per_step / timed_steps the summed kernel time
    of each of the last timed_steps steps), and the counter totals of every
    kernel whose name contains `kernel` or k_hbm_probe.  With window > 0 it
    also prints the median dispatch duration of every run of `window`
    consecutive dispatches of `kernel`, with its start time after the first
    dispatch (how the duration moves over a run)."""
    import collections
    import csv
    import glob

    lines = []
    for f in sorted(glob.glob(os.path.join(d, "*_kernel_stats.csv"))):
        rows = list(csv.DictReader(open(f)))
        lines.append(f"kernel statistics ({os.path.basename(f)}), top entries:")
        lines.append("| Kernel | Calls | Total (ns) | Average (ns) | % |")
        lines.append("|---|---|---|---|---|")
        for r in rows[:6]:
            lines.append(f"| {r['Name'][:70]} | {r['Calls']} | {r['TotalDurationNs']} | "
                         f"{float(r['AverageNs']):.0f} | {r['Percentage']} |")
    for f in sorted(glob.glob(os.path.join(d, "*_kernel_trace.csv"))):
        rows = [r for r in csv.DictReader(open(f)) if kernel in r["Kernel_Name"]]
        rows.sort(key=lambda r: int(r["Start_Timestamp"]))
        se = [(int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in rows]
        durs = [b - a for a, b in se]
        if not durs:
            continue
        lines.append(f"trace of {kernel} ({os.path.basename(f)}): {len(durs)} dispatches, "
                     f"average {sum(durs) / len(durs):.0f} ns")
        timed = bool(launches_per_step and timed_steps and len(durs) >= launches_per_step * timed_steps)
        if timed:
            tail = durs[-launches_per_step * timed_steps:]
            per = [sum(tail[i * launches_per_step:(i + 1) * launches_per_step]) for i in range(timed_steps)]
            lines.append(f"  last {timed_steps} steps ({launches_per_step} dispatches each): summed kernel time "
                         f"per step mean {sum(per) / len(per) / 1e6:.4f} ms, min {min(per) / 1e6:.4f}, "
                         f"max {max(per) / 1e6:.4f}")
        # spread of the dispatch durations and the idle time between dispatches
        # (end of one to start of the next), over the timed steps if known
        win = se[-launches_per_step * timed_steps:] if timed else se
        wd = sorted(b - a for a, b in win)
        lines.append(f"  per dispatch over the last {len(win)}: median {wd[len(wd) // 2]} ns, "
                     f"min {wd[0]}, max {wd[-1]}")
        gaps = {"within a step": [], "between steps" if timed else "": []}
        for i in range(len(win) - 1):
            inside = timed and (i + 1) % launches_per_step != 0
            gaps["within a step" if inside else ("between steps" if timed else "")].append(win[i + 1][0] - win[i][1])
        for what, g in gaps.items():
            if g:
                g.sort()
                lines.append(f"  gap to the next dispatch{' ' + what if what else ''}: median {g[len(g) // 2]} ns, "
                             f"min {g[0]}, max {g[-1]} ({len(g)} gaps)")
        if window > 0:
            cells = []
            for i in range(0, len(se), window):
                ch = se[i:i + window]
                ds = sorted(b - a for a, b in ch)
                cells.append(f"{(ch[0][0] - se[0][0]) / 1e6:.1f} ms: {ds[len(ds) // 2] / 1e3:.0f} us")
            lines.append(f"  median duration per {window} dispatches (start after the first dispatch): " + "; ".join(cells))
    for f in sorted(glob.glob(os.path.join(d, "*_counter_collection.csv"))):
        tot = collections.defaultdict(float)
        disp = collections.defaultdict(set)
        for r in csv.DictReader(open(f)):
            name = r["Kernel_Name"]
            key = kernel if kernel in name else ("k_hbm_probe" if "k_hbm_probe" in name else None)
            if key:
                tot[(key, r["Counter_Name"])] += float(r["Counter_Value"])
                disp[key].add(r["Dispatch_Id"])
        lines.append(f"counters ({os.path.basename(f)}):")
        for (key, counter), v in sorted(tot.items()):
            nd = len(disp[key])
            lines.append(f"  {key} {counter}: total {v:.0f} over {nd} dispatches, per dispatch {v / nd:.1f}")
    return "\n".join(lines)


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


def device_info(torch) -> dict:
    """The GPU the run used: name, architecture, compute units, the HIP
    runtime version, and the peak shader and memory clocks the runtime
    reports (hipDeviceGetAttribute: hipDeviceAttributeClockRate = 5,
    hipDeviceAttributeMemoryClockRate = 60, both in kHz)."""
    import ctypes
    p = torch.cuda.get_device_properties(0)
    info = {"name": p.name, "arch": p.gcnArchName, "cus": p.multi_processor_count, "hip": torch.version.hip}
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        for key, attr in (("peak_sclk_mhz", 5), ("peak_mclk_mhz", 60)):
            v = ctypes.c_int(0)
            if hip.hipDeviceGetAttribute(ctypes.byref(v), attr, torch.cuda.current_device()) == 0:
                info[key] = v.value / 1000.0
    except OSError:
        pass
    return info


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="c3_llama8b")
    ap.add_argument("--release", action="store_true", help="gradient-release mode: one call per chunk (c5 shapes)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true")
    ap.add_argument("--ceiling", action="store_true",
                    help="also time plain read / write / copy HBM streams in this process (fo_hbm_probe)")
    ap.add_argument("--copy-calib", action="store_true", help="also run a plain device copy of 4 GiB (counter calibration)")
    ap.add_argument("--variant", default=None, choices=sorted(VARIANTS),
                    help="optimizer variant: Adam with L2 decay (AdamW lists) or SGD with "
                         "Nesterov momentum / dampening (SGD-M lists)")
    ap.add_argument("--dropin", action="store_true",
                    help="time FlashAdamW/FlashSGD.step() end to end instead of the raw fused call "
                         "(with --release: the gradient-release hooks in backward order)")
    ap.add_argument("--quiet", action="store_true")
    ap.add_argument("--rocprof-summary", metavar="DIR", default=None,
                    help="print a text summary of the rocprofv3 CSV files in DIR and exit (no GPU use)")
    ap.add_argument("--kernel", default="k_fused_adamw", help="kernel name filter of --rocprof-summary")
    ap.add_argument("--launches-per-step", type=int, default=0, help="with --rocprof-summary: per-step sums")
    ap.add_argument("--window", type=int, default=0,
                    help="with --rocprof-summary: median dispatch duration per window of this many dispatches")
    args = ap.parse_args(argv)
    if args.rocprof_summary:
        print(rocprof_summary(args.rocprof_summary, args.kernel, args.launches_per_step, args.steps, args.window))
        return 0

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
    # K steps, each inside its own event pair, for the median and spread of
    # single steps.  The pairs add a completion signal between steps, so these
    # run before the timed region (a trace's last K steps stay the timed ones)
    # and feed no headline figure.
    pev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for k in range(K):
        step += 1
        pev[k][0].record(stream)
        launch(step)
        pev[k][1].record(stream)
    torch.cuda.synchronize()
    single = sorted(a.elapsed_time(b) for a, b in pev)
    per_step = {"median_ms": single[K // 2] if K % 2 else 0.5 * (single[K // 2 - 1] + single[K // 2]),
                "min_ms": single[0], "max_ms": single[-1], "steps": K}
    log(f"{K} single steps, one event pair each: median {per_step['median_ms']:.3f} ms, "
        f"min {single[0]:.3f}, max {single[-1]:.3f}")

    # the timed steps: one pair of HIP events on the launch stream around all
    # K of them (an event recorded between two steps adds a completion signal
    # and a gap of about 15 us between their dispatches, which back-to-back
    # optimizer steps do not have)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for k in range(K):
        step += 1
        launch(step)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    avg_ms = ev0.elapsed_time(ev1) / K
    ms_per_step = wall * 1e3 / K
    params = cfg.params
    bpp = cfg.bytes_per_param()
    alg_bytes = bpp * params
    achieved = alg_bytes / (avg_ms * 1e-3) / 1e9
    log(f"timed {K} steps: {ms_per_step:.3f} ms/step wall, {avg_ms:.3f} ms per step (events), "
        f"{achieved:.0f} GB/s algorithmic")

    probe_gbs = None
    # the stream probe moves the bytes of a step with 8-bit state codes
    if not args.no_probe and cfg.optimizer == "adamw" and cfg.codec != "companded4":
        pe0, pe1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for tl in lists:
            B.fo_stream_probe(tl, cfg.wfmt, cfg.ecc_bits, 0)
        torch.cuda.synchronize()
        pe0.record(stream)
        for k in range(K):
            for tl in lists:
                B.fo_stream_probe(tl, cfg.wfmt, cfg.ecc_bits, 0)
        pe1.record(stream)
        torch.cuda.synchronize()
        pms = pe0.elapsed_time(pe1) / K
        probe_gbs = alg_bytes / (pms * 1e-3) / 1e9
        log(f"stream probe (same bytes, no arithmetic): {pms:.3f} ms, {probe_gbs:.0f} GB/s")

    if args.copy_calib:
        # known traffic for the counters' scale: 4 GiB read + 4 GiB written per call
        src = torch.empty(4 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            B.fo_hbm_probe(dst, src, 4 << 30, "copy", 0)
        torch.cuda.synchronize()
        log("copy calibration: 3 x 4 GiB k_hbm_probe copies done")
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
                "c3_llama8b_s4": "Llama-3.1-8B-shaped parameter list, fused AdamW, bf16 + 8-bit ECC, "
                                 "companded 4-bit states",
                "c4_resnet50_s4": "ResNet-50-shaped parameter list, fused SGD-M, bf16 + 8-bit ECC, "
                                  "companded 4-bit states",
                "c5_flat1g_s4": "one 2^30-element tensor, fused AdamW, bf16 + 8-bit ECC, companded 4-bit states",
                "c3_llama8b_bs": "Llama-3.1-8B-shaped parameter list, fused AdamW, bf16 + 8-bit ECC, "
                                 "companded 8-bit states with bfloat16 block scales",
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
        "per_step_events": per_step,
        "device": device_info(torch),
        "stream_probe_gbs": probe_gbs,
        # the fused kernel against the same byte streams moved with no arithmetic
        "vs_stream_probe": (achieved / probe_gbs) if probe_gbs else None,
        "kernel_src_sha": kernel_source_hash(),
    }
    if args.ceiling:
        del states, lists
        states = lists = None
        torch.cuda.empty_cache()
        rb, wb = cfg.read_write_bytes_per_param()
        ceil = hbm_ceiling(rb, wb, log=log)
        if probe_gbs:
            ceil["stream_probe_gbs"] = probe_gbs
        ceil["fused_vs_stream_model"] = achieved / ceil["stream_model_gbs"]
        ceil["fused_vs_best_copy"] = achieved / ceil["best_copy_gbs"]
        line["ceiling"] = ceil
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
