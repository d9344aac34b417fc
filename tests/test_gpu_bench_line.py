"""bench.py's JSON line on the GPU: one line on stdout with the contract's
keys, a roofline object whose fraction is achieved / peak, the per-step
pass and the device record, on a small workload (the 2^20-element flat
list, no CPU baseline) so the test takes seconds.  bench.main runs in the
test's own process."""

import contextlib
import io
import json
import os
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_prints_one_contract_line():
    # in this process (the GPU is already in use here): bench.main with its
    # stdout captured
    sys.path.insert(0, ROOT)
    import bench
    out = io.StringIO()
    with contextlib.redirect_stdout(out):
        rc = bench.main(["--config", "c1_flat1m", "--steps", "5", "--warmup", "2", "--no-cpu-baseline", "--quiet"])
    assert rc in (0, None)
    lines = [ln for ln in out.getvalue().splitlines() if ln.strip()]
    assert len(lines) == 1, out.getvalue()
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
              "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 2
    assert d["unit"] == "params/s" and d["higher_is_better"] is True and d["value"] > 0
    assert d["config"]["workload"] and d["config"]["params"] == 1 << 20
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-12
    # achieved is the algorithmic bytes over the event time per step
    assert abs(rf["achieved"] - d["config"]["bytes_per_param_moved"] * (1 << 20) / (d["kernel_ms_avg"] * 1e6)) \
        < 1e-6 * rf["achieved"]
    assert d["cpu_baseline"] is None                       # --no-cpu-baseline
    ps = d["per_step_events"]
    assert ps["steps"] == 5 and 0 < ps["min_ms"] <= ps["median_ms"] <= ps["max_ms"]
    dev = d["device"]
    assert dev["cus"] > 0 and dev["arch"].startswith("gfx")
    print(f"bench line: {rf['achieved']:.0f} GB/s on {dev['arch']} ({dev['cus']} CUs)", flush=True)


@pytest.mark.parametrize("cfg,extra,cls", [("c1_flat1m", [], "FlashAdamW"),
                                           ("c4_resnet50", ["--release"], "FlashSGD")])
def test_bench_dropin_line(cfg, extra, cls):
    """--dropin: one JSON line with the drop-in step's GPU and host times."""
    sys.path.insert(0, ROOT)
    import bench
    from workloads.configs import config
    out = io.StringIO()
    with contextlib.redirect_stdout(out):
        rc = bench.main(["--dropin", "--config", cfg, *extra, "--steps", "3", "--warmup", "1", "--quiet"])
    assert rc in (0, None)
    lines = [ln for ln in out.getvalue().splitlines() if ln.strip()]
    assert len(lines) == 1, out.getvalue()
    d = json.loads(lines[0])
    assert d["steps"] == 3 and d["config"]["params"] == config(cfg).params
    assert d["gpu_ms_per_step"] > 0 and d["host_ms_per_step"] > 0 and d["value"] > 0
    assert d["config"]["workload"].startswith(f"{cls}.step() drop-in")
    assert ("gradient release" in d["config"]["workload"]) == bool(extra)
    r = d["roofline"]
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"])
