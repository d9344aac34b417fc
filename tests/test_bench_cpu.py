"""bench.py's parts that need no GPU: more than one GPU is refused with a
message, the launch count it reports matches the library's 2^18-tile launch
ranges, the rocprofv3 trace summary's statistics, and the flat sweep
workloads."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_launch_count_follows_the_tile_ranges():
    sys.path.insert(0, ROOT)
    import bench
    from workloads import config
    from workloads.configs import RELEASE_CHUNKS
    assert bench.launches_per_call([1]) == 1
    assert bench.launches_per_call([2048 << 18]) == 1
    assert bench.launches_per_call([(2048 << 18) + 1]) == 2
    assert bench.launches_per_call(config("c3_llama8b").numels) == 15
    assert bench.launches_per_call(config("c5_flat1g_bf16e8").numels) == 2
    assert sum(bench.launches_per_call([m]) for m in RELEASE_CHUNKS) == len(RELEASE_CHUNKS)


@pytest.mark.parametrize("name", ["c1_flat1m", "c3_llama8b_s4", "c4_resnet50_s4"])
def test_cpu_baseline_is_a_measured_wall_rate(name):
    # the oracle leg runs in worker processes released together at a barrier;
    # its value is elements / wall time of the compute phase, and every worker
    # is joined (none terminated); 4-bit configs run the oracle on packed states
    sys.path.insert(0, ROOT)
    import bench
    from workloads import config
    res = bench.cpu_baseline(config(name), segments=6, seg=4096, log=lambda m: None)
    assert res["kind"] == "oracle" and res["unit"] == "params/s"
    assert 1 <= res["cores"] <= 16 and res["value"] > 0
    assert "6 segments" in res["sample"] and "wall" in res["sample"]


def test_rocprof_summary_reports_dispatch_spread_and_gaps(tmp_path):
    """The trace summary sorts dispatches by start time, keeps the timed
    steps' dispatches (the last steps x launches-per-step of the kernel) and
    splits the idle gaps into those inside a step and those between steps."""
    import csv
    sys.path.insert(0, ROOT)
    import bench
    rows, t = [], 1000
    # 2 warm-up and 3 timed steps of 2 dispatches: durations 100 + i, gaps
    # 5 inside a step and 50 between steps; another kernel is ignored
    for i in range(10):
        rows.append({"Kernel_Name": "void fo::k_fused_adamw<0, 8, 0, false>(...)",
                     "Start_Timestamp": t, "End_Timestamp": t + 100 + i})
        t += 100 + i + (5 if i % 2 == 0 else 50)
    rows.append({"Kernel_Name": "void other(...)", "Start_Timestamp": 5, "End_Timestamp": 9})
    rows.reverse()                                   # trace files need not be in start order
    with open(tmp_path / "x_kernel_trace.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        w.writerows(rows)
    out = bench.rocprof_summary(str(tmp_path), "k_fused_adamw", launches_per_step=2, timed_steps=3)
    assert "10 dispatches, average 104 ns" in out
    assert "per dispatch over the last 6: median 107 ns, min 104, max 109" in out
    assert "gap to the next dispatch within a step: median 5 ns, min 5, max 5 (3 gaps)" in out
    assert "gap to the next dispatch between steps: median 50 ns, min 50, max 50 (2 gaps)" in out
    out = bench.rocprof_summary(str(tmp_path), "k_fused_adamw")
    assert "gap to the next dispatch: median 5 ns, min 5, max 50 (9 gaps)" in out



def test_rocprof_summary_window_medians(tmp_path):
    """--window: the median duration of each run of consecutive dispatches,
    with the run's start after the first dispatch."""
    import csv
    sys.path.insert(0, ROOT)
    import bench
    rows = [{"Kernel_Name": "void fo::k_fused_adamw<0, 8, 0, false>(...)",
             "Start_Timestamp": 5_000_000 + i * 1_000_000, "End_Timestamp": 5_000_000 + i * 1_000_000 + 100_000 + i * 1000}
            for i in range(10)]                          # 1 ms apart, 100..109 us long
    with open(tmp_path / "x_kernel_trace.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        w.writerows(rows)
    out = bench.rocprof_summary(str(tmp_path), "k_fused_adamw", window=4)
    line = [ln for ln in out.splitlines() if "per 4 dispatches" in ln][0]
    assert line.endswith("0.0 ms: 102 us; 4.0 ms: 106 us; 8.0 ms: 109 us"), line


def test_flat_sweep_configs():
    sys.path.insert(0, ROOT)
    import pytest
    from workloads import config
    c = config("flat_2p27")
    assert (c.params, c.optimizer, c.wfmt, c.ecc_bits, c.codec) == (1 << 27, "adamw", "bf16", 8, "companded")
    assert c.bytes_per_param() == 12.25
    c = config("flat_sgd_2p20")
    assert (c.params, c.optimizer) == (1 << 20, "sgdm")
    assert c.hp == config("c4_resnet50").hp
    for bad in ("flat_2p9", "flat_2p31", "flat_2px", "flat_sgd_2p"):
        with pytest.raises(KeyError):
            config(bad)
