"""bench.py's command-line contract that needs no GPU: more than one GPU is
refused with a message, and the launch count it reports matches the
library's 2^18-tile launch ranges."""

import os
import subprocess
import sys

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


def test_cpu_baseline_is_a_measured_wall_rate():
    # the oracle leg runs in worker processes released together at a barrier;
    # its value is elements / wall time of the compute phase, and every worker
    # is joined (none terminated)
    sys.path.insert(0, ROOT)
    import bench
    from workloads import config
    res = bench.cpu_baseline(config("c1_flat1m"), segments=6, seg=4096, log=lambda m: None)
    assert res["kind"] == "oracle" and res["unit"] == "params/s"
    assert 1 <= res["cores"] <= 16 and res["value"] > 0
    assert "6 segments" in res["sample"] and "wall" in res["sample"]
