"""Launch-table cache bookkeeping on the CPU: least-recently-used refill and
pinning of the slots a captured HIP graph reads (precision_optimizer_state_amd/
csrc/fo_slots.hpp, compiled here by g++ with tests/host/slots_check.cpp)."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "host", "slots_check.cpp")


def test_pinned_slots_are_never_refilled(tmp_path):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / "slots_check")
    subprocess.run(["g++", "-O1", "-std=c++17", "-Wall", "-Werror", SRC, "-o", exe], check=True)
    out = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0 and out.stdout.strip() == "ok", out.stdout
