"""The fused AdamW step's gradient range on 16-bit patterns: the host's
thresholds (precision_optimizer_state_amd/csrc/fo_grad16.hpp) against brute
force over every bfloat16 / binary16 pattern (CPU, g++)."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "host", "grad16_check.cpp")


def test_thresholds_match_brute_force(tmp_path):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / "grad16_check")
    subprocess.run(["g++", "-O2", "-std=c++17", "-Wall", "-Werror", SRC, "-o", exe], check=True)
    out = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0 and out.stdout.startswith("ok"), out.stdout
    print(out.stdout.strip())
