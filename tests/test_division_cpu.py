"""The residual-corrected division of the fused kernels equals IEEE division
(CPU, no GPU): on every binary32 pair whose quotient lies near a rounding
midpoint -- the only pairs where it could differ -- and exhaustively for
binary16 divisors and their squares, the divisors of the state codecs.
tests/host/division_check.c holds the enumeration; the device-side checks
of the same sequence are fo_selftest modes 3-5."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "host", "division_check.c")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path_factory.mktemp("div") / "division_check")
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", SRC, "-o", exe, "-lm"], check=True)
    return exe


def _run(exe, mode):
    out = subprocess.run([exe, mode], check=True, capture_output=True, text=True, timeout=600).stdout.split()
    return int(out[2]), int(out[4])


def test_one_correction_exact_near_every_midpoint(checker):
    cand, bad = _run(checker, "hard")
    print(f"pairs within 16 units of a midpoint: {cand}, mismatches {bad}")
    assert cand > 10 ** 8 and bad == 0


def test_one_correction_exact_for_every_fp16_divisor(checker):
    cand, bad = _run(checker, "fp16")
    assert cand == 2 * 1024 * 2 * (1 << 23) and bad == 0
