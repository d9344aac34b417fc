"""The host half of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

The library is rebuilt with the sanitizers on its host code only (device code
is compiled as usual), and tests/host/sanitized_abi_driver.py drives argument
validation, descriptor building, the 64-bit range arithmetic and the overlap
check with hundreds of fake tensor lists in a child process that preloads the
ASan runtime.  Any sanitizer report aborts the child."""

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "precision_optimizer_state_amd", "csrc", "fo_lib.hip")
HIPCC = "/opt/rocm/bin/hipcc"
# sanitizers on the host pass only
SAN = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-omit-frame-pointer".split()


def _asan_runtime():
    hits = glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    return hits[0] if hits else None


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    if not os.path.exists(HIPCC) or _asan_runtime() is None:
        pytest.skip("hipcc or the ASan runtime is not available")
    sys.path.insert(0, ROOT)
    from precision_optimizer_state_amd._build import FLAGS
    flags = [f for f in FLAGS if f not in ("-O3",)] + ["-O1", "-g", *SAN, "-shared-libsan"]
    out = str(tmp_path_factory.mktemp("asan") / "libfoamd_asan.so")
    r = subprocess.run([HIPCC, *flags, SRC, "-o", out], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    return out


def test_host_paths_clean_under_asan_and_ubsan(sanitized_lib):
    env = dict(os.environ)
    env["LD_PRELOAD"] = _asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    drv = os.path.join(ROOT, "tests", "host", "sanitized_abi_driver.py")
    r = subprocess.run([sys.executable, drv, sanitized_lib, ROOT], capture_output=True, text=True, env=env,
                       timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert "host paths exercised" in out
