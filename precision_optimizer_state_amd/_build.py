"""Build the HIP library in-tree (gfx950), and the drop-in optimizers' host
marshalling extension.  Used by __graft_entry__.build()."""

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(PKG, "csrc", "fo_lib.hip")
OUT_DIR = os.path.join(PKG, "lib")
OUT = os.path.join(OUT_DIR, "libfoamd.so")

# -ffp-contract=off: every float operation is rounded once (no FMA formation),
# which the fixed operation order of the update relies on.  Division and square
# root stay IEEE correctly rounded, denormals are preserved.  Packed-FP32
# instruction selection is disabled.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-variable", "-Wno-unknown-pragmas",
]


def build(verbose: bool = False, extra=()) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    tmp = OUT + ".tmp"
    cmd = ["/opt/rocm/bin/hipcc", *FLAGS, *extra, SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libfoamd.so")
    if verbose and res.stderr.strip():
        print("\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)[:4000])
    os.replace(tmp, OUT)
    return OUT


MARSHAL_SRC = os.path.join(PKG, "csrc", "fo_marshal.cpp")
MARSHAL_OUT = os.path.join(OUT_DIR, "fo_marshal.so")


def build_marshal(verbose: bool = False, out: str = MARSHAL_OUT) -> str:
    """Compile csrc/fo_marshal.cpp (host C++, torch headers) into `out`
    (lib/fo_marshal.so) with the flags torch's own C++ extensions use."""
    import sysconfig

    import torch
    from torch.utils import cpp_extension as ce

    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp"
    libdirs = ce.library_paths()
    # the defines are those torch.utils.cpp_extension.CppExtension passes for
    # this (ROCm) build of torch, so its headers see the configuration they
    # were built with; the source itself is host C++ with no GPU code
    cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-Wall",
           f"-D_GLIBCXX_USE_CXX11_ABI={int(torch._C._GLIBCXX_USE_CXX11_ABI)}",
           "-DTORCH_API_INCLUDE_EXTENSION_H", "-DTORCH_EXTENSION_NAME=fo_marshal",
           "-D__HIP_PLATFORM_AMD__=1", "-DUSE_ROCM=1",
           *[f"-I{d}" for d in ce.include_paths()], f"-I{sysconfig.get_paths()['include']}",
           MARSHAL_SRC, "-o", tmp,
           *[f"-L{d}" for d in libdirs], *[f"-Wl,-rpath,{d}" for d in libdirs],
           "-lc10", "-ltorch", "-ltorch_cpu", "-ltorch_python"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("g++ failed building fo_marshal.so")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_marshal(verbose=True))
