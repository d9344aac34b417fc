"""The drop-in optimizers' host marshalling extension (csrc/fo_marshal.cpp)
on the CPU: fill_rows writes the same launch rows as the Python formula
(w, ecc, grad, the rest of the fixed row), and refuses, with 1 + the index,
the first parameter whose gradient is missing, of another dtype, not
contiguous or of another size.  The extension reads addresses only, so CPU
tensors serve."""

import ctypes
import importlib.util
import os
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def fill_rows(tmp_path_factory):
    sys.path.insert(0, ROOT)
    from precision_optimizer_state_amd import _build
    path = _build.MARSHAL_OUT
    if not os.path.exists(path):
        path = _build.build_marshal(out=str(tmp_path_factory.mktemp("marshal") / "fo_marshal.so"))
    spec = importlib.util.spec_from_file_location("fo_marshal", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod.fill_rows


def _params(sizes, dt=torch.bfloat16):
    ps = []
    for n in sizes:
        p = torch.nn.Parameter(torch.zeros(n, dtype=dt))
        p.grad = torch.zeros(n, dtype=dt)
        ps.append(p)
    return ps


@pytest.mark.parametrize("k", [6, 4], ids=["adamw_rows", "sgdm_rows"])
def test_rows_match_the_python_formula(fill_rows, k):
    sizes = [1, 31, 32, 4097, 77]
    ps = _params(sizes)
    fixed = [tuple(1000 * i + j for j in range(k - 1)) + (n,) for i, n in enumerate(sizes)]
    buf = (ctypes.c_int64 * (len(ps) * (k + 2)))()
    assert fill_rows(ps, torch.tensor(fixed, dtype=torch.int64), ctypes.addressof(buf), torch.bfloat16) == 0
    got = [tuple(buf[i * (k + 2):(i + 1) * (k + 2)]) for i in range(len(ps))]
    want = [(p.data_ptr(), f[0], p.grad.data_ptr()) + f[1:] for p, f in zip(ps, fixed)]
    assert got == want


def test_refusals_name_the_first_bad_parameter(fill_rows):
    k = 6
    fixed = torch.tensor([(1, 2, 3, 4, 5, 64)] * 4, dtype=torch.int64)
    buf = (ctypes.c_int64 * (4 * (k + 2)))()
    addr = ctypes.addressof(buf)
    ps = _params([64] * 4)
    assert fill_rows(ps, fixed, addr, torch.bfloat16) == 0
    assert fill_rows(ps, fixed, addr, torch.float16) == 1            # another weight format
    ps[2].grad = None
    assert fill_rows(ps, fixed, addr, torch.bfloat16) == 3           # missing gradient
    ps[2].grad_dtype = None                                          # (torch refuses it otherwise)
    ps[2].grad = torch.zeros(64, dtype=torch.float16)
    assert fill_rows(ps, fixed, addr, torch.bfloat16) == 3           # gradient of another dtype
    ps[2].grad = torch.zeros(128, dtype=torch.bfloat16)[::2]
    assert fill_rows(ps, fixed, addr, torch.bfloat16) == 3           # not contiguous
    ps[2].grad = torch.zeros(64, dtype=torch.bfloat16)
    ps[1].data = torch.zeros(65, dtype=torch.bfloat16)               # gradient no longer of the parameter's size
    assert fill_rows(ps, fixed, addr, torch.bfloat16) == 2
    with pytest.raises(RuntimeError):
        fill_rows(ps, fixed[:3], addr, torch.bfloat16)               # one fixed row per parameter
    with pytest.raises(RuntimeError):
        fill_rows(ps, fixed.to(torch.int32), addr, torch.bfloat16)   # int64 fixed rows
