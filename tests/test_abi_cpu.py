"""The C-ABI library loads and exports every symbol include/foamd.h declares,
and host-side argument validation fails before any GPU work (CPU only: no
compute call reaches a kernel here)."""

import ctypes
import os
import re

import pytest

from precision_optimizer_state_amd import binding as B

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "foamd.h")


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\s*\*)\s+(fo_\w+)\s*\(", src, re.M)))


def test_library_exports_every_declared_symbol():
    lib = B.load()
    names = _declared()
    assert len(names) >= 9
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(B.EXPORTS)
    assert lib.fo_abi_version() == B.ABI_VERSION == 6


def test_struct_layouts_match_header():
    assert ctypes.sizeof(B.AdamWTensor) == 64
    assert ctypes.sizeof(B.AdamWHParams) == 64
    assert ctypes.sizeof(B.SGDMTensor) == 48
    assert ctypes.sizeof(B.SGDMHParams) == 56


def _rc(fn, *args):
    return fn(*args)


def test_invalid_arguments_are_rejected_on_the_host():
    lib = B.load()
    P = ctypes.c_void_p
    # unsupported format/ECC combination, n < 0, NULL pointers, misalignment
    assert lib.fo_split_weights(P(16), 8, B.FO_FP16, 16, P(16), P(16), None) == B.FO_EINVAL
    assert "unsupported" in B.fo_last_error()
    assert lib.fo_split_weights(P(16), -1, B.FO_BF16, 8, P(16), P(16), None) == B.FO_EINVAL
    assert lib.fo_split_weights(None, 8, B.FO_BF16, 8, P(16), P(16), None) == B.FO_EINVAL
    assert lib.fo_split_weights(P(18), 8, B.FO_BF16, 8, P(4096), P(8192), None) == B.FO_EINVAL
    assert "aligned" in B.fo_last_error()
    # overlapping output arrays are rejected before launch
    assert lib.fo_split_weights(P(4096), 64, B.FO_BF16, 8, P(4096 + 64), P(1 << 20), None) == B.FO_EALIAS
    assert lib.fo_companded_quantize(P(16), 8, 7, 0, P(16), P(16), None) == B.FO_EINVAL
    assert lib.fo_dequantize(P(16), P(16), 8, 0, 9, P(16), None) == B.FO_EINVAL
    # n == 0 is a no-op
    assert lib.fo_split_weights(None, 0, B.FO_BF16, 8, None, None, None) == B.FO_OK
    assert lib.fo_reconstruct_weights(None, None, 0, B.FO_BF16, 16, None, None) == B.FO_OK


def test_step_hparams_are_validated():
    lib = B.load()
    t = (B.AdamWTensor * 1)()
    hp = B.adamw_hparams(1e-3, 0.9, 0.999, 1e-8, 0.0, 0)
    assert lib.fo_fused_adamw_step(t, 1, ctypes.byref(hp), None) == B.FO_EINVAL      # step 0
    hp = B.adamw_hparams(1e-3, 1.5, 0.999, 1e-8, 0.0, 1)
    assert lib.fo_fused_adamw_step(t, 1, ctypes.byref(hp), None) == B.FO_EINVAL      # beta1 >= 1
    hp = B.adamw_hparams(1e-3, 0.9, 0.999, 1e-8, 0.0, 1, wfmt="fp16", ecc_bits=16)
    assert lib.fo_fused_adamw_step(t, 1, ctypes.byref(hp), None) == B.FO_EINVAL
    hp = B.adamw_hparams(1e-3, 0.9, 0.999, 1e-8, 0.0, 1)
    assert lib.fo_fused_adamw_step(t, -1, ctypes.byref(hp), None) == B.FO_EINVAL
    assert lib.fo_fused_adamw_step(None, 3, ctypes.byref(hp), None) == B.FO_EINVAL
    assert lib.fo_fused_adamw_step(t, 0, ctypes.byref(hp), None) == B.FO_OK          # empty list
    sh = B.sgdm_hparams(0.1, 0.9, 1e-4, 1, codec=5)
    s = (B.SGDMTensor * 1)()
    assert lib.fo_fused_sgdm_step(s, 1, ctypes.byref(sh), None) == B.FO_EINVAL


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(ImportError):
        B._lib_saved = B._lib
        try:
            B._lib = None
            B.load(str(tmp_path / "missing.so"))
        finally:
            B._lib = B._lib_saved


def test_binding_rejects_host_tensors():
    # the binding hands the library device addresses only: a host tensor is
    # refused before any call (no GPU needed to check)
    import torch
    w = torch.zeros(64, dtype=torch.float32)
    st = {k: torch.zeros(64, dtype=torch.uint8) for k in ("w16", "ecc", "grad", "m_q", "m_s", "v_q", "v_s")}
    with pytest.raises(ValueError, match="GPU"):
        B.fo_split_weights(w, st["w16"], st["ecc"])
    with pytest.raises(ValueError, match="GPU"):
        B.AdamWList([st])
    with pytest.raises(ValueError, match="GPU"):
        B.SGDMList([{k: st[k] for k in ("w16", "ecc", "grad", "m_q", "m_s")} | {"b_q": st["m_q"], "b_s": st["m_s"]}])


def test_4bit_code_arrays_are_validated_at_half_size():
    """Under FO_COMPANDED4 a code array spans ceil(n/2) bytes: two code arrays
    n/2 bytes apart are disjoint there (validation passes; with no GPU the
    call then fails at the device, not with FO_EALIAS) and overlap under the
    8-bit codecs (FO_EALIAS).  The same extents hold for quantize."""
    lib = B.load()
    P = ctypes.c_void_p
    n = 4096
    base = 1 << 24
    w16, ecc, grad, mq, ms, vs = base, base + 2 * n, base + 3 * n, base + 5 * n, base + 7 * n, base + 8 * n
    vq = mq + n // 2
    t = (B.AdamWTensor * 1)(B.AdamWTensor(w16, ecc, grad, mq, ms, vq, vs, n))
    for codec, alias in (("companded4", False), ("companded", True), ("linear", True), ("companded_bf16scale", True)):
        hp = B.adamw_hparams(1e-3, 0.9, 0.999, 1e-8, 0.0, 1, codec=codec)
        rc = lib.fo_fused_adamw_step(t, 1, ctypes.byref(hp), None)
        assert (rc == B.FO_EALIAS) == alias, (codec, rc, B.fo_last_error())
        assert rc != B.FO_OK
    # n - 1 = 4095 codes: 2048 bytes at 4 bits, so the SGD-M buffer ends at vq
    s2 = (B.SGDMTensor * 2)(B.SGDMTensor(w16, ecc, grad, mq, ms, n - 1),
                            B.SGDMTensor(w16 + (1 << 20), ecc + (1 << 20), grad + (1 << 20), vq, vs, 16))
    for codec, alias in (("companded4", False), ("companded", True)):
        sh = B.sgdm_hparams(0.1, 0.9, 1e-4, 1, codec=codec)
        rc = lib.fo_fused_sgdm_step(s2, 2, ctypes.byref(sh), None)
        assert (rc == B.FO_EALIAS) == alias, (codec, rc, B.fo_last_error())
    # quantize: codes of ceil(n/2) bytes right below the input are disjoint at 4 bits only
    x = base + (1 << 20)
    assert lib.fo_companded_quantize(P(x), n, 0, B.FO_COMPANDED, P(x - n // 2), P(base), None) == B.FO_EALIAS
    assert lib.fo_companded_quantize(P(x), n, 0, B.FO_COMPANDED4, P(x - n // 2), P(base), None) != B.FO_EALIAS
    assert lib.fo_companded_quantize(P(x), n, 0, B.FO_COMPANDED_BF16SCALE, P(x - n // 2), P(base),
                                     None) == B.FO_EALIAS
    assert lib.fo_companded_quantize(P(x), n, 0, 4, P(x - n // 2), P(base), None) == B.FO_EINVAL
    assert lib.fo_dequantize(P(x - n // 2), P(base), n, 1, B.FO_COMPANDED4, P(x), None) != B.FO_EALIAS
    assert lib.fo_dequantize(P(x - n // 2), P(base), n, 1, B.FO_COMPANDED, P(x), None) == B.FO_EALIAS
