"""Thin ctypes binding over libfoamd.so (the C ABI declared in include/foamd.h).

Argument marshalling only: every step of the optimizer runs in the HIP
kernels.  Functions carry the C names.  Tensors are torch tensors living on
the current HIP device; the stream defaults to torch's current stream.  There
is no CPU fallback: if the library is missing the first call raises.
"""

from __future__ import annotations

import ctypes
import os
from ctypes import c_double, c_int, c_int32, c_int64, c_uint32, c_void_p
from typing import Iterable, Mapping, Sequence

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libfoamd.so")

FO_OK, FO_EINVAL, FO_EALIAS, FO_EHIP, FO_ENOMEM = 0, -1, -2, -3, -4
FO_BF16, FO_FP16 = 0, 1
FO_COMPANDED, FO_LINEAR, FO_COMPANDED4, FO_COMPANDED_BF16SCALE = 0, 1, 2, 3
FO_MOMENTUM, FO_VARIANCE = 0, 1

EXPORTS = (
    "fo_split_weights", "fo_reconstruct_weights", "fo_companded_quantize", "fo_dequantize",
    "fo_fused_adamw_step", "fo_fused_adamw_step_noalloc", "fo_fused_sgdm_step", "fo_stream_probe", "fo_hbm_probe",
    "fo_selftest", "fo_cache_pinned", "fo_last_error", "fo_abi_version",
)

WFMT = {"bf16": FO_BF16, "fp16": FO_FP16}
CODEC = {"companded": FO_COMPANDED, "linear": FO_LINEAR, "companded4": FO_COMPANDED4,
         "companded_bf16scale": FO_COMPANDED_BF16SCALE}
KIND = {"m": FO_MOMENTUM, "v": FO_VARIANCE}


class FoError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class AdamWTensor(ctypes.Structure):
    _fields_ = [("w16", c_void_p), ("ecc", c_void_p), ("grad", c_void_p), ("m_q", c_void_p),
                ("m_s", c_void_p), ("v_q", c_void_p), ("v_s", c_void_p), ("n", c_int64)]


class AdamWHParams(ctypes.Structure):
    _fields_ = [("lr", c_double), ("beta1", c_double), ("beta2", c_double), ("eps", c_double),
                ("weight_decay", c_double), ("step", c_int64), ("wfmt", c_int32), ("ecc_bits", c_int32),
                ("codec", c_int32), ("l2_decay", c_int32)]


class SGDMTensor(ctypes.Structure):
    _fields_ = [("w16", c_void_p), ("ecc", c_void_p), ("grad", c_void_p), ("b_q", c_void_p),
                ("b_s", c_void_p), ("n", c_int64)]


class SGDMHParams(ctypes.Structure):
    _fields_ = [("lr", c_double), ("momentum", c_double), ("weight_decay", c_double), ("dampening", c_double),
                ("step", c_int64), ("wfmt", c_int32), ("ecc_bits", c_int32), ("codec", c_int32),
                ("nesterov", c_int32)]


_lib = None
ABI_VERSION = 6          # FO_ABI_VERSION of include/foamd.h (struct layouts below)


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the library (once).  Raises ImportError when it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with __graft_entry__.build() "
                          "(the optimizer has no CPU fallback)")
    lib = ctypes.CDLL(path)
    P = c_void_p
    lib.fo_split_weights.argtypes = [P, c_int64, c_int, c_int, P, P, P]
    lib.fo_reconstruct_weights.argtypes = [P, P, c_int64, c_int, c_int, P, P]
    lib.fo_companded_quantize.argtypes = [P, c_int64, c_int, c_int, P, P, P]
    lib.fo_dequantize.argtypes = [P, P, c_int64, c_int, c_int, P, P]
    lib.fo_fused_adamw_step.argtypes = [ctypes.POINTER(AdamWTensor), c_int32, ctypes.POINTER(AdamWHParams), P]
    lib.fo_fused_adamw_step_noalloc.argtypes = [ctypes.POINTER(AdamWTensor), c_int32, ctypes.POINTER(AdamWHParams), P]
    lib.fo_fused_sgdm_step.argtypes = [ctypes.POINTER(SGDMTensor), c_int32, ctypes.POINTER(SGDMHParams), P]
    lib.fo_stream_probe.argtypes = [ctypes.POINTER(AdamWTensor), c_int32, c_int32, c_int32, c_uint32, P]
    lib.fo_hbm_probe.argtypes = [P, P, c_int64, c_int32, c_int32, c_uint32, P]
    lib.fo_selftest.argtypes = [c_int, c_uint32, ctypes.c_uint64, ctypes.POINTER(ctypes.c_uint64), P]
    for name in EXPORTS:
        getattr(lib, name).restype = c_int
    lib.fo_cache_pinned.argtypes = []
    lib.fo_last_error.restype = ctypes.c_char_p
    lib.fo_last_error.argtypes = []
    lib.fo_abi_version.argtypes = []
    if lib.fo_abi_version() != ABI_VERSION:
        raise ImportError(f"{path} implements C ABI version {lib.fo_abi_version()}, this binding needs "
                          f"{ABI_VERSION}: rebuild it with __graft_entry__.build()")
    _lib = lib
    return lib


def _check(rc: int) -> None:
    if rc != FO_OK:
        raise FoError(rc, load().fo_last_error().decode())


def _stream(stream):
    if stream is not None:
        return c_void_p(int(stream))
    import torch
    return c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t) -> c_void_p:
    """Device address of a contiguous tensor on the current GPU (the library
    launches on the current device and dereferences the address there)."""
    if t is None:
        return c_void_p(0)
    if t.device.type != "cuda":
        raise ValueError(f"tensors passed to the library must live on the GPU (got one on {t.device})")
    import torch
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"a tensor lives on {t.device}, but the current device is "
                         f"cuda:{torch.cuda.current_device()}")
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return c_void_p(t.data_ptr())


def _fmt(x, table):
    return table[x] if isinstance(x, str) else int(x)


# ---------------------------------------------------------------------------
# element-wise entry points
# ---------------------------------------------------------------------------
def fo_split_weights(w32, w16_out, ecc_out, wfmt="bf16", ecc_bits=8, stream=None) -> None:
    _check(load().fo_split_weights(_ptr(w32), w32.numel(), _fmt(wfmt, WFMT), int(ecc_bits),
                                   _ptr(w16_out), _ptr(ecc_out), _stream(stream)))


def fo_reconstruct_weights(w16, ecc, w32_out, wfmt="bf16", ecc_bits=8, stream=None) -> None:
    _check(load().fo_reconstruct_weights(_ptr(w16), _ptr(ecc), w16.numel(), _fmt(wfmt, WFMT), int(ecc_bits),
                                         _ptr(w32_out), _stream(stream)))


def fo_companded_quantize(x, codes_out, scales_out, kind="m", codec="companded", stream=None) -> None:
    _check(load().fo_companded_quantize(_ptr(x), x.numel(), _fmt(kind, KIND), _fmt(codec, CODEC),
                                        _ptr(codes_out), _ptr(scales_out), _stream(stream)))


def fo_dequantize(codes, scales, x_out, kind="m", codec="companded", stream=None) -> None:
    _check(load().fo_dequantize(_ptr(codes), _ptr(scales), x_out.numel(), _fmt(kind, KIND), _fmt(codec, CODEC),
                                _ptr(x_out), _stream(stream)))


# ---------------------------------------------------------------------------
# multi-tensor steps
# ---------------------------------------------------------------------------
class AdamWList:
    """A marshalled tensor list for fo_fused_adamw_step / fo_stream_probe.

    `tensors` is a sequence of mappings with keys w16, ecc, grad, m_q, m_s,
    v_q, v_s (torch tensors).  The ctypes array is built once; the mapping
    objects are kept alive with it.
    """

    def __init__(self, tensors: Sequence[Mapping]):
        self.tensors = list(tensors)
        arr = (AdamWTensor * max(1, len(self.tensors)))()
        for i, t in enumerate(self.tensors):
            arr[i] = AdamWTensor(_ptr(t["w16"]), _ptr(t["ecc"]), _ptr(t["grad"]), _ptr(t["m_q"]),
                                 _ptr(t["m_s"]), _ptr(t["v_q"]), _ptr(t["v_s"]), t["w16"].numel())
        self.array = arr
        self.count = len(self.tensors)

    @classmethod
    def from_rows(cls, rows):
        """A list from raw rows (w16, ecc, grad, m_q, m_s, v_q, v_s, n) of device
        addresses and sizes.  It keeps no tensor alive: the caller guarantees
        the memory outlives every call that uses the list."""
        self = cls.__new__(cls)
        self.tensors = ()
        self.array = (AdamWTensor * max(1, len(rows)))(*[AdamWTensor(*r) for r in rows])
        self.count = len(rows)
        return self

    def __len__(self):
        return self.count


class SGDMList:
    def __init__(self, tensors: Sequence[Mapping]):
        self.tensors = list(tensors)
        arr = (SGDMTensor * max(1, len(self.tensors)))()
        for i, t in enumerate(self.tensors):
            arr[i] = SGDMTensor(_ptr(t["w16"]), _ptr(t["ecc"]), _ptr(t["grad"]), _ptr(t["b_q"]),
                                _ptr(t["b_s"]), t["w16"].numel())
        self.array = arr
        self.count = len(self.tensors)

    @classmethod
    def from_rows(cls, rows):
        """As AdamWList.from_rows with rows (w16, ecc, grad, b_q, b_s, n)."""
        self = cls.__new__(cls)
        self.tensors = ()
        self.array = (SGDMTensor * max(1, len(rows)))(*[SGDMTensor(*r) for r in rows])
        self.count = len(rows)
        return self

    def __len__(self):
        return self.count


def adamw_hparams(lr, beta1, beta2, eps, weight_decay, step, wfmt="bf16", ecc_bits=8, codec="companded",
                  l2_decay=False):
    return AdamWHParams(lr, beta1, beta2, eps, weight_decay, int(step), _fmt(wfmt, WFMT), int(ecc_bits),
                        _fmt(codec, CODEC), int(bool(l2_decay)))


def sgdm_hparams(lr, momentum, weight_decay, step, wfmt="bf16", ecc_bits=8, codec="companded",
                 dampening=0.0, nesterov=False):
    return SGDMHParams(lr, momentum, weight_decay, dampening, int(step), _fmt(wfmt, WFMT), int(ecc_bits),
                       _fmt(codec, CODEC), int(bool(nesterov)))


def fo_fused_adamw_step(tlist, hp, stream=None) -> None:
    """tlist: AdamWList (or a sequence of mappings); hp: AdamWHParams or a mapping
    with lr, beta1, beta2, eps, weight_decay, step and optionally wfmt, ecc_bits, codec."""
    if not isinstance(tlist, AdamWList):
        tlist = AdamWList(tlist)
    if not isinstance(hp, AdamWHParams):
        hp = adamw_hparams(**hp)
    _check(load().fo_fused_adamw_step(tlist.array, len(tlist), ctypes.byref(hp), _stream(stream)))


def fo_fused_adamw_step_noalloc(tlist, hp, stream=None) -> None:
    """fo_fused_adamw_step without any device allocation (the library's fixed
    per-GPU array holds the codec and launch tables; at most 2048 tensors;
    calls on one GPU must not overlap)."""
    if not isinstance(tlist, AdamWList):
        tlist = AdamWList(tlist)
    if not isinstance(hp, AdamWHParams):
        hp = adamw_hparams(**hp)
    _check(load().fo_fused_adamw_step_noalloc(tlist.array, len(tlist), ctypes.byref(hp), _stream(stream)))


def fo_fused_sgdm_step(tlist, hp, stream=None) -> None:
    if not isinstance(tlist, SGDMList):
        tlist = SGDMList(tlist)
    if not isinstance(hp, SGDMHParams):
        hp = sgdm_hparams(**hp)
    _check(load().fo_fused_sgdm_step(tlist.array, len(tlist), ctypes.byref(hp), _stream(stream)))


def fo_stream_probe(tlist, wfmt="bf16", ecc_bits=8, key=0, stream=None) -> None:
    if not isinstance(tlist, AdamWList):
        tlist = AdamWList(tlist)
    _check(load().fo_stream_probe(tlist.array, len(tlist), _fmt(wfmt, WFMT), int(ecc_bits), int(key),
                                  _stream(stream)))


HBM_PROBE_MODES = {"read": 0, "write": 1, "copy": 2, "inplace": 3}


def fo_hbm_probe(dst, src, nbytes, mode="copy", key=0, chunk_kib=8, stream=None) -> None:
    """Measurement only: plain read / write / copy / in-place streams of nbytes
    (a multiple of the chunk) in the fused kernels' access style, one wave
    per chunk of chunk_kib (1, 2, 4 or 8) KiB."""
    _check(load().fo_hbm_probe(_ptr(dst), _ptr(src), int(nbytes), _fmt(mode, HBM_PROBE_MODES), int(chunk_kib),
                               int(key), _stream(stream)))


def fo_selftest(what: int, lo: int, count: int, stream=None) -> int:
    """Mismatch count of the device's fast exact arithmetic: over the f32
    patterns [lo, lo + count) for 0 = reciprocal, 1 = square root,
    2 = float-to-u8, 6 = square root from the successor's estimate; over
    `count` seeded (by lo) pairs for 3 = division (normal quotients),
    4 = division by a block scale, 5 = division with a subnormal quotient
    (outside the fast step's domain)."""
    out = ctypes.c_uint64(0)
    _check(load().fo_selftest(int(what), int(lo), int(count), ctypes.byref(out), _stream(stream)))
    return int(out.value)


def fo_abi_version() -> int:
    return load().fo_abi_version()


def fo_last_error() -> str:
    return load().fo_last_error().decode()
