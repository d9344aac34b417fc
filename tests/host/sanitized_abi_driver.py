"""Drives the host-side logic of the C ABI (argument validation, descriptor
building with 64-bit range arithmetic, the overlap check) with fake but
well-formed device addresses, no GPU needed.  Run by
tests/test_abi_sanitized.py in a subprocess against a library whose host
code is built with AddressSanitizer and UndefinedBehaviorSanitizer; any
report aborts the process.  Without a device the entry points stop at their
first HIP call with FO_EHIP, after the host logic has run."""

import ctypes
import random
import sys

sys.path.insert(0, sys.argv[2])
from precision_optimizer_state_amd import binding as B  # noqa: E402

lib = B.load(sys.argv[1])
assert hasattr(ctypes.CDLL(None), "__asan_init"), "the AddressSanitizer runtime is not loaded"
rng = random.Random(1234)
BASE = 1 << 44
P = ctypes.c_void_p


def fake_adamw_list(sizes, overlap=False, misalign=False):
    arr = (B.AdamWTensor * max(1, len(sizes)))()
    addr = BASE
    for i, n in enumerate(sizes):
        fields = []
        for nbytes in (2 * n, n, 2 * n, n, 2 * ((n + 31) // 32), n, 2 * ((n + 31) // 32)):
            fields.append(addr)
            addr += (nbytes + 255) // 256 * 256 + 256
        if overlap and i == len(sizes) - 1 and len(sizes) > 1:
            fields[3] = arr[0].m_q                      # reuse tensor 0's momentum codes
        if misalign and i == len(sizes) // 2:
            fields[0] += 2
        arr[i] = B.AdamWTensor(*fields, n)
    return arr


def fake_sgdm_list(sizes):
    arr = (B.SGDMTensor * max(1, len(sizes)))()
    addr = BASE
    for i, n in enumerate(sizes):
        fields = []
        for nbytes in (2 * n, n, 2 * n, n, 2 * ((n + 31) // 32)):
            fields.append(addr)
            addr += (nbytes + 255) // 256 * 256 + 256
        arr[i] = B.SGDMTensor(*fields, n)
    return arr


def overlaps(arr, sizes):
    """Brute-force overlap test of the arrays of the non-empty tensors."""
    spans = []
    for i, n in enumerate(sizes):
        if n == 0:
            continue
        t = arr[i]
        nb = (n + 31) // 32
        for p, nbytes in ((t.w16, 2 * n), (t.ecc, n), (t.grad, 2 * n), (t.m_q, n), (t.m_s, 2 * nb),
                          (t.v_q, n), (t.v_s, 2 * nb)):
            spans.append((p, p + nbytes))
    return any(a[0] < b[1] and b[0] < a[1] for k, a in enumerate(spans) for b in spans[k + 1:])


hp = B.adamw_hparams(1e-3, 0.9, 0.999, 1e-8, 0.01, 3)
hp_l2 = B.adamw_hparams(1e-3, 0.9, 0.999, 1e-8, 0.01, 3, l2_decay=True)
sh = B.sgdm_hparams(0.1, 0.9, 1e-4, 2, nesterov=True)
seen = set()
for trial in range(300):
    count = rng.choice([1, 2, 3, 17, 64, 291, 300])
    sizes = [rng.choice([0, 1, 31, 32, 33, 2047, 2048, 2049, rng.randrange(1, 1 << 24),
                         (1 << 31) + 77, 1 << 40]) for _ in range(count)]
    kind = trial % 5
    if kind == 0:
        rc = lib.fo_fused_adamw_step(fake_adamw_list(sizes), count, ctypes.byref(hp if trial % 8 else hp_l2), None)
        want = {B.FO_EHIP} if any(sizes) else {B.FO_OK}
    elif kind == 1:
        lst = fake_adamw_list(sizes, overlap=True)
        rc = lib.fo_fused_adamw_step(lst, count, ctypes.byref(hp), None)
        want = {B.FO_EALIAS} if overlaps(lst, sizes) else ({B.FO_EHIP} if any(sizes) else {B.FO_OK})
    elif kind == 2:
        rc = lib.fo_fused_adamw_step(fake_adamw_list(sizes, misalign=True), count, ctypes.byref(hp), None)
        want = {B.FO_EINVAL} if sizes[count // 2] else ({B.FO_EHIP} if any(sizes) else {B.FO_OK})
    elif kind == 3:
        rc = lib.fo_fused_sgdm_step(fake_sgdm_list(sizes), count, ctypes.byref(sh), None)
        want = {B.FO_EHIP} if any(sizes) else {B.FO_OK}
    else:
        # the allocation-free entry point: the same validation into its static
        # host arrays, then its first device call
        lst = fake_adamw_list(sizes, overlap=trial % 10 == 4)
        rc = lib.fo_fused_adamw_step_noalloc(lst, count, ctypes.byref(hp), None)
        want = {B.FO_EALIAS} if overlaps(lst, sizes) else ({B.FO_EHIP} if any(sizes) else {B.FO_OK})
    assert rc in want, (trial, kind, sizes[:5], rc, want, B.fo_last_error())
    seen.add((kind, rc))
    assert isinstance(B.fo_last_error(), str)

# the allocation-free entry point takes at most 2048 tensors, and a full-size
# list fills its static descriptor and range arrays to the end
assert lib.fo_fused_adamw_step_noalloc(fake_adamw_list([64] * 2049), 2049, ctypes.byref(hp), None) == B.FO_EINVAL
assert lib.fo_fused_adamw_step_noalloc(fake_adamw_list([2049] * 2048), 2048, ctypes.byref(hp), None) == B.FO_EHIP
assert lib.fo_cache_pinned() == 0

# the bandwidth probe validates mode, chunk and size before its first device call
assert lib.fo_hbm_probe(P(BASE), P(BASE + (1 << 40)), 1 << 20, 4, 8, 0, None) == B.FO_EINVAL
assert lib.fo_hbm_probe(P(BASE), P(BASE + (1 << 40)), 1 << 20, 2, 3, 0, None) == B.FO_EINVAL
assert lib.fo_hbm_probe(P(BASE), P(BASE + (1 << 40)), (1 << 20) + 1024, 2, 2, 0, None) == B.FO_EINVAL
assert lib.fo_hbm_probe(P(BASE), None, 1 << 20, 3, 1, 0, None) == B.FO_EHIP

# element counts beyond any device memory are rejected before any size arithmetic
for huge in ((1 << 56) + 1, 1 << 62, (1 << 63) - 1):
    assert lib.fo_fused_adamw_step(fake_adamw_list([33, huge]), 2, ctypes.byref(hp), None) == B.FO_EINVAL
    assert lib.fo_fused_sgdm_step(fake_sgdm_list([huge]), 1, ctypes.byref(sh), None) == B.FO_EINVAL
    assert lib.fo_split_weights(P(BASE), huge, B.FO_BF16, 8, P(BASE), P(BASE), None) == B.FO_EINVAL
    assert lib.fo_dequantize(P(BASE), P(BASE), huge, 0, 0, P(BASE), None) == B.FO_EINVAL

# element-wise entry points: validation and the overlap check on their arrays
for n in (1, 33, 4096, (1 << 31) + 5):
    step = (16 * n + 511) // 256 * 256            # disjoint regions, each larger than any array

    def at(k):
        return P(BASE + k * step)

    rc = lib.fo_split_weights(at(0), n, B.FO_BF16, 8, at(1), at(2), None)
    assert rc == B.FO_EHIP, (n, rc, B.fo_last_error())
    rc = lib.fo_split_weights(at(0), n, B.FO_BF16, 8, P(BASE + (16 if n > 4 else 0)), at(2), None)
    assert rc == B.FO_EALIAS, (n, rc, B.fo_last_error())
    rc = lib.fo_companded_quantize(at(0), n, 1, 0, at(1), at(2), None)
    assert rc == B.FO_EHIP, (n, rc, B.fo_last_error())
    rc = lib.fo_reconstruct_weights(at(0), at(1), n, B.FO_FP16, 8, at(2), None)
    assert rc == B.FO_EHIP, (n, rc, B.fo_last_error())
    rc = lib.fo_dequantize(at(0), at(1), n, 0, 1, at(2), None)
    assert rc == B.FO_EHIP, (n, rc, B.fo_last_error())
print("host paths exercised:", sorted(seen), flush=True)
