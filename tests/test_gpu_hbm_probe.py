"""fo_hbm_probe (the plain streams behind bench.py --ceiling) moves exactly
the bytes it claims, for every chunk size: write fills, copy transforms every
word, the in-place update rewrites every word, read leaves the output alone."""

import pytest
import torch

from precision_optimizer_state_amd import binding as B

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kib", [1, 2, 4, 8])
def test_probe_streams_touch_every_word(kib):
    n = 24 * 1024 * kib                          # 24 chunks
    src = torch.empty(n // 4, dtype=torch.int32, device="cuda")
    dst = torch.zeros(n // 4, dtype=torch.int32, device="cuda")
    B.fo_hbm_probe(src, None, n, "write", 0x12345678, chunk_kib=kib)
    torch.cuda.synchronize()
    assert bool((src == 0x12345678).all())
    B.fo_hbm_probe(dst, src, n, "copy", 0x0F0F0F0F, chunk_kib=kib)
    torch.cuda.synchronize()
    assert bool((dst == (0x12345678 ^ 0x0F0F0F0F)).all())
    B.fo_hbm_probe(dst, None, n, "inplace", 0x0F0F0F0F, chunk_kib=kib)
    torch.cuda.synchronize()
    assert bool((dst == 0x12345678).all())
    before = dst.clone()
    B.fo_hbm_probe(dst, src, n, "read", 0x7FFFFFFF, chunk_kib=kib)   # the XOR of the words never matches
    torch.cuda.synchronize()
    assert torch.equal(dst, before)


def test_probe_rejects_bad_chunks():
    t = torch.zeros(4096, dtype=torch.int32, device="cuda")
    with pytest.raises(B.FoError):
        B.fo_hbm_probe(t, t, 16384, "copy", 0, chunk_kib=3)
    with pytest.raises(B.FoError):
        B.fo_hbm_probe(t, t, 16384 + 1024, "copy", 0, chunk_kib=2)
