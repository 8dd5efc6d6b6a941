"""The measured-peak microbenchmarks (include/mla_peaks.h) run on the GPU and
read what they are given: the register-load read of a buffer of zeros folds
to zero, of a buffer with one nonzero 16-byte chunk to that chunk's fold."""

import pytest
import torch

from decode_attention_03_amd import _lib

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def test_peak_read_folds_the_data():
    print("[peaks] read fold", flush=True)
    buf = torch.zeros(64 << 20, dtype=torch.uint8, device=DEV)
    sink = torch.full((64,), -1, dtype=torch.int32, device=DEV)
    _lib.peak_hbm_read(buf, _lib.PEAK_READ_VGPR, sink, 64)
    torch.cuda.synchronize()
    assert (sink == 0).all()
    # one chunk of four words a, b, c, d, read by thread 1 of workgroup 5 (chunk
    # 256 * 5 + 1 in the first grid-stride round): it folds a ^ b ^ c ^ d, and
    # the workgroup's word folds lanes 0..2 of its first wave
    words = torch.tensor([0x11, 0x2200, 0x330000, 0x44000000], dtype=torch.int32)
    c = 256 * 5 + 1
    buf.view(torch.int32)[4 * c:4 * c + 4] = words.to(DEV)
    sink.fill_(-1)
    _lib.peak_hbm_read(buf, _lib.PEAK_READ_VGPR, sink, 64)
    torch.cuda.synchronize()
    got = [int(x) & 0xFFFFFFFF for x in sink.cpu()]
    assert got[5] == 0x44332211 and all(v == 0 for i, v in enumerate(got) if i != 5)


def test_peak_kernels_run():
    print("[peaks] lds read and mfma", flush=True)
    buf = torch.ones(16 << 20, dtype=torch.uint8, device=DEV)
    isink = torch.zeros(1024, dtype=torch.int32, device=DEV)
    fsink = torch.zeros(1024, dtype=torch.float32, device=DEV)
    _lib.peak_hbm_read(buf, _lib.PEAK_READ_LDS, isink, 256)
    _lib.peak_mfma(_lib.PEAK_MFMA_FP8, 16, fsink, 256)
    _lib.peak_mfma(_lib.PEAK_MFMA_BF16, 16, fsink, 256)
    torch.cuda.synchronize()
    assert (fsink == 0).all()
