"""The roofline probes of include/fa_probe.h return plausible rates on the
GPU: a positive sustained MFMA rate no higher than the dense bf16 peak at the
top engine clock, and a copy bandwidth below the HBM3E peak."""
import pytest
import torch

import exact_tiled_attention_fwd_amd as fa

pytestmark = pytest.mark.gpu


def test_mfma_probe():
    tf = fa.fa_probe_mfma_bf16(20000)
    assert 100.0 < tf <= 2516.6 * 1.02, tf


def test_copy_probe():
    src = torch.ones(64 << 20, dtype=torch.uint8, device="cuda")
    dst = torch.zeros_like(src)
    gbs = fa.fa_probe_copy(src, dst, 5)
    assert 100.0 < gbs < 8000.0 * 1.05, gbs
    assert torch.equal(src, dst)


def test_copy_probe_rejects_overlap():
    buf = torch.ones(1 << 20, dtype=torch.uint8, device="cuda")
    with pytest.raises(fa.FAError):
        fa.fa_probe_copy(buf[: 1 << 19], buf[1 << 18: (1 << 18) + (1 << 19)], 1)
