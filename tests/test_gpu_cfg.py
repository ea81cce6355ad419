"""Parity of the alternative kernel shapes behind the tuning switches.

FA_FWD_CFG and FA_BWD_CFG (read by the library on every call) select the
kernel shapes that the tile-size comparison keeps. The default shapes are
covered by test_gpu_fwd / test_gpu_bwd; here every other shape meets the same
oracle bar on ragged sizes and all three masks, so that no timed alternative
is an untested one.

Forward, d = 128: 1 = tile kernel 8 waves x 64 keys, 2 = block-pipelined
kernel 128 keys, 3 = block-pipelined 64 keys, 4 = tile kernel 4 waves x 64
keys (the band default is 4 waves x 32 keys; 5, 6: the default). d = 64: 1 = tile kernel 8 x 64, 2 = block-pipelined
128 keys, 3 = tile kernel 8 x 128, 4 = tile kernel 4 x 64, 5 = block-pipelined
64 keys, 6 = the two-block tile kernel at the other workgroup size (4 or 8
waves) than the mask would choose. Backward: 2
swaps the workgroup size (4 or 8 waves) that the mask would otherwise choose.
"""
import pytest

from tests.test_gpu_bwd import run_case as bwd_case
from tests.test_gpu_fwd import run_case as fwd_case, BF16

pytestmark = pytest.mark.gpu

FWD_CASES = [
    ((1, 2, 300, 128), "causal", 0, 1.0),
    ((1, 2, 513, 128), "none", 0, 1.0),
    ((1, 2, 700, 128), "local", 37, 1.0),
    ((1, 2, 600, 128), "local", 128, 8.0),  # large logits: rescale path
    ((2, 2, 257, 64), "causal", 0, 1.0),
    ((1, 2, 777, 64), "local", 64, 1.0),
    ((1, 1, 65, 64), "none", 0, 1.0),
    ((1, 2, 600, 64), "none", 0, 8.0),
]


@pytest.mark.parametrize("cfg", ["1", "2", "3", "4", "5", "6"])
@pytest.mark.parametrize("shape,mask,window,mult", FWD_CASES,
                         ids=[f"{s}-{m}-{w}-x{k:g}" for s, m, w, k in FWD_CASES])
def test_fwd_cfg(monkeypatch, cfg, shape, mask, window, mult):
    monkeypatch.setenv("FA_FWD_CFG", cfg)
    fwd_case(shape, BF16, mask, window, qk_mult=mult, seed=int(cfg) * 1000 + shape[2])


BWD_CASES = [
    ((1, 2, 300, 128), "causal", 0),
    ((1, 2, 400, 128), "local", 1),
    ((1, 1, 513, 128), "none", 0),
    ((2, 2, 130, 64), "causal", 0),
    ((1, 2, 300, 64), "local", 17),
]


@pytest.mark.parametrize("shape,mask,window", BWD_CASES,
                         ids=[f"{s}-{m}-{w}" for s, m, w in BWD_CASES])
def test_bwd_cfg(monkeypatch, shape, mask, window):
    monkeypatch.setenv("FA_BWD_CFG", "2")
    bwd_case(shape, BF16, mask, window, seed=shape[2] + 2)
