"""Parity of the alternative kernel shapes behind the tuning entry points.

fa_fwd_tuned and fa_bwd_tuned (include/fa_tuning.h) run the same attention
with an explicitly chosen kernel shape; fa_fwd / fa_bwd always run the
default, which test_gpu_fwd / test_gpu_bwd cover. Here every other shape meets
the same oracle bar on ragged sizes and all three masks, so that no timed
alternative is an untested one. cfg 7 and 8 are the tile that "What the
tiling is actually constrained by" derives from the on-chip memory
(B_c = ceil(M / 4d): 160 keys at d = 128, 320 at d = 64), once with its
B_r = min(B_c, d) rows in the tile kernel and once at 256 rows in the
block-pipelined kernel. The header lists what each cfg selects.
"""
import pytest
import torch

from exact_tiled_attention_fwd_amd import FAError, fa_bwd_tuned, fa_fwd_tuned
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


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5, 6, 7, 8, 9])
@pytest.mark.parametrize("shape,mask,window,mult", FWD_CASES,
                         ids=[f"{s}-{m}-{w}-x{k:g}" for s, m, w, k in FWD_CASES])
def test_fwd_cfg(cfg, shape, mask, window, mult):
    fwd_case(shape, BF16, mask, window, qk_mult=mult, seed=cfg * 1000 + shape[2], cfg=cfg)


# the derived tiles span several key tiles and a ragged tail at these lengths
@pytest.mark.parametrize("cfg", [7, 8])
@pytest.mark.parametrize("shape,mask", [((1, 2, 1000, 128), "causal"), ((1, 1, 1401, 64), "none"),
                                        ((1, 2, 1000, 64), "causal")])
def test_fwd_derived_tile_long(cfg, shape, mask):
    fwd_case(shape, BF16, mask, 0, seed=cfg + shape[2], cfg=cfg)


# cfg 9 (ping-pong schedule): an odd and an even number of key tiles, one
# tile, the band, and rows past the last full workgroup
@pytest.mark.parametrize("shape,mask,window", [((1, 2, 1000, 128), "causal", 0),
                                               ((1, 2, 1100, 128), "none", 0),
                                               ((1, 1, 100, 128), "none", 0),
                                               ((1, 2, 1500, 128), "local", 200),
                                               ((1, 2, 1000, 64), "causal", 0),
                                               ((1, 1, 1401, 64), "none", 0),
                                               ((1, 2, 999, 64), "local", 100)])
def test_fwd_pingpong_long(shape, mask, window):
    fwd_case(shape, BF16, mask, window, seed=9 + shape[2], cfg=9)


BWD_CASES = [
    ((1, 2, 300, 128), "causal", 0),
    ((1, 2, 400, 128), "local", 1),
    ((1, 1, 513, 128), "none", 0),
    ((2, 2, 130, 64), "causal", 0),
    ((1, 2, 300, 64), "local", 17),
]


@pytest.mark.parametrize("shape,mask,window", BWD_CASES,
                         ids=[f"{s}-{m}-{w}" for s, m, w in BWD_CASES])
def test_bwd_cfg(shape, mask, window):
    bwd_case(shape, BF16, mask, window, seed=shape[2] + 2, cfg=2)


def test_unknown_cfg_rejected():
    q = torch.zeros((1, 1, 8, 64), dtype=BF16, device="cuda")
    o, lse = torch.empty_like(q), torch.empty((1, 1, 8), dtype=torch.float32, device="cuda")
    for bad in (-1, 10, 100):
        with pytest.raises(FAError):
            fa_fwd_tuned(q, q.clone(), q.clone(), o, lse, 0.125, None, 0, bad)
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    g = [torch.empty_like(q) for _ in range(3)]
    with pytest.raises(FAError):
        fa_bwd_tuned(q, q.clone(), q.clone(), o, q.clone(), lse, *g, ws, 0.125, None, 0, 1)
