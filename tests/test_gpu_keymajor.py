"""Parity of the key-major forward, fa_fwd_keymajor (outer loop over key
blocks, running state in device memory), against the CPU oracle on the same
seeded inputs, with fa_fwd's tolerances, for every supported key-block size."""
import math

import pytest
import torch

import oracle
from exact_tiled_attention_fwd_amd import (FAError, fa_fwd_keymajor,
                                           fa_fwd_keymajor_workspace_bytes)
from exact_tiled_attention_fwd_amd.synth import random_inputs
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

BF16 = torch.bfloat16


def run_km(shape, mask, window, bc, scale=None, qk_mult=1.0, seed=0):
    B, H, N, d = shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    inp = random_inputs(shape, BF16, seed=seed, qk_mult=qk_mult)
    q, k, v = (G.to_dev(inp[n]) for n in ("q", "k", "v"))
    print(f"key-major case shape={shape} mask={mask} w={window} bc={bc} scale={scale}", flush=True)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(fa_fwd_keymajor_workspace_bytes(B, H, N, d, BF16), dtype=torch.uint8,
                     device="cuda")
    fa_fwd_keymajor(q, k, v, o, lse, ws, scale, mask, window, bc)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.fwd_dense(inp["q"], inp["k"], inp["v"], scale, mask, window)
    return G.check_fwd(o, lse, o_ref, lse_ref, BF16, f"key-major {shape} {mask} {window} bc={bc}")


CASES = [
    ((1, 1, 1, 128), "none", 0, 32),
    ((1, 2, 6, 64), "causal", 0, 64),
    ((2, 3, 17, 128), "causal", 0, 128),
    ((1, 2, 300, 128), "none", 0, 32),
    ((1, 2, 300, 128), "causal", 0, 64),
    ((1, 2, 513, 64), "none", 0, 256),
    ((1, 2, 700, 128), "local", 1, 64),
    ((1, 2, 1000, 64), "local", 128, 128),
    ((2, 2, 257, 64), "causal", 0, 32),
]


@pytest.mark.parametrize("shape,mask,window,bc", CASES,
                         ids=[f"{s}-{m}-{w}-bc{b}" for s, m, w, b in CASES])
def test_keymajor_small(shape, mask, window, bc):
    run_km(shape, mask, window, bc, seed=sum(shape) + window + bc)


@pytest.mark.parametrize("scale", [0.0, -0.25, 2.0])
def test_keymajor_scales(scale):
    run_km((1, 2, 200, 128), "causal", 0, 64, scale=scale, seed=21)


def test_keymajor_large_logits():
    # the running reference moves between launches: logits with std ~64
    run_km((1, 2, 600, 128), "local", 128, 64, qk_mult=8.0, seed=22)
    run_km((1, 2, 600, 64), "none", 0, 32, qk_mult=8.0, seed=23)


def test_keymajor_errors():
    q = torch.zeros(1, 1, 8, 128, dtype=BF16, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty(1, 1, 8, dtype=torch.float32, device="cuda")
    ws = torch.empty(fa_fwd_keymajor_workspace_bytes(1, 1, 8, 128, BF16), dtype=torch.uint8,
                     device="cuda")
    with pytest.raises(FAError):
        fa_fwd_keymajor(q, q, q, o, lse, ws, 0.1, block_keys=256)   # 256 needs d = 64
    with pytest.raises(FAError):
        fa_fwd_keymajor(q, q, q, o, lse, ws[:16], 0.1, block_keys=64)
