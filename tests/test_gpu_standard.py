"""Parity of the standard (unfused) attention baseline, fa_fwd_standard
(S, P and O through device memory), against the CPU oracle on the same
seeded inputs, with the same tolerances as fa_fwd."""
import math

import numpy as np
import pytest
import torch

import oracle
from exact_tiled_attention_fwd_amd import (FAError, fa_fwd_standard,
                                           fa_fwd_standard_workspace_bytes)
from exact_tiled_attention_fwd_amd.synth import random_inputs
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

BF16 = torch.bfloat16


def run_std(shape, mask, window, scale=None, qk_mult=1.0, seed=0):
    B, H, N, d = shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    inp = random_inputs(shape, BF16, seed=seed, qk_mult=qk_mult)
    q, k, v = (G.to_dev(inp[n]) for n in ("q", "k", "v"))
    print(f"standard case shape={shape} mask={mask} w={window} scale={scale}", flush=True)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(fa_fwd_standard_workspace_bytes(B, H, N, d, BF16), dtype=torch.uint8,
                     device="cuda")
    fa_fwd_standard(q, k, v, o, lse, ws, scale, mask, window)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.fwd_dense(inp["q"], inp["k"], inp["v"], scale, mask, window)
    return G.check_fwd(o, lse, o_ref, lse_ref, BF16, f"standard {shape} {mask} {window}")


CASES = [
    ((1, 1, 1, 128), "none", 0),
    ((1, 2, 6, 64), "none", 0),
    ((2, 3, 17, 128), "causal", 0),
    ((1, 2, 129, 128), "none", 0),     # one past a 128-key score tile
    ((2, 2, 300, 128), "causal", 0),   # N not a multiple of 4 or 8: padded rows
    ((1, 3, 513, 64), "none", 0),
    ((1, 2, 700, 128), "local", 1),
    ((1, 2, 1000, 64), "local", 128),
    ((1, 2, 1001, 64), "causal", 0),
]


@pytest.mark.parametrize("shape,mask,window", CASES, ids=[f"{s}-{m}-{w}" for s, m, w in CASES])
def test_standard_small(shape, mask, window):
    run_std(shape, mask, window, seed=sum(shape) + window + 1)


@pytest.mark.parametrize("scale", [0.0, -0.25, 2.0])
def test_standard_scales(scale):
    run_std((1, 2, 200, 64), "causal", 0, scale=scale, seed=11)


def test_standard_large_logits():
    run_std((1, 2, 600, 128), "none", 0, qk_mult=8.0, seed=12)


def test_standard_matches_fused_at_2048():
    """The standard baseline and the fused forward on P3's N=2048, d=64
    setting (one head of [1, 16, 2048, 64]): both within the oracle's
    tolerance on sampled rows, and within twice of it of each other."""
    from exact_tiled_attention_fwd_amd import attention_fwd
    shape = (1, 16, 2048, 64)
    inp = random_inputs(shape, BF16, seed=13)
    q, k, v = (G.to_dev(inp[n]) for n in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty(shape[:3], dtype=torch.float32, device="cuda")
    ws = torch.empty(fa_fwd_standard_workspace_bytes(*shape, BF16), dtype=torch.uint8, device="cuda")
    fa_fwd_standard(q, k, v, o, lse, ws, 0.125, "none", 0)
    o2, lse2 = attention_fwd(q, k, v, 0.125, "none", 0)
    torch.cuda.synchronize()
    bh, rows, heads = G.sample_rows(16, 2048, 24, seed=14)
    o_ref, lse_ref = G.oracle_rows(inp, 0.125, "none", 0, bh, rows, heads)
    for oo, ll, what in ((o, lse, "standard"), (o2, lse2, "fused")):
        G.check_fwd(oo.reshape(16, 2048, 64)[bh, rows], ll.reshape(16, 2048)[bh, rows],
                    o_ref, lse_ref, BF16, what)
    d = (o.float() - o2.float()).abs().max().item()
    assert d <= 2 * G.TOL_O[BF16], d


def test_standard_errors():
    q = torch.zeros(1, 1, 8, 64, dtype=BF16, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty(1, 1, 8, dtype=torch.float32, device="cuda")
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(FAError):
        fa_fwd_standard(q, q, q, o, lse, small, 0.125)
    qf = torch.zeros(1, 1, 8, 64, dtype=torch.float32, device="cuda")
    ws = torch.empty(1 << 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(FAError):
        fa_fwd_standard(qf, qf, qf, torch.empty_like(qf), lse, ws, 0.125)


# ---------------------------------------------------------------- backward
def run_std_bwd(shape, mask, window, scale=None, qk_mult=1.0, seed=0):
    """fa_fwd_standard then fa_bwd_standard (reading the stored P) against
    the oracle's dense backward: relative Frobenius error of each gradient."""
    from exact_tiled_attention_fwd_amd import fa_bwd_standard, fa_bwd_standard_workspace_bytes
    B, H, N, d = shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    inp = random_inputs(shape, BF16, seed=seed, qk_mult=qk_mult, with_dout=True)
    q, k, v, do = (G.to_dev(inp[n]) for n in ("q", "k", "v", "dout"))
    print(f"standard bwd case shape={shape} mask={mask} w={window} scale={scale}", flush=True)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    fws = torch.empty(fa_fwd_standard_workspace_bytes(B, H, N, d, BF16), dtype=torch.uint8,
                      device="cuda")
    fa_fwd_standard(q, k, v, o, lse, fws, scale, mask, window)
    ws = torch.empty(fa_bwd_standard_workspace_bytes(B, H, N, d, BF16), dtype=torch.uint8,
                     device="cuda")
    dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
    fa_bwd_standard(q, k, v, do, fws, dq, dk, dv, ws, scale)
    torch.cuda.synchronize()
    ref = oracle.bwd_dense(inp["q"], inp["k"], inp["v"], inp["dout"], scale, mask, window)
    errs = {}
    for name, g in (("dq", dq), ("dk", dk), ("dv", dv)):
        gn = G.f64(g)
        assert np.all(np.isfinite(gn)), name
        nr = np.linalg.norm(ref[name])
        errs[name] = float(np.linalg.norm(gn - ref[name]) / (nr if nr > 0 else 1.0))
        assert errs[name] <= G.TOL_GRAD_REL, (name, errs[name])
    return errs


BWD_CASES = [
    ((1, 1, 1, 128), "none", 0),
    ((1, 2, 6, 64), "causal", 0),
    ((2, 3, 17, 128), "causal", 0),
    ((1, 2, 129, 128), "none", 0),     # one past a 128-key score tile
    ((2, 2, 300, 128), "causal", 0),   # padded rows; several 256-row output tiles
    ((1, 3, 513, 64), "none", 0),
    ((1, 2, 700, 128), "local", 1),
    ((1, 2, 1000, 64), "local", 128),
    ((1, 2, 1001, 64), "causal", 0),
]


@pytest.mark.parametrize("shape,mask,window", BWD_CASES,
                         ids=[f"{s}-{m}-{w}" for s, m, w in BWD_CASES])
def test_standard_backward(shape, mask, window):
    run_std_bwd(shape, mask, window, seed=sum(shape) + window + 3)


@pytest.mark.parametrize("scale", [0.0, -0.25, 2.0])
def test_standard_backward_scales(scale):
    run_std_bwd((1, 2, 200, 128), "causal", 0, scale=scale, seed=17)


def test_standard_backward_large_logits():
    run_std_bwd((1, 1, 300, 128), "local", 64, qk_mult=4.0, seed=18)


def test_standard_backward_errors():
    from exact_tiled_attention_fwd_amd import fa_bwd_standard
    q = torch.zeros(1, 1, 8, 64, dtype=BF16, device="cuda")
    g = [torch.empty_like(q) for _ in range(3)]
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    big = torch.empty(1 << 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(FAError):  # forward workspace too small
        fa_bwd_standard(q, q.clone(), q.clone(), q.clone(), small, *g, big, 0.125)
    with pytest.raises(FAError):  # own workspace too small
        fa_bwd_standard(q, q.clone(), q.clone(), q.clone(), big, *g, small, 0.125)
    with pytest.raises(FAError):  # the two workspaces are one buffer
        fa_bwd_standard(q, q.clone(), q.clone(), q.clone(), big, *g, big, 0.125)
