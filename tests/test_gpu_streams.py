"""Stream and graph behaviour of the boundary. fa_fwd and fa_bwd only enqueue
kernels on the stream they are given: no synchronisation, no allocation, no
memset. The same calls therefore run on a side stream, and inside a captured
HIP graph replayed several times, with results bit-identical to the
default-stream calls (every kernel is deterministic). Outputs are filled with
NaN before each run, so a result also shows that O, LSE, dQ, dK and dV are
overwritten in full."""
import math

import pytest
import torch

from exact_tiled_attention_fwd_amd import fa_bwd, fa_bwd_workspace_bytes, fa_fwd
from exact_tiled_attention_fwd_amd.synth import random_inputs
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

BF16 = torch.bfloat16
OUTS = ("o", "lse", "dq", "dk", "dv")
INS = ("q", "k", "v", "dout")

# ragged N in every case; each head dimension and mask of the bf16 path
CASES = [
    ((2, 4, 1000, 128), "causal", 0),
    ((1, 3, 777, 64), "local", 100),
    ((2, 2, 513, 128), "none", 0),
]


def _alloc(shape, seed):
    inp = random_inputs(shape, BF16, seed=seed, with_dout=True)
    t = {n: G.to_dev(inp[n]) for n in INS}
    B, H, N, d = shape
    t["o"] = torch.empty_like(t["q"])
    t["lse"] = torch.empty((B, H, N), device="cuda", dtype=torch.float32)
    for n in ("dq", "dk", "dv"):
        t[n] = torch.empty_like(t["q"])
    t["ws"] = torch.empty(max(1, fa_bwd_workspace_bytes(B, H, N, d, BF16)), dtype=torch.uint8,
                          device="cuda")
    return t


def _step(t, scale, mask, window, stream=None):
    fa_fwd(t["q"], t["k"], t["v"], t["o"], t["lse"], scale, mask, window, stream=stream)
    fa_bwd(t["q"], t["k"], t["v"], t["o"], t["dout"], t["lse"], t["dq"], t["dk"], t["dv"],
           t["ws"], scale, mask, window, stream=stream)


def _poison(t):
    for n in OUTS:
        t[n].fill_(float("nan"))


def _check_equal(t, ref, what):
    for n in OUTS:
        assert torch.equal(t[n], ref[n]), f"{what}: {n} differs from the default-stream result"


@pytest.mark.parametrize("shape,mask,window", CASES)
def test_side_stream_matches_default(shape, mask, window):
    scale = 1.0 / math.sqrt(shape[3])
    print(f"side stream shape={shape} mask={mask} w={window}", flush=True)
    t = _alloc(shape, seed=11)
    _step(t, scale, mask, window)
    torch.cuda.synchronize()
    ref = {n: t[n].clone() for n in OUTS}
    assert all(torch.isfinite(ref[n].float()).all() for n in OUTS)

    side = torch.cuda.Stream()
    # the current stream inside a stream context
    _poison(t)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _step(t, scale, mask, window)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    _check_equal(t, ref, "side stream (context)")
    # an explicit stream argument
    _poison(t)
    side.wait_stream(torch.cuda.current_stream())
    _step(t, scale, mask, window, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    _check_equal(t, ref, "side stream (argument)")


@pytest.mark.parametrize("shape,mask,window", CASES)
def test_graph_capture_replay(shape, mask, window):
    scale = 1.0 / math.sqrt(shape[3])
    print(f"graph shape={shape} mask={mask} w={window}", flush=True)
    # eager results for two input sets
    t = _alloc(shape, seed=21)
    t2 = _alloc(shape, seed=22)
    _step(t, scale, mask, window)
    _step(t2, scale, mask, window)
    torch.cuda.synchronize()
    refs = [{n: t[n].clone() for n in OUTS}, {n: t2[n].clone() for n in OUTS}]
    inputs = [{n: t[n].clone() for n in INS}, {n: t2[n].clone() for n in INS}]

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _step(t, scale, mask, window)  # warm-up on the capture stream's side
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        _step(t, scale, mask, window)
    torch.cuda.synchronize()

    # replays alternate the two input sets; the copies, the NaN fill and a
    # synchronisation run eagerly between them
    for rep in range(6):
        src = inputs[rep % 2]
        for n in INS:
            t[n].copy_(src[n])
        _poison(t)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _check_equal(t, refs[rep % 2], f"graph replay {rep}")
