"""fa_bwd_noalloc (include/fa.h), the backward without a workspace for
callers that cannot allocate: its gradients equal fa_bwd's bit for bit (the
same kernels, D in the library's static device array instead of the caller's
workspace) and meet the oracle's bar, on two calls in a row where the second
is smaller, so that the array holds the first call's D when the second starts.
Sizes beyond the array are rejected before anything is enqueued."""
import math

import numpy as np
import pytest
import torch

import oracle
from exact_tiled_attention_fwd_amd import _native, attention_bwd, attention_fwd, FAError
from exact_tiled_attention_fwd_amd.synth import random_inputs
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

BF16, F32 = torch.bfloat16, torch.float32


def run_pair(shape, dtype, mask, window, seed):
    B, H, N, d = shape
    scale = 1.0 / math.sqrt(d)
    inp = random_inputs(shape, dtype, seed=seed, with_dout=True)
    q, k, v, do = (G.to_dev(inp[n]) for n in ("q", "k", "v", "dout"))
    print(f"noalloc case shape={shape} dtype={dtype} mask={mask} w={window}", flush=True)
    o, lse = attention_fwd(q, k, v, scale, mask, window)
    ref_dq, ref_dk, ref_dv = attention_bwd(q, k, v, o, lse, do, scale, mask, window)
    dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
    _native.fa_bwd_noalloc(q, k, v, o, do, lse, dq, dk, dv, scale, mask, window)
    torch.cuda.synchronize()
    assert torch.equal(dq, ref_dq) and torch.equal(dk, ref_dk) and torch.equal(dv, ref_dv)
    ref = oracle.bwd_dense(inp["q"], inp["k"], inp["v"], inp["dout"], scale, mask, window)
    for name, g in (("dq", dq), ("dk", dk), ("dv", dv)):
        gn = G.f64(g)
        e = float(np.linalg.norm(gn - ref[name]) / np.linalg.norm(ref[name]))
        assert e <= (G.TOL_GRAD_REL if dtype == BF16 else 1e-4), (name, e)


@pytest.mark.parametrize("dtype", [BF16, F32])
def test_noalloc_matches_fa_bwd_two_calls(dtype):
    d = 128 if dtype == BF16 else 32
    run_pair((2, 3, 700, d), dtype, "causal", 0, seed=31)   # 4200 rows of D
    run_pair((1, 2, 257, d), dtype, "local", 40, seed=32)   # then 514: smaller


def test_noalloc_rejects_oversize():
    rows = _native.FA_BWD_NOALLOC_MAX_ROWS
    N = rows // 64 + 1  # B * H * N just past the array with B * H = 64
    q = torch.zeros((1, 1, 8, 64), dtype=BF16, device="cuda")
    lib = _native.load()
    ins = [q.data_ptr()] * 6  # validation stops at the size, before the pointers matter
    st = lib.fa_bwd_noalloc(*ins, 0x100000, 0x200000, 0x300000, 8, 8, N, 64, 1, 0.125, 0, 0, None)
    assert st == 8  # FA_ERR_WORKSPACE, before any launch
    with pytest.raises(FAError):
        big = torch.zeros((1, 1, 8, 64), dtype=BF16, device="cuda")
        _native.fa_bwd_noalloc(big, big, big, big, big, torch.zeros((1, 1, 8), device="cuda"),
                               big.clone(), big.clone(), big.clone(), float("nan"))
