"""Backward parity: fa_bwd (HIP, through the C ABI) against the CPU oracle's
dense chain-rule backward on the same seeded inputs. The GPU consumes its own
forward's O and LSE; the oracle uses its double-precision O."""
import math

import numpy as np
import pytest
import torch

import oracle
from exact_tiled_attention_fwd_amd import (attention_bwd, attention_fwd, fa_bwd, fa_bwd_tuned,
                                           fa_bwd_workspace_bytes, FAError)
from exact_tiled_attention_fwd_amd.synth import WORKLOADS, make_inputs, random_inputs
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

BF16, F32 = torch.bfloat16, torch.float32


def rel(g, ref):
    g = G.f64(g)
    n = np.linalg.norm(ref)
    return float(np.linalg.norm(g - ref) / (n if n > 0 else 1.0))


def run_case(shape, dtype, mask, window, scale=None, seed=0, qk_mult=1.0, cfg=0):
    """fa_fwd then fa_bwd (or, with cfg != 0, fa_bwd_tuned with that kernel
    shape) on seeded inputs against the oracle's dense backward."""
    B, H, N, d = shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    inp = random_inputs(shape, dtype, seed=seed, qk_mult=qk_mult, with_dout=True)
    q, k, v, do = (G.to_dev(inp[n]) for n in ("q", "k", "v", "dout"))
    print(f"bwd case shape={shape} dtype={dtype} mask={mask} w={window} scale={scale} cfg={cfg}",
          flush=True)
    o, lse = attention_fwd(q, k, v, scale, mask, window)
    if cfg:
        ws = torch.empty(fa_bwd_workspace_bytes(B, H, N, d, q.dtype), dtype=torch.uint8,
                         device=q.device)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        fa_bwd_tuned(q, k, v, o, do, lse, dq, dk, dv, ws, scale, mask, window, cfg)
    else:
        dq, dk, dv = attention_bwd(q, k, v, o, lse, do, scale, mask, window)
    torch.cuda.synchronize()
    ref = oracle.bwd_dense(inp["q"], inp["k"], inp["v"], inp["dout"], scale, mask, window)
    errs = {}
    for name, g in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert torch.isfinite(g.float()).all(), f"{name} not finite"
        errs[name] = rel(g, ref[name])
        assert errs[name] <= G.TOL_GRAD_REL, (name, errs[name])
    return errs


SMALL = [
    ((1, 1, 1, 128), "none", 0),
    ((1, 2, 6, 128), "causal", 0),
    ((2, 2, 33, 128), "none", 0),
    ((1, 2, 129, 128), "causal", 0),
    ((1, 2, 300, 128), "causal", 0),
    ((1, 1, 513, 128), "none", 0),
    ((1, 2, 400, 128), "local", 0),
    ((1, 2, 400, 128), "local", 1),
    ((1, 2, 700, 128), "local", 100),
    ((1, 1, 5, 64), "none", 0),
    ((2, 2, 130, 64), "causal", 0),
    ((1, 2, 300, 64), "local", 17),
    ((1, 1, 257, 64), "none", 0),
]


@pytest.mark.parametrize("shape,mask,window", SMALL, ids=[f"{s}-{m}-{w}" for s, m, w in SMALL])
def test_bf16_small(shape, mask, window):
    run_case(shape, BF16, mask, window, seed=11 + shape[2] + window)


@pytest.mark.parametrize("scale", [0.0, -0.1, 0.3])
def test_bf16_scales(scale):
    run_case((1, 2, 160, 128), BF16, "causal", 0, scale=scale, seed=4)


def test_bf16_large_logits():
    run_case((1, 1, 300, 128), BF16, "local", 64, qk_mult=4.0, seed=6)


F32_CASES = [((1, 1, 6, 4), "none", 0), ((1, 2, 6, 4), "causal", 0), ((1, 1, 40, 4), "local", 2),
             ((1, 2, 150, 33), "causal", 0), ((1, 1, 130, 64), "none", 0),
             ((1, 1, 70, 128), "causal", 0)]


@pytest.mark.parametrize("shape,mask,window", F32_CASES, ids=[f"{s}-{m}-{w}" for s, m, w in F32_CASES])
def test_f32(shape, mask, window):
    errs = run_case(shape, F32, mask, window, seed=2)
    assert max(errs.values()) <= 1e-4, errs


def test_workspace_error():
    q = torch.zeros((1, 1, 64, 64), dtype=BF16, device="cuda")
    lse = torch.zeros((1, 1, 64), dtype=torch.float32, device="cuda")
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    t = [torch.zeros_like(q) for _ in range(7)]
    with pytest.raises(FAError):
        fa_bwd(q, t[0], t[1], t[2], t[3], lse, t[4], t[5], t[6], small, 0.125)


def test_deterministic():
    shape = (1, 2, 600, 128)
    inp = random_inputs(shape, BF16, seed=3, with_dout=True)
    q, k, v, do = (G.to_dev(inp[n]) for n in ("q", "k", "v", "dout"))
    o, lse = attention_fwd(q, k, v, None, "causal")
    a = attention_bwd(q, k, v, o, lse, do, None, "causal")
    b = attention_bwd(q, k, v, o, lse, do, None, "causal")
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(a, b))


def test_full_size_backward_workload():
    """The causal backward workload [2, 16, 4096, 128] in the bench's launch
    configuration: all 32 (b, h) slices against the oracle's dense backward,
    relative Frobenius error of each gradient over the whole tensor (the worst
    slice is reported too), and the gradient invariants."""
    import time
    w = WORKLOADS["bf16_causal_bwd_b2h16_n4096_d128"]
    inp = make_inputs(w)
    q, k, v, do = (G.to_dev(inp[n]) for n in ("q", "k", "v", "dout"))
    print("full-size backward", flush=True)
    o, lse = attention_fwd(q, k, v, w.scale, w.mask, w.window)
    dq, dk, dv = attention_bwd(q, k, v, o, lse, do, w.scale, w.mask, w.window)
    torch.cuda.synchronize()
    B, H, N, d = w.shape
    t0 = time.perf_counter()
    ref = oracle.bwd_dense(inp["q"], inp["k"], inp["v"], inp["dout"], w.scale, w.mask, w.window)
    print(f"oracle dense backward over {B * H} slices: {time.perf_counter() - t0:.1f} s", flush=True)
    for name, g in (("dq", dq), ("dk", dk), ("dv", dv)):
        gn = G.f64(g).reshape(B * H, N, d)
        rn = ref[name].reshape(B * H, N, d)
        e = float(np.linalg.norm(gn - rn) / np.linalg.norm(rn))
        per = np.linalg.norm((gn - rn).reshape(B * H, -1), axis=1) / np.linalg.norm(
            rn.reshape(B * H, -1), axis=1)
        print(f"{name}: rel {e:.3e} over the whole tensor; worst slice {int(per.argmax())}: "
              f"{float(per.max()):.3e}", flush=True)
        assert np.all(np.isfinite(gn)) and e <= G.TOL_GRAD_REL, (name, e)
    # invariants on every slice: sum_j dK_j = 0, sum_j dV_j = sum_i dO_i
    dkf, dvf, dof = dk.double(), dv.double(), do.double()
    sk = dkf.sum(dim=2).norm() / dkf.norm()
    sv = (dvf.sum(dim=2) - dof.sum(dim=2)).norm() / dof.sum(dim=2).norm()
    print(f"invariants: |sum dK|/|dK| = {float(sk):.2e}, |sum dV - sum dO| rel = {float(sv):.2e}")
    assert float(sk) <= 2e-2 and float(sv) <= 1e-2


def test_full_size_band_backward():
    """The band workload's shape and logit scale ([1, 32, 16384, 128], Q and
    K x8, |i - j| <= 128) through the backward in the default launch
    configuration: sampled dQ rows and dK/dV rows (edges, tile boundaries and
    random rows of four heads) against the oracle's row-sampled backward,
    relative Frobenius error over the sampled rows; plus the invariants on
    every slice. Sampled, not whole: the oracle's dense backward holds two
    N x N matrices per head (2 x 2 GB here) and visits every pair, masked or
    not, which at this length takes several host minutes per run."""
    w = WORKLOADS["bf16_local128_x8_bwd_b1h32_n16384_d128"]
    inp = make_inputs(w)
    q, k, v, do = (G.to_dev(inp[n]) for n in ("q", "k", "v", "dout"))
    print("full-size band backward", flush=True)
    o, lse = attention_fwd(q, k, v, w.scale, w.mask, w.window)
    dq, dk, dv = attention_bwd(q, k, v, o, lse, do, w.scale, w.mask, w.window)
    torch.cuda.synchronize()
    B, H, N, d = w.shape
    bh, rows, heads = G.sample_rows(B * H, N, 40, seed=61)
    sel = {h_: i for i, h_ in enumerate(heads)}
    pick = {n: inp[n].reshape(B * H, N, d)[heads] for n in ("q", "k", "v", "dout")}
    lb = np.array([sel[h_] for h_ in bh])
    ref = oracle.bwd_rows(pick["q"], pick["k"], pick["v"], pick["dout"], w.scale, lb, rows, lb,
                          rows, w.mask, w.window)
    for name, g in (("dq", dq), ("dk", dk), ("dv", dv)):
        gs = G.f64(g.reshape(B * H, N, d)[torch.as_tensor(bh), torch.as_tensor(rows)])
        e = float(np.linalg.norm(gs - ref[name]) / np.linalg.norm(ref[name]))
        print(f"{name}: rel {e:.3e} over {len(rows)} rows", flush=True)
        assert np.all(np.isfinite(gs)) and e <= G.TOL_GRAD_REL, (name, e)
    dkf, dvf, dof = dk.double(), dv.double(), do.double()
    sk = dkf.sum(dim=2).norm() / dkf.norm()
    sv = (dvf.sum(dim=2) - dof.sum(dim=2)).norm() / dof.sum(dim=2).norm()
    print(f"invariants: |sum dK|/|dK| = {float(sk):.2e}, |sum dV - sum dO| rel = {float(sv):.2e}")
    assert float(sk) <= 2e-2 and float(sv) <= 1e-2


# Under the band mask every kernel visits its tiles in a rotated order (by tile
# index modulo the tile count of an interior window). These lengths give
# dozens of interior workgroups with every rotation offset, plus ragged ends;
# radii that are not multiples of any tile size, at both head dimensions.
BAND_ROTATION_CASES = [((1, 2, 2500, 128), 31), ((1, 2, 2500, 128), 200),
                       ((1, 2, 3001, 64), 33), ((1, 2, 3001, 64), 300)]


@pytest.mark.parametrize("shape,window", BAND_ROTATION_CASES,
                         ids=[f"{s}-w{w}" for s, w in BAND_ROTATION_CASES])
def test_band_backward_rotated_order(shape, window):
    run_case(shape, BF16, "local", window, seed=shape[2] + window)
