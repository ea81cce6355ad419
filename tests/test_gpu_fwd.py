"""Forward parity: fa_fwd (HIP, through the C ABI) against the CPU oracle on
the same seeded inputs, element by element."""
import math

import numpy as np
import pytest
import torch

import oracle
from exact_tiled_attention_fwd_amd import fa_fwd, fa_fwd_tuned, attention_fwd, FAError
from exact_tiled_attention_fwd_amd.synth import WORKLOADS, make_inputs, random_inputs
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

BF16, F32 = torch.bfloat16, torch.float32


def run_case(shape, dtype, mask, window, scale=None, qk_mult=1.0, seed=0, cfg=0):
    """fa_fwd (or, with cfg != 0, fa_fwd_tuned with that kernel shape) on
    seeded inputs against the dense oracle, element by element."""
    B, H, N, d = shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    inp = random_inputs(shape, dtype, seed=seed, qk_mult=qk_mult)
    q, k, v = (G.to_dev(inp[n]) for n in ("q", "k", "v"))
    print(f"case shape={shape} dtype={dtype} mask={mask} w={window} scale={scale} cfg={cfg}",
          flush=True)
    if cfg:
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
        fa_fwd_tuned(q, k, v, o, lse, scale, mask, window, cfg)
    else:
        o, lse = attention_fwd(q, k, v, scale, mask, window)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.fwd_dense(inp["q"], inp["k"], inp["v"], scale, mask, window)
    return G.check_fwd(o, lse, o_ref, lse_ref, dtype, f"{shape} {mask} {window}")


SMALL = [
    # (B, H, N, d), mask, window  -- several tiles and ragged tails
    ((1, 1, 1, 128), "none", 0),
    ((1, 2, 6, 128), "none", 0),
    ((2, 3, 17, 128), "causal", 0),
    ((1, 2, 127, 128), "none", 0),
    ((1, 2, 129, 128), "causal", 0),
    ((2, 2, 300, 128), "causal", 0),
    ((1, 3, 513, 128), "none", 0),
    ((1, 2, 700, 128), "local", 0),
    ((1, 2, 700, 128), "local", 1),
    ((1, 2, 700, 128), "local", 37),
    ((1, 2, 1000, 128), "local", 128),
    ((1, 1, 600, 128), "local", 5000),
    ((1, 1, 1, 64), "none", 0),
    ((2, 2, 33, 64), "none", 0),
    ((1, 2, 257, 64), "causal", 0),
    ((1, 2, 1000, 64), "causal", 0),
    ((1, 2, 777, 64), "local", 64),
    ((3, 5, 65, 64), "local", 3),
    ((1, 2, 700, 64), "local", 0),
    ((1, 1, 600, 64), "local", 5000),
    ((1, 2, 1000, 64), "local", 128),
]


@pytest.mark.parametrize("shape,mask,window", SMALL, ids=[f"{s}-{m}-{w}" for s, m, w in SMALL])
def test_bf16_small(shape, mask, window):
    run_case(shape, BF16, mask, window, seed=sum(shape) + window)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("scale", [0.0, -0.125, 0.5, 2.0])
def test_bf16_scales(d, scale):
    run_case((1, 2, 200, d), BF16, "causal", 0, scale=scale, seed=7)


def test_bf16_large_logits():
    # Q, K x8 as in the large-logit band workload: logits with std ~64
    run_case((1, 2, 600, 128), BF16, "local", 128, qk_mult=8.0, seed=9)
    run_case((1, 2, 600, 128), BF16, "none", 0, qk_mult=8.0, seed=10)


F32_CASES = [((1, 1, 6, 4), "none", 0), ((1, 1, 6, 4), "causal", 0), ((1, 1, 6, 4), "local", 1),
             ((2, 2, 130, 1), "none", 0), ((1, 2, 257, 33), "causal", 0),
             ((1, 1, 300, 64), "local", 20), ((1, 2, 129, 128), "none", 0),
             ((1, 1, 50, 100), "causal", 0)]


@pytest.mark.parametrize("shape,mask,window", F32_CASES, ids=[f"{s}-{m}-{w}" for s, m, w in F32_CASES])
def test_f32(shape, mask, window):
    run_case(shape, F32, mask, window, seed=3)


def test_toy_workload_all_tiles():
    """The toy float32 run ([1, 6, 4], seed 0, scale 1/2): the GPU output
    equals the dense oracle and every tiled oracle of the page's tile sizes."""
    w = WORKLOADS["toy_fp32_n6_d4"]
    inp = make_inputs(w)
    q, k, v = (G.to_dev(inp[n]) for n in ("q", "k", "v"))
    o, lse = attention_fwd(q, k, v, w.scale)
    torch.cuda.synchronize()
    od, ld = oracle.fwd_dense(inp["q"], inp["k"], inp["v"], w.scale)
    G.check_fwd(o, lse, od, ld, F32, "toy dense")
    for t in w.tiles:
        ot, lt = oracle.fwd_tiled(inp["q"], inp["k"], inp["v"], w.scale, t, t)
        G.check_fwd(o, lse, ot, lt, F32, f"toy tiled {t}")


def test_rows_sum_to_one_on_gpu():
    """V = 1 gives O = 1 up to the rounding of P to bf16 (rows of P sum to 1)."""
    shape = (1, 2, 513, 128)
    inp = random_inputs(shape, BF16, seed=5)
    q, k = G.to_dev(inp["q"]), G.to_dev(inp["k"])
    v = torch.ones(shape, dtype=BF16, device="cuda")
    for mask, window in (("none", 0), ("causal", 0), ("local", 9)):
        o, _ = attention_fwd(q, k, v, None, mask, window)
        torch.cuda.synchronize()
        assert float((o.float() - 1).abs().max()) <= 2 ** -7


def test_deterministic():
    shape = (2, 2, 1000, 128)
    inp = random_inputs(shape, BF16, seed=8)
    q, k, v = (G.to_dev(inp[n]) for n in ("q", "k", "v"))
    o1, l1 = attention_fwd(q, k, v, None, "causal")
    o2, l2 = attention_fwd(q, k, v, None, "causal")
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_errors_raise():
    q = torch.zeros((1, 1, 8, 96), dtype=BF16, device="cuda")
    with pytest.raises(FAError):
        attention_fwd(q, q.clone(), q.clone())
    q = torch.zeros((1, 1, 8, 64), dtype=BF16, device="cuda")
    with pytest.raises(FAError):
        attention_fwd(q, q.clone(), q.clone(), mask="local", window=-1)
    with pytest.raises(FAError):
        attention_fwd(q, q.clone(), q.clone(), scale=float("nan"))


@pytest.mark.parametrize("name", ["bf16_b4h16_n2048_d64", "bf16_causal_b2h16_n8192_d128",
                                  "bf16_local128_x8_b1h32_n16384_d128"])
def test_full_size_whole_tensor(name):
    """Full workload sizes in the bench's launch configuration: every row of
    O and LSE against the dense oracle on the same seeded inputs (max-abs
    2e-2 on O; 1e-4 + 1e-5 |LSE| on LSE)."""
    import time
    w = WORKLOADS[name]
    inp = make_inputs(w)
    q, k, v = (G.to_dev(inp[n]) for n in ("q", "k", "v"))
    print(f"full-size {name}", flush=True)
    o, lse = attention_fwd(q, k, v, w.scale, w.mask, w.window)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    o_ref, lse_ref = oracle.fwd_dense(inp["q"], inp["k"], inp["v"], w.scale, w.mask, w.window)
    t_or = time.perf_counter() - t0
    eo, el = G.check_fwd(o, lse, o_ref, lse_ref, BF16, name)
    B, H, N, d = w.shape
    print(f"{name}: max|dO|={eo:.3e} max|dLSE|={el:.3e} over all {B * H * N} rows "
          f"(oracle {t_or:.1f} s on the host)", flush=True)


# The band forward's rotated key-tile order (see the backward's test of the
# same name): many interior workgroups, ragged ends, odd radii, both d.
@pytest.mark.parametrize("shape,window", [((1, 2, 2500, 128), 31), ((1, 2, 2500, 128), 200),
                                          ((1, 2, 3001, 64), 33), ((1, 2, 3001, 64), 300)])
def test_band_forward_rotated_order(shape, window):
    run_case(shape, BF16, "local", window, seed=shape[2] + window + 1)
