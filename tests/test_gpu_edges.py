"""Edge cases of size: long sequences (up to 131072 rows, i.e. 512 query
tiles and over a thousand key tiles per head, with a ragged last tile), many
heads with short sequences (4096 slices of 33 rows), the backward at a long
band sequence, and tensors past 2^31 elements (64-bit offsets); sampled rows
against the oracle, finiteness at every row."""
import math

import numpy as np
import pytest
import torch

import oracle
from exact_tiled_attention_fwd_amd import attention_bwd, attention_fwd
from exact_tiled_attention_fwd_amd.synth import device_inputs, random_inputs
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

BF16 = torch.bfloat16


@pytest.mark.parametrize("shape,mask,window", [
    ((1, 1, 131072, 64), "causal", 0),
    ((1, 2, 65536, 128), "local", 512),
    ((1, 1, 50001, 128), "none", 0),      # ragged, long
])
def test_long_sequence_forward(shape, mask, window):
    B, H, N, d = shape
    scale = 1.0 / math.sqrt(d)
    inp = random_inputs(shape, BF16, seed=N % 1000 + d)
    q, k, v = (G.to_dev(inp[n]) for n in ("q", "k", "v"))
    print(f"long forward {shape} {mask} {window}", flush=True)
    o, lse = attention_fwd(q, k, v, scale, mask, window)
    torch.cuda.synchronize()
    bh, rows, heads = G.sample_rows(B * H, N, 24, seed=N)
    o_ref, lse_ref = G.oracle_rows(inp, scale, mask, window, bh, rows, heads)
    o_g = o.reshape(B * H, N, d)[torch.as_tensor(bh), torch.as_tensor(rows)]
    l_g = lse.reshape(B * H, N)[torch.as_tensor(bh), torch.as_tensor(rows)]
    eo, el = G.check_fwd(o_g, l_g, o_ref, lse_ref, BF16, f"long {shape}")
    print(f"max|dO|={eo:.3e} max|dLSE|={el:.3e} rows={len(rows)}", flush=True)
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()


def test_many_short_heads():
    # 4096 (batch, head) slices of 33 rows: every workgroup is a ragged tile
    shape = (64, 64, 33, 64)
    inp = random_inputs(shape, BF16, seed=77)
    q, k, v = (G.to_dev(inp[n]) for n in ("q", "k", "v"))
    o, lse = attention_fwd(q, k, v, 0.125, "causal")
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.fwd_dense(inp["q"], inp["k"], inp["v"], 0.125, "causal")
    G.check_fwd(o, lse, o_ref, lse_ref, BF16, "many short heads")


def test_long_band_backward():
    # backward at N = 65536 under a band: sampled dQ and dK/dV rows
    shape = (1, 2, 65536, 128)
    B, H, N, d = shape
    scale = 1.0 / math.sqrt(d)
    inp = random_inputs(shape, BF16, seed=65, with_dout=True)
    q, k, v, do = (G.to_dev(inp[n]) for n in ("q", "k", "v", "dout"))
    print("long band backward", flush=True)
    o, lse = attention_fwd(q, k, v, scale, "local", 64)
    dq, dk, dv = attention_bwd(q, k, v, o, lse, do, scale, "local", 64)
    torch.cuda.synchronize()
    bh, rows, heads = G.sample_rows(B * H, N, 24, seed=66)
    sel = {h_: i for i, h_ in enumerate(heads)}
    pick = {n: inp[n].reshape(B * H, N, d)[heads] for n in ("q", "k", "v", "dout")}
    lb = np.array([sel[h_] for h_ in bh])
    ref = oracle.bwd_rows(pick["q"], pick["k"], pick["v"], pick["dout"], scale, lb, rows, lb,
                          rows, "local", 64)
    for name, g in (("dq", dq), ("dk", dk), ("dv", dv)):
        gs = G.f64(g.reshape(B * H, N, d)[torch.as_tensor(bh), torch.as_tensor(rows)])
        e = float(np.linalg.norm(gs - ref[name]) / np.linalg.norm(ref[name]))
        print(f"{name}: rel {e:.3e} over {len(rows)} rows", flush=True)
        assert np.all(np.isfinite(gs)) and e <= G.TOL_GRAD_REL, (name, e)
    for g in (dq, dk, dv):
        assert torch.isfinite(g.float()).all()


def test_past_2g_elements():
    # [1, 16640, 1024, 128] bf16: 2.18e9 elements per tensor (4.36e9 bytes), so the
    # last heads start past 2^31 elements and 2^32 bytes; their rows are checked
    # against the oracle, forward and backward, under the causal mask
    shape = (1, 16640, 1024, 128)
    B, H, N, d = shape
    per = B * H * N * d * 2
    free, _ = torch.cuda.mem_get_info()
    if free < 10 * per:
        pytest.skip(f"needs {10 * per / 1e9:.0f} GB of free device memory")
    scale = 1.0 / math.sqrt(d)
    print("past 2^31 elements: inputs", flush=True)
    t = device_inputs(shape, BF16, seed=31, with_dout=True)
    print("past 2^31 elements: forward + backward", flush=True)
    o, lse = attention_fwd(t["q"], t["k"], t["v"], scale, "causal")
    dq, dk, dv = attention_bwd(t["q"], t["k"], t["v"], o, lse, t["dout"], scale, "causal")
    torch.cuda.synchronize()
    heads = [0, 8191, 16383, 16384, 16500, H - 1]
    assert heads[-1] * N * d > 2 ** 31 and heads[-1] * N * d * 2 > 2 ** 32
    rng = np.random.default_rng(32)
    rows = sorted({0, 1, 255, 256, N - 2, N - 1} | set(rng.integers(0, N, 10).tolist()))
    bh = np.repeat(np.arange(len(heads)), len(rows))
    rr = np.tile(np.array(rows), len(heads))
    idx = torch.as_tensor(heads, device="cuda")
    pick = {n: t[n].reshape(B * H, N, d).index_select(0, idx).cpu() for n in t}
    print("past 2^31 elements: oracle", flush=True)
    o_ref, lse_ref = oracle.fwd_dense_rows(pick["q"], pick["k"], pick["v"], scale, bh, rr, "causal", 0)
    hb = torch.as_tensor([heads[i] for i in bh])
    G.check_fwd(o.reshape(B * H, N, d)[hb, torch.as_tensor(rr)],
                lse.reshape(B * H, N)[hb, torch.as_tensor(rr)], o_ref, lse_ref, BF16,
                "past 2^31 elements")
    ref = oracle.bwd_rows(pick["q"], pick["k"], pick["v"], pick["dout"], scale, bh, rr, bh, rr,
                          "causal", 0)
    for name, g in (("dq", dq), ("dk", dk), ("dv", dv)):
        gs = G.f64(g.reshape(B * H, N, d)[hb, torch.as_tensor(rr)])
        e = float(np.linalg.norm(gs - ref[name]) / np.linalg.norm(ref[name]))
        print(f"{name}: rel {e:.3e} over {len(rr)} rows", flush=True)
        assert np.all(np.isfinite(gs)) and e <= G.TOL_GRAD_REL, (name, e)
