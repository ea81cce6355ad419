"""Helpers shared by the GPU parity tests (inputs on the host from the seeded
generators, the library call on the GPU, the oracle on the CPU)."""
import numpy as np
import torch

import oracle

# Tolerances: float32 inputs max-abs 1e-5 on O; bf16 inputs with float32
# accumulation max-abs 2e-2 on O; LSE (not fixed by the workload statement,
# derived from float32 rounding of the logits): 1e-4 + 1e-5*|LSE| for bf16,
# 1e-5 + 1e-6*|LSE| for float32; backward: ||G - G_ref||_F / ||G_ref||_F <= 1e-2.
TOL_O = {torch.bfloat16: 2e-2, torch.float32: 1e-5}
TOL_LSE = {torch.bfloat16: (1e-4, 1e-5), torch.float32: (1e-5, 1e-6)}
TOL_GRAD_REL = 1e-2


def have_gpu():
    return torch.cuda.is_available()


def to_dev(t):
    return t.to("cuda").contiguous()


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def check_fwd(o_gpu, lse_gpu, o_ref, lse_ref, dtype, what=""):
    """Element-wise comparison with the tolerance of the dtype; returns the
    max errors for reporting."""
    o = f64(o_gpu)
    lse = f64(lse_gpu)
    assert np.all(np.isfinite(o)), f"{what}: non-finite O"
    assert np.all(np.isfinite(lse)), f"{what}: non-finite LSE"
    eo = np.abs(o - o_ref)
    el = np.abs(lse - lse_ref)
    a, r = TOL_LSE[dtype]
    assert eo.max(initial=0.0) <= TOL_O[dtype], f"{what}: max |dO| {eo.max()} > {TOL_O[dtype]}"
    bad = el > a + r * np.abs(lse_ref)
    assert not bad.any(), f"{what}: LSE error {el.max()} (at {np.argwhere(bad)[:3].tolist()})"
    return float(eo.max(initial=0.0)), float(el.max(initial=0.0))


def sample_rows(BH, N, n_random, seed, tile=256):
    """(bh, row) pairs: edge rows of a few heads, rows at tile boundaries and
    random rows."""
    rng = np.random.default_rng(seed)
    heads = sorted({0, BH - 1} | set(rng.integers(0, BH, size=2).tolist()))
    rows = {0, 1, N - 1, N - 2, N // 2}
    for t in range(tile, N, tile * max(1, N // (8 * tile))):
        rows |= {t - 1, t}
    bh, rr = [], []
    for h in heads:
        picks = sorted(rows | set(rng.integers(0, N, size=n_random).tolist()))
        for r in picks:
            if 0 <= r < N:
                bh.append(h)
                rr.append(r)
    return np.array(bh, dtype=np.int64), np.array(rr, dtype=np.int64), heads


def oracle_rows(inp, w_scale, mask, window, bh, rows, heads):
    """Dense oracle rows for the selected heads only (double on the CPU)."""
    B, H, N, d = inp["q"].shape
    sel = {h: i for i, h in enumerate(heads)}
    def pick(t):
        return t.reshape(B * H, N, d)[heads]
    q, k, v = (pick(inp[n]) for n in ("q", "k", "v"))
    o, lse = oracle.fwd_dense_rows(q, k, v, w_scale, [sel[h] for h in bh], rows, mask, window)
    return o, lse
