"""Pin checks for the CPU oracle, written as functions of an oracle instance
so the same checks run against the real oracle (tests/test_oracle_pins.py)
and against copies with planted mistakes (tests/test_oracle_mutations.py).

Every check compares the oracle with something other than itself: values a
page prints, closed forms, invariants of the mathematics, brute force, or an
independent library routine (torch float64 softmax / autograd).
"""
import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float64).numpy()


def torch_reference(q, k, v, scale, mask, window):
    """Independent library evaluation of the definition: torch float64
    softmax over scale*QK^T with masked entries at -inf."""
    q, k, v = (torch.as_tensor(np.asarray(x, dtype=np.float64)) for x in (q, k, v))
    N = q.shape[-2]
    s = scale * (q @ k.transpose(-1, -2))
    i = torch.arange(N).view(-1, 1)
    j = torch.arange(N).view(1, -1)
    if mask == "causal":
        s = s.masked_fill(~(j <= i), float("-inf"))
    elif mask == "local":
        s = s.masked_fill(~((i - j).abs() <= window), float("-inf"))
    p = torch.softmax(s, dim=-1)
    lse = torch.logsumexp(s, dim=-1)
    return (p @ v).numpy(), lse.numpy()


# ---------------------------------------------------------------- P3 example
def pin_p3_worked_example(orc):
    g = golden("p3_worked_example.json")
    Q, K, V = (np.array(g[x], dtype=np.float64) for x in ("Q", "K", "V"))
    scale = g["scale"]
    tol = 0.5 * 10.0 ** (-g["printed_decimals"]) + 1e-12
    o, lse = orc.fwd_dense(Q, K, V, scale)
    # the printed output of row 0
    assert np.all(np.abs(o[0] - np.array(g["row0_O"])) <= tol), o[0]
    # closed form of row 0: weights [1, w, 1, w] on V rows with w = e^{-1/sqrt 2}
    w = math.exp(-1.0 / math.sqrt(2.0))
    exact = np.array([(1 + 3 * w) / (2 + 2 * w), (3 + w) / (2 + 2 * w)])
    assert np.max(np.abs(o[0] - exact)) <= 1e-15, (o[0], exact)
    assert abs(lse[0] - (1.0 / math.sqrt(2.0) + math.log(2 + 2 * w))) <= 1e-15
    # rows 1 and 3 (not printed): closed forms give [1, 1]; row 3 sees all zeros -> ln 4
    assert np.max(np.abs(o[1] - 1.0)) <= 1e-15 and np.max(np.abs(o[3] - 1.0)) <= 1e-15
    assert abs(lse[3] - math.log(4.0)) <= 1e-15
    # each V row sums to 2, so each output row sums to 2
    assert np.max(np.abs(o.sum(-1) - 2.0)) <= 1e-14
    # the tiled oracle with the page's block size 2 reproduces the printed intermediates
    for Br in (1, 2, 4):
        ot, lt, tm, tl, to = orc.fwd_tiled(Q, K, V, scale, Br, g["block"], trace=True)
        acc1 = to[0, 0, 0] * tl[0, 0, 0]
        acc2 = to[0, 1, 0] * tl[0, 1, 0]
        assert abs(tm[0, 0, 0] - g["row0_block1_m"]) <= tol
        assert abs(tl[0, 0, 0] - g["row0_block1_l"]) <= tol
        assert np.all(np.abs(acc1 - np.array(g["row0_block1_Otilde"])) <= tol)
        # block 2 on its own: the page's m^(2), l^(2), Otilde^(2)
        assert abs(tm[0, 1, 0] - g["row0_block2_m"]) <= tol  # equal maxima, so alpha = 1
        assert abs((tl[0, 1, 0] - tl[0, 0, 0]) - g["row0_block2_l"]) <= tol
        assert np.all(np.abs((acc2 - acc1) - np.array(g["row0_block2_Otilde"])) <= tol)
        assert abs(tl[0, 1, 0] - g["row0_l_new"]) <= tol
        assert np.all(np.abs(acc2 - np.array(g["row0_merged_numerator"])) <= tol)
        assert np.max(np.abs(ot - o)) <= 1e-15 and np.max(np.abs(lt - lse)) <= 1e-15


# ------------------------------------------------------- P2 three-tile replay
def _p2_inputs(g):
    """Inputs whose score matrix rows 0-1 equal the printed tiles: q0 = e0,
    q1 = e1 and k_j = [S0j, S1j, 0, 0], scale 1 (the products are exact)."""
    N, d = g["columns"], 4
    S = np.zeros((2, N))
    for t, tile in enumerate(g["score_tiles"]):
        S[0, 2 * t], S[0, 2 * t + 1], S[1, 2 * t], S[1, 2 * t + 1] = tile
    Q = np.zeros((N, d))
    Q[0, 0] = 1.0
    Q[1, 1] = 1.0
    K = np.zeros((N, d))
    K[:, 0] = S[0]
    K[:, 1] = S[1]
    V = _rand((N, d), 11)
    return Q, K, V, S


def pin_p2_recurrence(orc):
    g = golden("p2_three_tile_schedule.json")
    Q, K, V, S = _p2_inputs(g)
    _, lse, tm, tl, _ = orc.fwd_tiled(Q, K, V, 1.0, g["tile_rows"], g["tile_cols"], trace=True)
    for t in range(3):
        for r in range(2):
            m_ref = g["running_max"][t][r]
            l_ref = g["running_denominator"][t][r]
            assert abs(tm[0, t, r] - m_ref) <= 2 * np.spacing(abs(m_ref)), (t, r, tm[0, t, r], m_ref)
            assert abs(tl[0, t, r] - l_ref) <= 4 * np.spacing(l_ref), (t, r, tl[0, t, r], l_ref)
    # dense LSE of rows 0-1 equals the printed final max + ln(final denominator)
    _, lse_d = orc.fwd_dense(Q, K, V, 1.0)
    for r in range(2):
        ref = g["running_max"][2][r] + math.log(g["running_denominator"][2][r])
        assert abs(lse_d[r] - ref) <= 1e-15 * max(1.0, abs(ref)), (r, lse_d[r], ref)
        assert abs(lse[r] - ref) <= 1e-15 * max(1.0, abs(ref))


def pin_p2_metrics_reading():
    """The printed per-tile metric for tiles 1 and 2 is the max difference of
    the printed query-0 partial output from the printed final output; this
    fixes the reading 'partial output = normalized acc/l over keys seen'."""
    g = golden("p2_three_tile_schedule.json")
    fin = np.array(g["final_dense_output_query0"])
    for t in range(2):
        part = np.array(g["partial_output_query0"][t])
        assert np.max(np.abs(part - fin)) == g["max_diff_from_final_rows01"][t]
    # the last partial is the final output to within rounding
    assert np.max(np.abs(np.array(g["partial_output_query0"][2]) - fin)) <= \
        g["max_diff_from_final_rows01"][2]


def pin_partial_is_dense_over_prefix(orc):
    """P2's partial output after tile t is the exact attention over keys seen
    so far: compare the tiled trace with the dense oracle on truncated K/V."""
    N, d = 9, 3
    Q, K, V = _rand((N, d), 21), _rand((N, d), 22), _rand((N, d), 23)
    Bc = 2
    _, _, tm, tl, to = orc.fwd_tiled(Q, K, V, 0.8, 3, Bc, trace=True)
    for t in range((N + Bc - 1) // Bc):
        n = min(N, (t + 1) * Bc)
        # prefix attention by brute force (all queries against first n keys)
        s = 0.8 * Q @ K[:n].T
        p = np.exp(s - s.max(1, keepdims=True))
        o_pre = (p / p.sum(1, keepdims=True)) @ V[:n]
        assert np.max(np.abs(to[0, t] - o_pre)) <= 1e-13
        assert np.max(np.abs(tm[0, t] + np.log(tl[0, t]) - np.log(np.exp(s).sum(1)))) <= 1e-13


# ----------------------------------------------------------- tiled == dense
TILE_PAIRS = [(t, t) for t in (1, 2, 3, 4, 6)] + [(4, 1), (3, 4), (6, 4), (5, 5), (1, 6), (2, 5)]


def pin_tiled_equals_dense_toy(orc):
    """P2 numerical check: tiled matches dense across five tile sizes and
    uneven final tiles, on the toy [1, 6, 4] float32 randn shape (seed 0)."""
    g = torch.Generator().manual_seed(0)
    Q, K, V = (torch.randn((1, 6, 4), generator=g, dtype=torch.float32).double().numpy()
               for _ in range(3))
    for mask, window in (("none", 0), ("causal", 0), ("local", 1), ("local", 2)):
        od, ld = orc.fwd_dense(Q, K, V, 0.5, mask, window)
        ot_, lt_ = torch_reference(Q[0], K[0], V[0], 0.5, mask, window)
        assert np.max(np.abs(od[0] - ot_)) <= 1e-13 and np.max(np.abs(ld[0] - lt_)) <= 1e-13
        for Br, Bc in TILE_PAIRS:
            ot, lt = orc.fwd_tiled(Q, K, V, 0.5, Br, Bc, mask, window)
            assert np.max(np.abs(ot - od)) <= 1e-13, (mask, Br, Bc)
            assert np.max(np.abs(lt - ld)) <= 1e-13, (mask, Br, Bc)


def pin_against_library(orc):
    """Dense and tiled oracle against torch float64 softmax on random shapes,
    several heads, every mask, including ragged tiles and d = 1."""
    for seed, (BH, N, d) in enumerate([(3, 37, 8), (2, 17, 1), (1, 64, 16), (2, 5, 3)]):
        Q, K, V = _rand((BH, N, d), 100 + seed), _rand((BH, N, d), 200 + seed), _rand((BH, N, d), 300 + seed)
        for mask, window in (("none", 0), ("causal", 0), ("local", 0), ("local", 3), ("local", 100)):
            scale = 1.0 / math.sqrt(d)
            od, ld = orc.fwd_dense(Q, K, V, scale, mask, window)
            orf, lrf = torch_reference(Q, K, V, scale, mask, window)
            assert np.max(np.abs(od - orf)) <= 1e-12, (seed, mask, window)
            assert np.max(np.abs(ld - lrf)) <= 1e-12, (seed, mask, window)
            for Br, Bc in ((16, 16), (5, 7), (64, 3), (1, N)):
                ot, lt = orc.fwd_tiled(Q, K, V, scale, Br, Bc, mask, window)
                assert np.max(np.abs(ot - od)) <= 1e-12 and np.max(np.abs(lt - ld)) <= 1e-12
            # sampled rows agree with the full dense evaluation
            bh = np.arange(BH * N) // N
            rows = np.arange(BH * N) % N
            orow, lrow = orc.fwd_dense_rows(Q, K, V, scale, bh, rows, mask, window)
            assert np.max(np.abs(orow - od.reshape(-1, d))) == 0.0
            assert np.max(np.abs(lrow - ld.reshape(-1))) == 0.0


# ---------------------------------------------------------------- invariants
def pin_rows_sum_to_one(orc):
    N = 11
    # d = N so that V can be the identity
    Q, K = _rand((N, N), 31), _rand((N, N), 32)
    for mask, window in (("none", 0), ("causal", 0), ("local", 2)):
        # V = identity: the output row is the probability row itself
        o, _ = orc.fwd_dense(Q, K, np.eye(N), 0.9, mask, window)
        assert np.max(np.abs(o.sum(1) - 1.0)) <= 1e-14
        assert o.min() >= 0.0
        for i in range(N):
            for j in range(N):
                if not orc.allowed(i, j, mask, window):
                    assert o[i, j] == 0.0
        ot, _ = orc.fwd_tiled(Q, K, np.eye(N), 0.9, 4, 3, mask, window)
        assert np.max(np.abs(ot.sum(1) - 1.0)) <= 1e-14
        # V = ones: output is exactly one up to rounding
        o1, _ = orc.fwd_dense(Q, K, np.ones((N, N)), 0.9, mask, window)
        assert np.max(np.abs(o1 - 1.0)) <= 1e-14


def pin_large_logits(orc):
    """P2 numerical check: the running-max correction stays finite and correct
    for large logits (here |z| up to ~800, where exp(z) overflows double)."""
    N, d = 16, 8
    Q, K, V = _rand((N, d), 41), _rand((N, d), 42), _rand((N, d), 43)
    scale = 800.0 / np.max(np.abs(Q @ K.T))
    with np.errstate(over="ignore", invalid="ignore"):
        naive = np.exp(scale * Q @ K.T)
        assert not np.all(np.isfinite(naive / naive.sum(1, keepdims=True)))  # negative control
    for mask, window in (("none", 0), ("causal", 0), ("local", 2)):
        od, ld = orc.fwd_dense(Q, K, V, scale, mask, window)
        assert np.all(np.isfinite(od)) and np.all(np.isfinite(ld))
        orf, lrf = torch_reference(Q, K, V, scale, mask, window)
        assert np.max(np.abs(od - orf)) <= 1e-12 and np.max(np.abs(ld - lrf)) <= 1e-9
        for Br, Bc in ((1, 1), (4, 3), (16, 5)):
            ot, lt = orc.fwd_tiled(Q, K, V, scale, Br, Bc, mask, window)
            assert np.all(np.isfinite(ot)) and np.max(np.abs(ot - od)) <= 1e-12
            assert np.max(np.abs(lt - ld)) <= 1e-9
    # hardmax limit: with a huge scale each row picks the V row of its top score
    z = Q @ K.T
    o, _ = orc.fwd_dense(Q, K, V, 1e6, "none", 0)
    assert np.max(np.abs(o - V[np.argmax(z, axis=1)])) <= 1e-12


def pin_special_cases(orc):
    N, d = 9, 4
    Q, K, V = _rand((N, d), 51), _rand((N, d), 52), _rand((N, d), 53)
    for mask, window in (("none", 0), ("causal", 0), ("local", 1)):
        # scale 0: uniform weights over the allowed keys
        o, lse = orc.fwd_dense(Q, K, V, 0.0, mask, window)
        ot, lt = orc.fwd_tiled(Q, K, V, 0.0, 2, 4, mask, window)
        for i in range(N):
            js = [j for j in range(N) if orc.allowed(i, j, mask, window)]
            assert np.max(np.abs(o[i] - V[js].mean(0))) <= 1e-14
            assert abs(lse[i] - math.log(len(js))) <= 1e-14
            assert np.max(np.abs(ot[i] - V[js].mean(0))) <= 1e-14
        # constant V rows give that constant
        c = np.tile(np.array([1.5, -2.0, 0.25, 3.0]), (N, 1))
        oc, _ = orc.fwd_dense(Q, K, c, 0.7, mask, window)
        assert np.max(np.abs(oc - c)) <= 1e-14
        # negative scale equals positive scale with Q negated
        on, ln_ = orc.fwd_dense(Q, K, V, -0.7, mask, window)
        op, lp = orc.fwd_dense(-Q, K, V, 0.7, mask, window)
        assert np.max(np.abs(on - op)) <= 1e-15 and np.max(np.abs(ln_ - lp)) <= 1e-15
    # causal row 0 sees only key 0
    o, lse = orc.fwd_dense(Q, K, V, 0.6, "causal", 0)
    assert np.max(np.abs(o[0] - V[0])) <= 1e-15
    assert abs(lse[0] - 0.6 * float(Q[0] @ K[0])) <= 1e-14
    # all keys equal: uniform weights, LSE = z + ln N
    Ke = np.tile(K[3], (N, 1))
    o, lse = orc.fwd_dense(Q, Ke, V, 0.6)
    assert np.max(np.abs(o - V.mean(0))) <= 1e-14
    assert np.max(np.abs(lse - (0.6 * Q @ K[3] + math.log(N)))) <= 1e-13
    # window wider than the sequence equals no mask
    a = orc.fwd_dense(Q, K, V, 0.6, "local", N)
    b = orc.fwd_dense(Q, K, V, 0.6, "none", 0)
    assert np.max(np.abs(a[0] - b[0])) == 0.0


def pin_mask_matrix(orc):
    g = golden("p3_local_window_matrix.json")
    N, w = g["N"], g["window_radius"]
    got = [[int(orc.allowed(i, j, "local", w)) for j in range(N)] for i in range(N)]
    assert got == g["allowed"]
    assert [[int(orc.allowed(i, j, "causal")) for j in range(4)] for i in range(4)] == \
        [[1, 0, 0, 0], [1, 1, 0, 0], [1, 1, 1, 0], [1, 1, 1, 1]]
    assert all(orc.allowed(i, j, "none") for i in range(5) for j in range(5))


def pin_fully_masked_row_in_visited_tile(orc):
    """Rows that have no allowed key inside a visited key tile (band mask)
    must leave their running state untouched, with no NaN."""
    N, d = 6, 4
    Q, K, V = _rand((N, d), 61), _rand((N, d), 62), _rand((N, d), 63)
    od, ld = orc.fwd_dense(Q, K, V, 0.5, "local", 1)
    _, _, tm, tl, to = orc.fwd_tiled(Q, K, V, 0.5, 2, 2, "local", 1, trace=True)
    # row 5 has no key in tile 0 -> still empty after tile 0
    assert tm[0, 0, 5] == -np.inf and tl[0, 0, 5] == 0.0
    # row 0 has no key in tile 1 -> unchanged from tile 0 to tile 1
    assert tm[0, 1, 0] == tm[0, 0, 0] and tl[0, 1, 0] == tl[0, 0, 0]
    ot, lt = orc.fwd_tiled(Q, K, V, 0.5, 2, 2, "local", 1)
    assert np.all(np.isfinite(ot)) and np.max(np.abs(ot - od)) <= 1e-14
    assert np.max(np.abs(lt - ld)) <= 1e-14


# ------------------------------------------------------------------ backward
def _loss(orc, Q, K, V, dO, scale, mask, window):
    o, _ = orc.fwd_dense(Q, K, V, scale, mask, window)
    return float(np.sum(o * dO))


def pin_backward_finite_difference(orc):
    h = 1e-6
    for seed, (N, d, mask, window) in enumerate([(5, 3, "none", 0), (7, 2, "causal", 0),
                                                 (8, 4, "local", 1), (6, 1, "local", 2)]):
        Q, K, V, dO = (_rand((N, d), 70 + 4 * seed + t) for t in range(4))
        scale = 0.9
        g = orc.bwd_dense(Q, K, V, dO, scale, mask, window)
        for name, X in (("dq", Q), ("dk", K), ("dv", V)):
            num = np.zeros_like(X)
            for idx in np.ndindex(X.shape):
                Xp, Xm = X.copy(), X.copy()
                Xp[idx] += h
                Xm[idx] -= h
                args = {"dq": (Xp, K, V), "dk": (Q, Xp, V), "dv": (Q, K, Xp)}[name]
                argm = {"dq": (Xm, K, V), "dk": (Q, Xm, V), "dv": (Q, K, Xm)}[name]
                num[idx] = (_loss(orc, *args, dO, scale, mask, window)
                            - _loss(orc, *argm, dO, scale, mask, window)) / (2 * h)
            err = np.max(np.abs(num - g[name])) / max(1e-12, np.max(np.abs(num)))
            assert err <= 1e-6, (name, mask, err)


def pin_backward_invariants(orc):
    N, d = 10, 4
    Q, K, V, dO = (_rand((N, d), 90 + t) for t in range(4))
    for mask, window in (("none", 0), ("causal", 0), ("local", 2)):
        g = orc.bwd_dense(Q, K, V, dO, 0.7, mask, window)
        # logits of a row shift together when every key moves by the same vector
        assert np.max(np.abs(g["dk"].sum(0))) <= 1e-13
        # probability rows sum to one
        assert np.max(np.abs(g["dv"].sum(0) - dO.sum(0))) <= 1e-13
        # the backward's own O and LSE agree with the forward oracle
        of, lf = orc.fwd_dense(Q, K, V, 0.7, mask, window)
        assert np.max(np.abs(g["o"] - of)) <= 1e-14 and np.max(np.abs(g["lse"] - lf)) <= 1e-14
        assert np.max(np.abs(g["D"] - (dO * of).sum(1))) <= 1e-13
        # all V rows equal: the output ignores P, so dQ = dK = 0
        Vc = np.tile(V[2], (N, 1))
        gc = orc.bwd_dense(Q, K, Vc, dO, 0.7, mask, window)
        assert np.max(np.abs(gc["dq"])) <= 1e-13 and np.max(np.abs(gc["dk"])) <= 1e-13


def pin_backward_against_autograd(orc):
    for seed, (BH, N, d, mask, window) in enumerate([(2, 13, 4, "none", 0), (1, 20, 8, "causal", 0),
                                                     (2, 9, 3, "local", 2)]):
        Q, K, V, dO = (_rand((BH, N, d), 130 + 4 * seed + t) for t in range(4))
        scale = 1.0 / math.sqrt(d)
        g = orc.bwd_dense(Q, K, V, dO, scale, mask, window)
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (Q, K, V))
        s = scale * (tq @ tk.transpose(-1, -2))
        i = torch.arange(N).view(-1, 1)
        j = torch.arange(N).view(1, -1)
        if mask == "causal":
            s = s.masked_fill(~(j <= i), float("-inf"))
        elif mask == "local":
            s = s.masked_fill(~((i - j).abs() <= window), float("-inf"))
        o = torch.softmax(s, -1) @ tv
        (o * torch.tensor(dO)).sum().backward()
        for name, t in (("dq", tq), ("dk", tk), ("dv", tv)):
            assert np.max(np.abs(g[name] - t.grad.numpy())) <= 1e-12, (name, mask)


def pin_backward_rows_match_dense(orc):
    """The row-sampled backward (used for full-size sampled checks) returns
    exactly the rows of the dense backward, which the finite-difference and
    autograd pins fix, for every mask, edge rows and several heads."""
    BH, N, d = 3, 29, 5
    Q, K, V, dO = (_rand((BH, N, d), 120 + t) for t in range(4))
    qb = np.array([0, 0, 1, 2, 2, 1]); qr = np.array([0, N - 1, 7, 13, 28, 1])
    kb = np.array([2, 1, 0, 0, 1]); kr = np.array([0, N - 1, 3, 28, 14])
    for mask, window in (("none", 0), ("causal", 0), ("local", 2), ("local", 0)):
        ref = orc.bwd_dense(Q, K, V, dO, 0.6, mask, window)
        got = orc.bwd_rows(Q, K, V, dO, 0.6, qb, qr, kb, kr, mask, window)
        assert np.max(np.abs(got["dq"] - ref["dq"][qb, qr])) <= 1e-13, mask
        assert np.max(np.abs(got["dk"] - ref["dk"][kb, kr])) <= 1e-13, mask
        assert np.max(np.abs(got["dv"] - ref["dv"][kb, kr])) <= 1e-13, mask


ALL_PINS = [
    pin_p3_worked_example, pin_p2_recurrence, pin_partial_is_dense_over_prefix,
    pin_tiled_equals_dense_toy, pin_against_library, pin_rows_sum_to_one, pin_large_logits,
    pin_special_cases, pin_mask_matrix, pin_fully_masked_row_in_visited_tile,
    pin_backward_finite_difference, pin_backward_invariants, pin_backward_against_autograd,
    pin_backward_rows_match_dense,
]
