"""CPU oracle for exact attention — TEST INFRASTRUCTURE ONLY.

A ctypes wrapper over ``liboracle.so`` (plain double-precision C in
``oracle.c``). Only ``tests/``, the smoke check and the bench's CPU-baseline
leg may import this package; the GPU path never does, and the two share no
code. Each function names the page passage it follows:

* ``fwd_dense`` / ``fwd_dense_rows`` — the definition ``O = softmax(scale QK^T) V``
  (P3 "The Standard Attention Problem", safe softmax of "Step 1").
* ``fwd_tiled`` — the incremental softmax merge over query/key tiles
  (P3 "Derivation: Incremental Softmax", Steps 2–3; P2 step "tiles").
* ``bwd_dense`` — gradients of ``sum(dO * O)`` by the chain rule (the pages
  give no backward formulas; P3 "Backward Pass: Recomputation" only says S and
  P are recomputed).
* ``allowed`` — the mask predicate (P3 "Worked example Local Attention Window";
  causal j <= i).

Page titles: [P2] TensorViz "Compute attention one tile at a time";
[P3] "Flash attention and efficient attention — Hinglish notes".

Parity status: every function here is pinned by ``tests/test_oracle_*.py``.
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(HERE, "liboracle.so")
MASKS = {"none": 0, None: 0, "causal": 1, "local": 2}

_dp = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)
_i64 = ctypes.c_int64


def _bind(lib):
    lib.oracle_allowed.argtypes = [_i64, _i64, ctypes.c_int, _i64]
    lib.oracle_allowed.restype = ctypes.c_int
    lib.oracle_attn_fwd_dense.argtypes = [_dp, _dp, _dp, _dp, _dp, _i64, _i64, _i64,
                                          ctypes.c_double, ctypes.c_int, _i64]
    lib.oracle_attn_fwd_dense.restype = None
    lib.oracle_attn_fwd_dense_rows.argtypes = [_dp, _dp, _dp, _i64, _i64, _i64, ctypes.c_double,
                                               ctypes.c_int, _i64, _i64p, _i64p, _i64, _dp, _dp]
    lib.oracle_attn_fwd_dense_rows.restype = None
    lib.oracle_attn_fwd_tiled.argtypes = [_dp, _dp, _dp, _dp, _dp, _i64, _i64, _i64,
                                          ctypes.c_double, ctypes.c_int, _i64, _i64, _i64,
                                          _dp, _dp, _dp]
    lib.oracle_attn_fwd_tiled.restype = ctypes.c_int
    lib.oracle_attn_bwd_dense.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _dp, _i64, _i64, _i64,
                                          ctypes.c_double, ctypes.c_int, _i64, _dp, _dp, _dp]
    lib.oracle_attn_bwd_dense.restype = ctypes.c_int
    lib.oracle_attn_bwd_rows.argtypes = [_dp, _dp, _dp, _dp, _i64, _i64, _i64, ctypes.c_double,
                                         ctypes.c_int, _i64, _i64p, _i64p, _i64, _i64p, _i64p,
                                         _i64, _dp, _dp, _dp]
    lib.oracle_attn_bwd_rows.restype = ctypes.c_int
    return lib


def _f64(a):
    """Contiguous float64 copy/view of an array-like (bf16 torch tensors are
    widened exactly: every bf16 value is a double)."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return a.ctypes.data_as(_dp) if a is not None else None


def _mask_code(mask):
    if mask not in MASKS:
        raise ValueError(f"unknown mask {mask!r}")
    return MASKS[mask]


def _as3(x):
    """[..., N, d] -> ([BH, N, d] float64, leading shape)."""
    x = _f64(x)
    lead = x.shape[:-2]
    return x.reshape((-1,) + x.shape[-2:]), lead


class Oracle:
    """The oracle functions over one loaded copy of the C library. The default
    instance (module-level functions below) loads ``liboracle.so``; tests that
    plant mistakes in a rebuilt copy of ``oracle.c`` load that copy instead."""

    def __init__(self, lib_path=None):
        if lib_path is None:
            lib_path = _LIB_PATH
            if not os.path.exists(lib_path) or (
                    os.path.getmtime(lib_path) < os.path.getmtime(os.path.join(HERE, "oracle.c"))):
                from . import build as _b
                _b.build()
        self.lib = _bind(ctypes.CDLL(lib_path))

    def allowed(self, i, j, mask="none", window=0):
        return bool(self.lib.oracle_allowed(int(i), int(j), _mask_code(mask), int(window)))

    def fwd_dense(self, q, k, v, scale, mask="none", window=0):
        """Dense forward: returns (O, LSE) in float64 with q's leading shape."""
        q3, lead = _as3(q)
        k3, _ = _as3(k)
        v3, _ = _as3(v)
        BH, N, d = q3.shape
        o = np.empty_like(q3)
        lse = np.empty((BH, N), dtype=np.float64)
        self.lib.oracle_attn_fwd_dense(_ptr(q3), _ptr(k3), _ptr(v3), _ptr(o), _ptr(lse), BH, N, d,
                                       float(scale), _mask_code(mask), int(window))
        return o.reshape(lead + (N, d)), lse.reshape(lead + (N,))

    def fwd_dense_rows(self, q, k, v, scale, bh_idx, row_idx, mask="none", window=0):
        """Dense forward for selected rows. q/k/v are [BH, N, d] (or reshaped
        to it); bh_idx/row_idx select the rows. Returns (O rows [n, d], LSE [n])."""
        q3, _ = _as3(q)
        k3, _ = _as3(k)
        v3, _ = _as3(v)
        BH, N, d = q3.shape
        bh_idx = np.ascontiguousarray(np.asarray(bh_idx, dtype=np.int64))
        row_idx = np.ascontiguousarray(np.asarray(row_idx, dtype=np.int64))
        if bh_idx.shape != row_idx.shape or bh_idx.ndim != 1:
            raise ValueError("bh_idx and row_idx must be 1-D of equal length")
        if len(bh_idx) and (bh_idx.min() < 0 or bh_idx.max() >= BH or row_idx.min() < 0
                            or row_idx.max() >= N):
            raise ValueError("row selection out of range")
        n = len(bh_idx)
        o = np.empty((n, d), dtype=np.float64)
        lse = np.empty((n,), dtype=np.float64)
        self.lib.oracle_attn_fwd_dense_rows(_ptr(q3), _ptr(k3), _ptr(v3), BH, N, d, float(scale),
                                            _mask_code(mask), int(window),
                                            bh_idx.ctypes.data_as(_i64p),
                                            row_idx.ctypes.data_as(_i64p), n, _ptr(o), _ptr(lse))
        return o, lse

    def fwd_tiled(self, q, k, v, scale, Br, Bc, mask="none", window=0, trace=False):
        """Tiled online-softmax forward. Returns (O, LSE) or, with trace=True,
        (O, LSE, trace_m [BH,Tc,N], trace_l [BH,Tc,N], trace_o [BH,Tc,N,d])."""
        q3, lead = _as3(q)
        k3, _ = _as3(k)
        v3, _ = _as3(v)
        BH, N, d = q3.shape
        Tc = (N + Bc - 1) // Bc if Bc >= 1 else 0
        o = np.empty_like(q3)
        lse = np.empty((BH, N), dtype=np.float64)
        tm = tl = to = None
        if trace:
            tm = np.empty((BH, Tc, N))
            tl = np.empty((BH, Tc, N))
            to = np.empty((BH, Tc, N, d))
        rc = self.lib.oracle_attn_fwd_tiled(_ptr(q3), _ptr(k3), _ptr(v3), _ptr(o), _ptr(lse), BH,
                                            N, d, float(scale), _mask_code(mask), int(window),
                                            int(Br), int(Bc), _ptr(tm), _ptr(tl), _ptr(to))
        if rc != 0:
            raise ValueError(f"oracle_attn_fwd_tiled failed (Br={Br}, Bc={Bc})")
        out = (o.reshape(lead + (N, d)), lse.reshape(lead + (N,)))
        if trace:
            return out + (tm, tl, to)
        return out

    def bwd_dense(self, q, k, v, dout, scale, mask="none", window=0):
        """Dense backward. Returns dict with dq, dk, dv, o, lse, D (float64)."""
        q3, lead = _as3(q)
        k3, _ = _as3(k)
        v3, _ = _as3(v)
        do3, _ = _as3(dout)
        BH, N, d = q3.shape
        dq = np.empty_like(q3)
        dk = np.empty_like(q3)
        dv = np.empty_like(q3)
        o = np.empty_like(q3)
        lse = np.empty((BH, N))
        D = np.empty((BH, N))
        rc = self.lib.oracle_attn_bwd_dense(_ptr(q3), _ptr(k3), _ptr(v3), _ptr(do3), _ptr(dq),
                                            _ptr(dk), _ptr(dv), BH, N, d, float(scale),
                                            _mask_code(mask), int(window), _ptr(o), _ptr(lse),
                                            _ptr(D))
        if rc != 0:
            raise MemoryError("oracle_attn_bwd_dense: allocation failed")
        sh = lead + (N, d)
        return {"dq": dq.reshape(sh), "dk": dk.reshape(sh), "dv": dv.reshape(sh),
                "o": o.reshape(sh), "lse": lse.reshape(lead + (N,)), "D": D.reshape(lead + (N,))}

    def bwd_rows(self, q, k, v, dout, scale, q_bh, q_row, k_bh, k_row, mask="none", window=0):
        """Backward for chosen rows: dQ of the query rows (q_bh[r], q_row[r])
        and dK, dV of the key rows (k_bh[r], k_row[r]); heads index the
        flattened [B*H] axis. Returns dict with dq [nq, d], dk, dv [nk, d]."""
        q3, _ = _as3(q)
        k3, _ = _as3(k)
        v3, _ = _as3(v)
        do3, _ = _as3(dout)
        BH, N, d = q3.shape
        qb = np.ascontiguousarray(q_bh, dtype=np.int64)
        qr = np.ascontiguousarray(q_row, dtype=np.int64)
        kb = np.ascontiguousarray(k_bh, dtype=np.int64)
        kr = np.ascontiguousarray(k_row, dtype=np.int64)
        for b_, r_ in ((qb, qr), (kb, kr)):
            if b_.shape != r_.shape or (b_.size and (b_.min() < 0 or b_.max() >= BH or
                                                     r_.min() < 0 or r_.max() >= N)):
                raise ValueError("row indices out of range")
        dq = np.empty((qb.size, d))
        dk = np.empty((kb.size, d))
        dv = np.empty((kb.size, d))
        ip = lambda a: a.ctypes.data_as(_i64p)
        rc = self.lib.oracle_attn_bwd_rows(_ptr(q3), _ptr(k3), _ptr(v3), _ptr(do3), BH, N, d,
                                           float(scale), _mask_code(mask), int(window), ip(qb),
                                           ip(qr), qb.size, ip(kb), ip(kr), kb.size, _ptr(dq),
                                           _ptr(dk), _ptr(dv))
        if rc != 0:
            raise MemoryError("oracle_attn_bwd_rows: allocation failed")
        return {"dq": dq, "dk": dk, "dv": dv}


_default = None


def default():
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def allowed(*a, **kw):
    return default().allowed(*a, **kw)


def fwd_dense(*a, **kw):
    return default().fwd_dense(*a, **kw)


def fwd_dense_rows(*a, **kw):
    return default().fwd_dense_rows(*a, **kw)


def fwd_tiled(*a, **kw):
    return default().fwd_tiled(*a, **kw)


def bwd_dense(*a, **kw):
    return default().bwd_dense(*a, **kw)


def bwd_rows(*a, **kw):
    return default().bwd_rows(*a, **kw)
