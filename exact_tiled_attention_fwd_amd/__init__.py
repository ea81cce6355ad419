"""Exact tiled attention for MI355X (gfx950): O = softmax(scale Q K^T) V.

The computation runs in hand-written HIP kernels behind the C ABI of
include/fa.h (libfa.so). This package is the thin Python side: the ctypes
binding (same names as the C entry points of include/fa.h and the roofline
probes of include/fa_probe.h) plus two convenience wrappers that allocate
outputs with torch.
"""
import math

import torch

from ._native import (FAError, fa_bwd, fa_bwd_noalloc, fa_bwd_standard,
                      fa_bwd_standard_workspace_bytes, fa_bwd_tuned, fa_bwd_workspace_bytes, fa_fwd,
                      fa_fwd_keymajor, fa_fwd_keymajor_workspace_bytes, fa_fwd_standard,
                      fa_fwd_standard_workspace_bytes, fa_fwd_tuned, fa_probe_copy,
                      fa_probe_mfma_bf16, fa_status_string, load)

__all__ = ["FAError", "fa_fwd", "fa_bwd", "fa_bwd_workspace_bytes", "fa_status_string", "load",
           "fa_fwd_tuned", "fa_bwd_tuned", "fa_bwd_noalloc", "fa_bwd_standard",
           "fa_bwd_standard_workspace_bytes",
           "fa_fwd_standard", "fa_fwd_standard_workspace_bytes", "fa_fwd_keymajor",
           "fa_fwd_keymajor_workspace_bytes", "fa_probe_mfma_bf16",
           "fa_probe_copy", "attention_fwd", "attention_bwd"]


def _default_scale(d):
    return 1.0 / math.sqrt(d)


def attention_fwd(q, k, v, scale=None, mask=None, window=0, stream=None):
    """Allocate O and LSE and run fa_fwd. Returns (o, lse)."""
    if scale is None:
        scale = _default_scale(q.shape[-1])
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    fa_fwd(q, k, v, o, lse, scale, mask, window, stream)
    return o, lse


def attention_bwd(q, k, v, o, lse, dout, scale=None, mask=None, window=0, stream=None):
    """Allocate dQ, dK, dV and the workspace and run fa_bwd. Returns (dq, dk, dv)."""
    if scale is None:
        scale = _default_scale(q.shape[-1])
    B, H, N, d = q.shape
    ws = torch.empty(fa_bwd_workspace_bytes(B, H, N, d, q.dtype), dtype=torch.uint8,
                     device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, ws, scale, mask, window, stream)
    return dq, dk, dv
