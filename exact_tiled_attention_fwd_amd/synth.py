"""Seeded synthetic inputs for attention workloads.

This module only draws random tensors and names workload shapes; it holds
none of the attention arithmetic. Both the GPU parity tests and the CPU
oracle read the same host tensors produced here (for multi-GB tensors, the
same recipe runs on the device and the oracle reads slices copied back).

Recipe: one ``torch.Generator`` per workload seeded with the workload's seed,
``torch.randn`` in float32 on the CPU, drawn in the order Q, K, V (then dO);
optional power-of-two multiplier on Q and K (exact in any binary format);
then, for bf16 workloads, round-to-nearest-even to bfloat16. The shapes
follow the pages' toy run (TensorViz "Compute attention one tile at a time":
[1, 6, 4] float32 randn, seed 0) and the attention shapes the workloads below
name.
"""
from dataclasses import dataclass, field
import math

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str            # "fp32" or "bf16"
    mask: str = "none"    # "none" | "causal" | "local"
    window: int = 0       # band radius when mask == "local": |i - j| <= window
    seed: int = 0
    qk_mult: float = 1.0  # multiplier on Q and K (power of two)
    backward: bool = False
    tiles: tuple = field(default=())  # oracle tile sizes exercised (toy case)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def shape(self):
        return (self.B, self.H, self.N, self.d)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16


WORKLOADS = {
    w.name: w for w in [
        Workload("toy_fp32_n6_d4", 1, 1, 6, 4, "fp32", seed=0, tiles=(1, 2, 3, 4, 6)),
        Workload("bf16_b4h16_n2048_d64", 4, 16, 2048, 64, "bf16", seed=2),
        Workload("bf16_causal_b2h16_n8192_d128", 2, 16, 8192, 128, "bf16", "causal", seed=3),
        Workload("bf16_local128_x8_b1h32_n16384_d128", 1, 32, 16384, 128, "bf16", "local", 128,
                 seed=4, qk_mult=8.0),
        Workload("bf16_causal_bwd_b2h16_n4096_d128", 2, 16, 4096, 128, "bf16", "causal", seed=5,
                 backward=True),
        # the band workload's shape and logit scale, for the backward
        Workload("bf16_local128_x8_bwd_b1h32_n16384_d128", 1, 32, 16384, 128, "bf16", "local",
                 128, seed=6, qk_mult=8.0, backward=True),
    ]
}

# The workload the bench's headline line is taken on (the causal d=128 long
# sequence forward).
HEADLINE = "bf16_causal_b2h16_n8192_d128"


def make_inputs(w: Workload, with_dout: bool = False, shape=None):
    """Return dict of CPU tensors q, k, v (and dout) in the workload's dtype.
    ``shape`` overrides (B, H, N, d) for reduced-size cases of the same recipe."""
    shp = tuple(shape) if shape is not None else w.shape
    g = torch.Generator().manual_seed(w.seed)
    q = torch.randn(shp, generator=g, dtype=torch.float32)
    k = torch.randn(shp, generator=g, dtype=torch.float32)
    v = torch.randn(shp, generator=g, dtype=torch.float32)
    out = {"q": q, "k": k, "v": v}
    if with_dout or w.backward:
        out["dout"] = torch.randn(shp, generator=g, dtype=torch.float32)
    if w.qk_mult != 1.0:
        out["q"] = out["q"] * w.qk_mult
        out["k"] = out["k"] * w.qk_mult
    return {n: t.to(w.torch_dtype).contiguous() for n, t in out.items()}


def random_inputs(shape, dtype=torch.bfloat16, seed=0, qk_mult=1.0, with_dout=False):
    """Same recipe for an arbitrary shape (edge-case tests)."""
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(shape, generator=g, dtype=torch.float32) * qk_mult
    k = torch.randn(shape, generator=g, dtype=torch.float32) * qk_mult
    v = torch.randn(shape, generator=g, dtype=torch.float32)
    out = {"q": q, "k": k, "v": v}
    if with_dout:
        out["dout"] = torch.randn(shape, generator=g, dtype=torch.float32)
    return {n: t.to(dtype).contiguous() for n, t in out.items()}


def device_inputs(shape, dtype=torch.bfloat16, seed=0, with_dout=False, device="cuda"):
    """The same recipe drawn by a generator on `device`, for tensors too large
    to draw and copy from the host (several GB each). The values differ from
    random_inputs with the same seed; a test hands the oracle slices copied
    back from these tensors."""
    g = torch.Generator(device=device).manual_seed(seed)
    out = {}
    for n in ("q", "k", "v") + (("dout",) if with_dout else ()):
        out[n] = torch.randn(shape, generator=g, dtype=torch.float32, device=device).to(dtype)
    return out
