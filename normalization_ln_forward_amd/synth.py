"""Seeded synthetic inputs for the normalization forward passes.

This module only draws random tensors of the workloads' shapes and value
distributions; it holds none of the normalization arithmetic and is shared by
the tests, the smoke check and the benchmark (the one module both the GPU
path's callers and the oracle's callers use).

Workloads (shapes from the three pages' problem statements, distributions as
stated for each workload below):
  gn   GroupNorm+LeakyReLU+x2   x [1024, 8192] ~ N(0,1), 512 groups of 16 channels,
                                gamma ~ N(1, 0.1), beta ~ N(0, 0.1), eps 1e-5, slope 0.01
  ln   LayerNorm                x [16, 64, 256, 256] ~ N(0,1), normalized over (64,256,256),
                                weight ~ N(1, 0.1), bias ~ N(0, 0.1), eps 1e-5
  rms  RMSNorm over dim 1       x [112, 64, 512, 512] ~ N(0,1), eps 1e-5, no affine
  ln_stress  LayerNorm          as ln with x ~ N(100, 0.01) (large mean, tiny variance)
  fc_gn  fc -> GN epilogue      x [1024, 8192] ~ N(0,1), W [8192, 8192] and b [8192]
                                ~ U(-1/sqrt(8192), 1/sqrt(8192)), then the gn epilogue
Draws use torch.Generator(device).manual_seed(seed) in a fixed order per
workload (x, then W, b, then the affine tensors), so a (workload, shape,
seed, device) tuple always yields the same tensors.
"""
import math
from dataclasses import dataclass, field
from typing import Dict, Tuple

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                       # "gn" | "ln" | "rms" | "fc_gn"
    shape: Tuple[int, ...]          # x's shape
    x_dist: Tuple[str, float, float]
    params: Dict[str, float] = field(default_factory=dict)


WORKLOADS = {
    "gn_lrelu_x2_1024x8192": Workload(
        "gn_lrelu_x2_1024x8192", "gn", (1024, 8192), ("normal", 0.0, 1.0),
        {"num_groups": 512, "eps": 1e-5, "negative_slope": 0.01}),
    "ln_16x64x256x256": Workload(
        "ln_16x64x256x256", "ln", (16, 64, 256, 256), ("normal", 0.0, 1.0),
        {"normalized_ndim": 3, "eps": 1e-5}),
    "rms_ch_112x64x512x512": Workload(
        "rms_ch_112x64x512x512", "rms", (112, 64, 512, 512), ("normal", 0.0, 1.0),
        {"eps": 1e-5}),
    "ln_stress_16x64x256x256": Workload(
        "ln_stress_16x64x256x256", "ln", (16, 64, 256, 256), ("normal", 100.0, 0.01),
        {"normalized_ndim": 3, "eps": 1e-5}),
    "fc_gn_1024x8192x8192": Workload(
        "fc_gn_1024x8192x8192", "fc_gn", (1024, 8192), ("normal", 0.0, 1.0),
        {"hidden": 8192, "num_groups": 512, "eps": 1e-5, "negative_slope": 0.01}),
}

# The order the workloads are listed in (index i uses seed 1000 + i by default).
ORDER = ["gn_lrelu_x2_1024x8192", "ln_16x64x256x256", "rms_ch_112x64x512x512",
         "ln_stress_16x64x256x256", "fc_gn_1024x8192x8192"]


def default_seed(name: str) -> int:
    return 1000 + ORDER.index(name)


def _draw(shape, dist, gen, device):
    kind, a, b = dist
    if kind == "normal":
        t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
        return t.mul_(b).add_(a)
    if kind == "uniform":  # U(a, b)
        t = torch.rand(shape, generator=gen, device=device, dtype=torch.float32)
        return t.mul_(b - a).add_(a)
    raise ValueError(kind)


def make(name: str, device="cpu", seed=None, shape=None, x_dist=None, **overrides):
    """Draw one workload's tensors.

    ``shape`` replaces the workload's x shape (same distributions), which the
    parity tests use for small and ragged cases.  Returns a dict of float32
    tensors on ``device`` plus the scalar parameters.
    """
    wl = WORKLOADS[name]
    shape = tuple(shape) if shape is not None else wl.shape
    seed = default_seed(name) if seed is None else seed
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    out = dict(wl.params)
    out.update(overrides)
    out["x"] = _draw(shape, x_dist or wl.x_dist, gen, device)
    if wl.kind == "ln":
        nd = out["normalized_ndim"]
        nshape = shape[len(shape) - nd:]
        out["weight"] = _draw(nshape, ("normal", 1.0, 0.1), gen, device)
        out["bias"] = _draw(nshape, ("normal", 0.0, 0.1), gen, device)
    elif wl.kind == "gn":
        C = shape[1]
        out["gamma"] = _draw((C,), ("normal", 1.0, 0.1), gen, device)
        out["beta"] = _draw((C,), ("normal", 0.0, 0.1), gen, device)
    elif wl.kind == "fc_gn":
        K = shape[1]
        hidden = out["hidden"]
        bound = 1.0 / math.sqrt(K)
        out["W"] = _draw((hidden, K), ("uniform", -bound, bound), gen, device)
        out["b"] = _draw((hidden,), ("uniform", -bound, bound), gen, device)
        out["gamma"] = _draw((hidden,), ("normal", 1.0, 0.1), gen, device)
        out["beta"] = _draw((hidden,), ("normal", 0.0, 0.1), gen, device)
    return out
