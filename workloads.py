"""Seeded synthetic inputs of the NVFP4 layer workloads.

Shared by the tests, the benchmark and the smoke check; it holds no NVFP4
arithmetic.  Every tensor is drawn on the CPU from torch's generator with a
fixed seed, so the GPU path and the CPU oracle see identical values.

Distributions (the layer shapes of a 12B-class FFN up-projection, K = 5120 ->
N = 20480, no dataset or trained weights available):
  activations X   N(0, 1), a Bernoulli(0.1%) subset multiplied by 50
  weights W       N(0, 0.02^2)
  gradients dY    Laplace(0, b = 1e-4), a Bernoulli(0.05%) subset x 100
  tiny operands   N(0, 1), a Bernoulli(1%) subset x 30 (fp32)
Outlier masks come from the same generator, after the base values.
"""
from __future__ import annotations

import torch

SEED_TINY, SEED_X, SEED_W, SEED_DY = 0, 1, 2, 3
SR_SEED = 1234
RHT_SEED = 0


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator()
    g.manual_seed(seed)
    return g


def _outliers(x: torch.Tensor, g: torch.Generator, p: float, mul: float) -> torch.Tensor:
    mask = torch.rand(x.shape, generator=g) < p
    x[mask] *= mul
    return x


def activations(M: int, K: int, seed: int = SEED_X, dtype=torch.bfloat16) -> torch.Tensor:
    g = _gen(seed)
    x = torch.randn(M, K, generator=g)
    return _outliers(x, g, 1e-3, 50.0).to(dtype)


def weights(N: int, K: int, seed: int = SEED_W, dtype=torch.bfloat16) -> torch.Tensor:
    g = _gen(seed)
    return (torch.randn(N, K, generator=g) * 0.02).to(dtype)


def gradients(M: int, N: int, seed: int = SEED_DY, dtype=torch.bfloat16) -> torch.Tensor:
    g = _gen(seed)
    e1 = torch.empty(M, N).exponential_(1.0, generator=g)
    e2 = torch.empty(M, N).exponential_(1.0, generator=g)
    x = (e1 - e2) * 1e-4  # difference of two Exp(1) draws is Laplace(0, 1)
    return _outliers(x, g, 5e-4, 100.0).to(dtype)


def tiny_pair(seed: int = SEED_TINY):
    """A [64, 256] and B [128, 256] fp32, N(0,1) with 1% of entries x 30."""
    g = _gen(seed)
    a = _outliers(torch.randn(64, 256, generator=g), g, 1e-2, 30.0)
    b = _outliers(torch.randn(128, 256, generator=g), g, 1e-2, 30.0)
    return a, b


# The layer shapes: Fprop / Dgrad / Wgrad / full layer.
LAYER_M, LAYER_K, LAYER_N = 8192, 5120, 20480
