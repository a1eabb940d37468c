"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle's
callers.  This module holds no attention arithmetic: it only draws N(0, 1)
values from a seeded torch generator and rounds them to the storage dtype
(fp32 -> bf16 is round-to-nearest-even, torch's conversion).

Seed recipe: base 1234 + 1000 * workload + 100 * layer + tensor offset, with
offsets Q:0 K:1 V:2 dO:3 q_dec:4 k_new:5 v_new:6 cache:7.
"""

from __future__ import annotations

import torch

TENSOR_OFFSET = {"q": 0, "k": 1, "v": 2, "do": 3, "q_dec": 4, "k_new": 5,
                 "v_new": 6, "cache": 7, "cache_v": 8}


def seed_for(workload: int, layer: int, tensor: str) -> int:
    return 1234 + 1000 * workload + 100 * layer + TENSOR_OFFSET[tensor]


def randn(shape, seed: int, dtype=torch.bfloat16, device="cpu"):
    """N(0,1) float32 draws from a seeded generator on ``device``, rounded to
    ``dtype``.  The same (shape, seed, device) always gives the same bytes."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(*shape, generator=g, dtype=torch.float32, device=device)
    return x.to(dtype)


def as_f64(t):
    """Exact float64 numpy copy of a (possibly device, possibly bf16) tensor."""
    return t.detach().to("cpu", torch.float64).numpy()
