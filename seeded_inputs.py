"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle's checks.

This module holds no arithmetic of the method: it only draws random tensors.
Every tensor is drawn in fp32 from a CPU ``torch.Generator`` seeded with

    seed = base + 1_000_000 * chunk + 1000 * pass_idx + tensor_id

and, for bf16 workloads, rounded once to bf16 with round-to-nearest-even
(torch's ``.to(torch.bfloat16)``).  The oracle consumes the exact upcast of
those rounded values, so both sides see bit-identical inputs.
"""
from __future__ import annotations

import numpy as np
import torch

# tensor ids inside one (chunk, pass) draw (NOISE: the sampler's fresh noise / starting latent)
Q, K, V, TEXT_K, TEXT_V, SINK_K, SINK_V, NOISE = 0, 1, 2, 3, 4, 5, 6, 7


def seed_for(base: int, chunk: int, pass_idx: int, tensor_id: int) -> int:
    return int(base) + 1_000_000 * int(chunk) + 1000 * int(pass_idx) + int(tensor_id)


def normal(shape, seed: int, dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """N(0, 1) tensor of ``shape`` drawn in fp32 on the CPU, then cast (RNE) to ``dtype``."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    x = torch.randn(tuple(int(s) for s in shape), generator=g, dtype=torch.float32)
    return x.to(dtype)


def draw(shape, base: int, chunk: int, pass_idx: int, tensor_id: int,
         dtype: torch.dtype = torch.float32) -> torch.Tensor:
    return normal(shape, seed_for(base, chunk, pass_idx, tensor_id), dtype)


def to_f64(x: torch.Tensor) -> np.ndarray:
    """Exact upcast of a CPU float tensor (fp32 or bf16) to a float64 ndarray."""
    return x.detach().to("cpu").to(torch.float64).numpy()
