"""Seeded synthetic inputs (activations, output gradients, weights).

Holds none of the method's arithmetic: only draws of the value distributions
the workloads use, in bf16 (or fp32) on the CPU, from torch's seeded CPU
generator, so that both the GPU path and the CPU oracle see identical bits.
"""
from __future__ import annotations

import numpy as np
import torch


def _gen(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) & 0x7FFFFFFFFFFFFFFF)
    return g


def normal_bf16(shape, std: float, seed: int, device="cpu") -> torch.Tensor:
    """N(0, std^2) rounded to bf16, drawn on `device` (large workloads draw on
    the GPU and copy the bits to the host for the oracle)."""
    x = torch.randn(*shape, generator=_gen(seed, device), dtype=torch.float32, device=device)
    return (x * std).to(torch.bfloat16)


def student_t_bf16(shape, nu: float, seed: int, device="cpu") -> torch.Tensor:
    """Student-t with nu degrees of freedom scaled to unit variance (nu > 2), bf16."""
    g = _gen(seed, device)
    z = torch.randn(*shape, generator=g, dtype=torch.float32, device=device)
    # chi-square(nu) as a sum of nu squared normals (nu integer here)
    chi = torch.zeros(*shape, dtype=torch.float32, device=device)
    for _ in range(int(nu)):
        chi += torch.randn(*shape, generator=g, dtype=torch.float32, device=device) ** 2
    t = z / torch.sqrt(chi / nu)
    return (t * float(np.sqrt((nu - 2.0) / nu))).to(torch.bfloat16)


def normal_f32(shape, std: float, seed: int) -> torch.Tensor:
    x = torch.randn(*shape, generator=_gen(seed), dtype=torch.float32)
    return x * std


def uniform_f32_bits(shape, seed: int) -> torch.Tensor:
    """Random fp32 bit patterns (finite and special), as an int32 tensor view source."""
    g = _gen(seed)
    return torch.randint(-(2**31), 2**31 - 1, shape, generator=g, dtype=torch.int64).to(torch.int32)


def to_numpy_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> uint16 bit patterns (numpy), for the oracle."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def from_numpy_bits(a: np.ndarray) -> torch.Tensor:
    """uint16 bit patterns -> bf16 CPU tensor."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
