"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no arithmetic of the method: it only draws random tensors.
Each tensor is keyed by (seed, tensor id, index) through SplitMix64, so any
expert's weights can be regenerated on their own.  Values are drawn with
torch's generator on the device the tensor is made on; the CPU and GPU
generators are different streams, so a test draws a tensor once and hands the
same values (copied to the host) to the oracle.
"""
from __future__ import annotations

import torch

# tensor ids
X = 1          # activations
W = 2          # dense weight
ROUTER = 3     # router weight [E][H]
BIAS = 4       # per-expert router bias
GATE = 5
UP = 6
DOWN = 7
LOGITS = 8

_M64 = (1 << 64) - 1


def _splitmix64(z: int) -> int:
    z = (z + 0x9E3779B97F4A7C15) & _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def key(seed: int, tensor_id: int, index: int = 0) -> int:
    z = _splitmix64(seed & _M64)
    z = _splitmix64(z ^ (tensor_id & _M64))
    z = _splitmix64(z ^ (index & _M64))
    return z & ((1 << 63) - 1)


def normal(shape, std: float, seed: int, tensor_id: int, index: int = 0,
           device="cpu", mean: float = 0.0) -> torch.Tensor:
    """fp32 tensor ~ N(mean, std^2)."""
    g = torch.Generator(device=device)
    g.manual_seed(key(seed, tensor_id, index))
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    if mean != 0.0:
        t.add_(mean)
    return t


def uniform_int(shape, lo: int, hi: int, seed: int, tensor_id: int, index: int = 0,
                device="cpu") -> torch.Tensor:
    """int64 tensor uniform on [lo, hi)."""
    g = torch.Generator(device=device)
    g.manual_seed(key(seed, tensor_id, index))
    return torch.randint(lo, hi, shape, generator=g, device=device)


def expert_weights(e: int, H: int, I: int, seed: int = 0, std: float = 0.02, device="cpu"):
    """gate [I][H], up [I][H], down [H][I] of expert e."""
    return (normal((I, H), std, seed, GATE, e, device),
            normal((I, H), std, seed, UP, e, device),
            normal((H, I), std, seed, DOWN, e, device))
