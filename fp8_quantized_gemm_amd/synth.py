"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no arithmetic of the method (no quantization, no GEMM, no
byte split): it only draws normal samples and rounds them to the 16-bit input
dtype with torch's own conversion.  Both the HIP path and the oracle receive
exactly the tensors made here.

Shapes and distributions stand in for the trained Llama-7B / Qwen-32B weights
and real activations of the pages' workloads, which are not available:
weights ~ N(0, 0.02) (Qwen-32B shapes: N(0, 0.015)) stored as fp16, activations
~ N(0, 1) stored as bf16 (fp16 for the NestedFP layers), optionally with 0.1%
of the channels scaled by 50 (prefill "outlier channels").
"""
from __future__ import annotations

import numpy as np
import torch

BASE_SEED = 0xF8E43A00

# Linear shapes (K -> N) of one transformer layer.
LLAMA7B_LINEARS = (
    ("qkv", 4096, 12288),
    ("o", 4096, 4096),
    ("gate_up", 4096, 22016),
    ("down", 11008, 4096),
)
QWEN32B_LINEARS = (
    ("qkv", 5120, 10240),
    ("o", 8192, 5120),
    ("gate_up", 5120, 51200),
    ("down", 25600, 5120),
)


def seed_for(*parts) -> int:
    """A stable 63-bit seed from a tuple of ints/strings (FNV-1a over the repr)."""
    h = 0xCBF29CE484222325
    for b in repr((BASE_SEED,) + tuple(parts)).encode():
        h ^= b
        h = (h * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
    return h & 0x7FFFFFFFFFFFFFFF


def _torch_dtype(dtype: str):
    return {"bf16": torch.bfloat16, "fp16": torch.float16}[dtype]


def normal(shape, sigma: float, dtype: str, seed: int, device: str = "cpu") -> torch.Tensor:
    """N(0, sigma^2) samples rounded to `dtype` ('bf16' | 'fp16') on `device`.

    On the CPU the draw is numpy's PCG64; on a GPU it is torch's device
    generator (much faster for multi-GB weights).  Either way the result is a
    deterministic function of (shape, sigma, dtype, seed, device kind).
    """
    shape = tuple(int(s) for s in shape)
    if device == "cpu":
        rng = np.random.Generator(np.random.PCG64(seed))
        v = rng.standard_normal(shape, dtype=np.float32) * np.float32(sigma)
        return torch.from_numpy(v).to(_torch_dtype(dtype))
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    v = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    v.mul_(sigma)
    return v.to(_torch_dtype(dtype))


def outlier_channels(K: int, seed: int) -> np.ndarray:
    """max(1, round(0.1% of K)) distinct channel indices, by a seeded permutation."""
    count = max(1, int(round(0.001 * K)))
    rng = np.random.Generator(np.random.PCG64(seed))
    return np.sort(rng.permutation(K)[:count])


def activation(M: int, K: int, seed: int, dtype: str = "bf16", outliers: bool = False,
               device: str = "cpu") -> torch.Tensor:
    """Activation [M,K] ~ N(0,1); with `outliers`, 0.1% of channels are x50."""
    shape = (M, K)
    if device == "cpu":
        rng = np.random.Generator(np.random.PCG64(seed))
        v = rng.standard_normal(shape, dtype=np.float32)
        if outliers:
            v[:, outlier_channels(K, seed ^ 0x5A5A)] *= np.float32(50.0)
        return torch.from_numpy(v).to(_torch_dtype(dtype))
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    v = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if outliers:
        idx = torch.from_numpy(outlier_channels(K, seed ^ 0x5A5A)).to(device)
        v[:, idx] *= 50.0
    return v.to(_torch_dtype(dtype))


def bits(t: torch.Tensor) -> np.ndarray:
    """The uint16 bit patterns of a 16-bit tensor, as a host numpy array."""
    assert t.dtype in (torch.bfloat16, torch.float16)
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def from_bits(b: np.ndarray, dtype: str) -> torch.Tensor:
    """Inverse of `bits`: uint16 patterns -> a CPU tensor of `dtype`."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return torch.from_numpy(b.view(np.int16).copy()).view(_torch_dtype(dtype))
