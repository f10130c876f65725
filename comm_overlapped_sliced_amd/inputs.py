"""Seeded synthetic inputs for the Flash-AG / Flash-RS workloads.

This module only draws numbers: it holds none of the method's arithmetic, so the CPU oracle's
tests and the HIP path can take their operands from the same place without sharing any
computation. bf16 operands are returned as ``uint16`` bit patterns (the upper half of the fp32
pattern after round-to-nearest-even), fp32 operands as ``float32``.

Generator: numpy ``Generator(PCG64(seed))`` with ``seed = 1000 * config + tensor_id``
(activation = 1, weight = 2, incoming partial from peer q = 10 + q).
"""
from __future__ import annotations

import numpy as np

X_ID = 1
W_ID = 2
PARTIAL_ID = 10


def seed_for(config: int, tensor_id: int) -> int:
    return 1000 * config + tensor_id


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to the nearest bf16 (ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 (for inspecting inputs)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal(seed: int, shape, std: float, dtype: str) -> np.ndarray:
    """N(0, std^2) samples, drawn in float32, stored as bf16 bits or float32."""
    x = _rng(seed).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


def integers(seed: int, shape, lo: int, hi: int, dtype: str) -> np.ndarray:
    """Integers uniform on the closed range [lo, hi], stored exactly as bf16 bits or float32."""
    x = _rng(seed).integers(lo, hi + 1, size=shape).astype(np.float32)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


def draw(config: int, tensor_id: int, shape, dist: tuple, dtype: str) -> np.ndarray:
    """dist is ("normal", std) or ("int", lo, hi)."""
    seed = seed_for(config, tensor_id)
    if dist[0] == "normal":
        return normal(seed, shape, dist[1], dtype)
    if dist[0] == "int":
        return integers(seed, shape, dist[1], dist[2], dtype)
    raise ValueError(f"unknown distribution {dist!r}")
