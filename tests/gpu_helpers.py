"""Shared helpers of the GPU tests: moving seeded numpy operands to the device and back, and the
relative Frobenius error used as the parity measure."""
from __future__ import annotations

import numpy as np

from comm_overlapped_sliced_amd import inputs

TOL_BF16 = 2e-3   # bf16 operands, fp32 accumulation
TOL_F32 = 1e-6    # fp32 operands


def to_dev(a: np.ndarray, dev):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def from_dev(t) -> np.ndarray:
    """Exact fp64 copy of a bf16 or fp32 device tensor."""
    import torch
    if t.dtype == torch.bfloat16:
        bits = t.view(torch.int16).cpu().numpy().view(np.uint16)
        return inputs.bf16_bits_to_f32(bits).astype(np.float64)
    return t.float().cpu().numpy().astype(np.float64)


def rel_frobenius(got: np.ndarray, ref: np.ndarray) -> float:
    got = np.asarray(got, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    n = np.linalg.norm(ref)
    d = np.linalg.norm(got - ref)
    return float(d / n) if n else float(d)


def sample_indices(rows: int, cols: int, n: int, seed: int, block_rows: int = 0):
    """n random (row, col) pairs plus the corners of the matrix and of every block of
    block_rows rows (slice edges), so that edge tiles are always sampled."""
    rng = np.random.default_rng(seed)
    r = list(rng.integers(0, rows, n))
    c = list(rng.integers(0, cols, n))
    starts = range(0, rows, block_rows) if block_rows else [0]
    for s in starts:
        last = min(rows, s + (block_rows or rows)) - 1
        for rr in (s, last):
            for cc in (0, cols - 1, cols // 2):
                r.append(rr)
                c.append(cc)
    return np.array(r, dtype=np.int64), np.array(c, dtype=np.int64)
