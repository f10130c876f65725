"""The five workloads of the Flash-AG / Flash-RS hot path, one tensor-parallel rank's share.

Shapes are those of one TP8 rank of the Llama-3.1-70B and -405B MLP projections (gate+up is
column-parallel: All-Gather then GEMM; down is row-parallel: GEMM then Reduce-Scatter).
Each case is synthetic: values come from ``inputs.draw`` with the seeds noted there.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import inputs


@dataclass(frozen=True)
class Case:
    config: int          # workload number (seed base = 1000 * config)
    call: str            # "ag" or "rs"
    P: int               # slices = tensor-parallel degree
    M: int               # tokens (rows of the gathered / sharded activation)
    K: int
    N: int
    dtype: str           # operand dtype: "bf16" or "f32"
    x_dist: tuple
    w_dist: tuple
    part_dist: tuple = ("normal", 1.0)
    name: str = ""

    @property
    def m(self) -> int:
        return self.M // self.P

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    def x(self) -> np.ndarray:
        """Activation [M, K] (AG: the gathered X; RS: this rank's X_shard)."""
        return inputs.draw(self.config, inputs.X_ID, (self.M, self.K), self.x_dist, self.dtype)

    def w(self) -> np.ndarray:
        """Weight shard [K, N], row-major."""
        return inputs.draw(self.config, inputs.W_ID, (self.K, self.N), self.w_dist, self.dtype)

    def partial(self, q: int) -> np.ndarray:
        """Peer q's fp32 [m, N] partial sum for this rank's chunk (RS only)."""
        return inputs.draw(self.config, inputs.PARTIAL_ID + q, (self.m, self.N), self.part_dist,
                           "f32")


_N01 = ("normal", 1.0)
_W = ("normal", 0.02)
_INT = ("int", -3, 3)

TINY_AG = Case(1, "ag", 4, 256, 256, 512, "f32", _INT, _INT, _INT, "tiny fp32 AG-GEMM")
TINY_RS = Case(1, "rs", 4, 256, 256, 512, "f32", _INT, _INT, _INT, "tiny fp32 GEMM-RS")
L70B_AG = Case(2, "ag", 8, 4096, 8192, 7168, "bf16", _N01, _W,
               name="Llama-3.1-70B MLP gate+up AG-GEMM, TP8 rank share")
L70B_RS = Case(3, "rs", 8, 4096, 3584, 8192, "bf16", _N01, _W, _N01,
               name="Llama-3.1-70B MLP down GEMM-RS, TP8 rank share")
SWEEP_AG = tuple(Case(4, "ag", 8, M, 8192, 7168, "bf16", _N01, _W,
                      name=f"70B gate+up AG-GEMM sweep, M={M}")
                 for M in (1024, 2048, 4096, 8192, 16384))
L405B_AG = Case(5, "ag", 8, 8192, 16384, 13312, "bf16", _N01, _W,
                name="Llama-3.1-405B MLP gate+up AG-GEMM, TP8 rank share, seq 8192")
L405B_RS = Case(5, "rs", 8, 8192, 6656, 16384, "bf16", _N01, _W, _N01,
                name="Llama-3.1-405B MLP down GEMM-RS, TP8 rank share, seq 8192")

ALL = (TINY_AG, TINY_RS, L70B_AG, L70B_RS) + SWEEP_AG + (L405B_AG, L405B_RS)


def scaled(case: Case, **kw) -> Case:
    """The same workload with some fields replaced (used for small parity cases)."""
    d = {f: getattr(case, f) for f in case.__dataclass_fields__}
    d.update(kw)
    return Case(**d)


@dataclass(frozen=True)
class AttnCase:
    """One rank's share of attention under Ulysses (sequence) parallelism: after the All-to-All
    the rank holds hq query heads and hkv key/value heads of the whole sequence of S = P*m
    tokens, as P slices of m tokens (one per peer)."""
    config: int
    P: int
    S: int
    hq: int
    hkv: int
    head_dim: int = 128
    causal: bool = True
    name: str = ""

    @property
    def m(self) -> int:
        return self.S // self.P

    @property
    def row(self) -> int:
        """Values per token row: [hq query heads | hkv key heads | hkv value heads] x head_dim."""
        return (self.hq + 2 * self.hkv) * self.head_dim

    @property
    def flops(self) -> int:
        """Score and value products over the (query, key) pairs attended (causal: j <= i)."""
        pairs = self.S * (self.S + 1) // 2 if self.causal else self.S * self.S
        return 4 * pairs * self.head_dim * self.hq

    def qkv(self) -> np.ndarray:
        """The gathered QKV rows [S, row] bf16: N(0, 1) queries, keys and values."""
        return inputs.draw(self.config, inputs.X_ID, (self.S, self.row), _N01, "bf16")


# Llama-3.1-70B attention (64 query heads, 8 key/value heads, head_dim 128) under Ulysses
# parallelism over 8 ranks: 8 query heads and 1 key/value head per rank, causal, 8K tokens
L70B_ATTN = AttnCase(6, 8, 8192, 8, 1, name="Llama-3.1-70B attention, Ulysses 8 rank share, seq 8192")

# the same share at 2K to 16K tokens: the attention gain against sequence length
SWEEP_ATTN = tuple(AttnCase(6, 8, S, 8, 1, name=f"Llama-3.1-70B attention, Ulysses 8 rank share, seq {S}")
                   for S in (2048, 4096, 8192, 16384))
