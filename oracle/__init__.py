"""CPU oracle for the Flash-Overlap hot path (fp64, plain C behind ctypes).

TEST INFRASTRUCTURE ONLY: only the tests, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this package. It shares no code with the HIP library and does
not import it.

What it computes follows the FlashOverlap page (gist.science paper 2604.24013), technical
summary section 2 "Methodology": Flash-AG (All-Gather then GEMM, local slice first, ring
arrivals after) and Flash-RS (GEMM then Reduce-Scatter, own chunk last, incoming partials added
into it). Section 3 calls the algorithm exact, so every result is the plain fp64 definition.

Operands are numpy arrays: bf16 as ``uint16`` bit patterns, fp32 as ``float32``. Results are
fp64 numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

BF16 = 0
F32 = 1

def build(force: bool = True, src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc (OpenMP, fp64, no FMA contraction)."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-Wall", "-shared", "-fPIC",
               src, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return out


def _dt(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return F32
    raise TypeError(f"oracle operands are uint16 (bf16 bits) or float32, got {a.dtype}")


def _c(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a)


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _ptr_array(arrs):
    a = (ctypes.c_void_p * len(arrs))()
    for i, x in enumerate(arrs):
        a[i] = None if x is None else _ptr(x)
    return a


def _idx(rows, cols):
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape or rows.ndim != 1:
        raise ValueError("rows and cols are equal-length 1-D index arrays")
    return rows, cols


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


class Oracle:
    """ctypes view of one build of oracle.c (the default build, or another for self-checks)."""

    def __init__(self, path: str = _LIB):
        if path == _LIB and not os.path.exists(path):
            build()
        lib = ctypes.CDLL(path)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        ip = ctypes.POINTER(ctypes.c_int)
        lib.oracle_ag_order.argtypes = [i32, i32, ip]
        lib.oracle_rs_order.argtypes = [i32, i32, ip]
        lib.oracle_gemm.argtypes = [vp, i32, vp, i32, vp, i64, i64, i64]
        lib.oracle_ag.argtypes = [vp, i32, vp, i32, vp, i32, i32, vp, i64, i64, i64]
        lib.oracle_rs.argtypes = [vp, i32, vp, i32, vp, vp, vp, i32, i32, i64, i64, i64]
        lib.oracle_ag_sampled.argtypes = [vp, i32, vp, i32, i32, i64, i64, i64, vp, vp, i64, vp]
        lib.oracle_rs_sampled.argtypes = [vp, i32, vp, i32, vp, i32, i32, i64, i64, i64, vp, vp,
                                          i64, vp]
        lib.oracle_rs_send_sampled.argtypes = [vp, i32, vp, i32, i32, i64, i64, i64, vp, vp, i64,
                                               vp]
        lib.oracle_num_threads.argtypes = []
        lib.oracle_swiglu.argtypes = [vp, i64, i64, vp]
        lib.oracle_swiglu_f64.argtypes = [vp, i64, i64, vp]
        lib.oracle_attn.argtypes = [vp, i64, i32, i32, i32, i32, vp, i64, vp]
        lib.oracle_round_bf16.argtypes = [vp, i64, vp]
        for f in (lib.oracle_ag_order, lib.oracle_rs_order, lib.oracle_gemm, lib.oracle_ag,
                  lib.oracle_rs, lib.oracle_ag_sampled, lib.oracle_rs_sampled,
                  lib.oracle_rs_send_sampled, lib.oracle_num_threads, lib.oracle_swiglu,
                  lib.oracle_swiglu_f64, lib.oracle_round_bf16, lib.oracle_attn):
            f.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    def ag_order(self, P: int, r: int) -> list:
        out = (ctypes.c_int * P)()
        _check(self.lib.oracle_ag_order(P, r, out), "ag_order")
        return list(out)

    def rs_order(self, P: int, r: int) -> list:
        out = (ctypes.c_int * P)()
        _check(self.lib.oracle_rs_order(P, r, out), "rs_order")
        return list(out)

    def gemm(self, A: np.ndarray, B: np.ndarray) -> np.ndarray:
        """C = A . B in fp64 (A [M,K], B [K,N])."""
        A, B = _c(A), _c(B)
        M, K = A.shape
        K2, N = B.shape
        if K != K2:
            raise ValueError("inner dimensions differ")
        C = np.empty((M, N), dtype=np.float64)
        _check(self.lib.oracle_gemm(_ptr(A), _dt(A), _ptr(B), _dt(B), _ptr(C), M, K, N), "gemm")
        return C

    def ag(self, x_slices, W: np.ndarray, P: int, r: int, order=None) -> np.ndarray:
        """Flash-AG output Y [P*m, N] of rank r; x_slices[s] is slice s ([m, K])."""
        xs = [_c(x) for x in x_slices]
        if len(xs) != P:
            raise ValueError("need one slice per rank")
        W = _c(W)
        m, K = xs[0].shape
        N = W.shape[1]
        dts = {_dt(x) for x in xs}
        if len(dts) != 1 or any(x.shape != (m, K) for x in xs):
            raise ValueError("slices must share shape and dtype")
        Y = np.empty((P * m, N), dtype=np.float64)
        ordp = None if order is None else (ctypes.c_int * P)(*order)
        rc = self.lib.oracle_ag(_ptr_array(xs), dts.pop(), _ptr(W), _dt(W), _ptr(Y), P, r,
                                ctypes.cast(ordp, ctypes.c_void_p) if ordp is not None else None,
                                m, K, N)
        _check(rc, "ag")
        return Y

    def rs(self, x_shard: np.ndarray, W: np.ndarray, partials, P: int, r: int,
           want_send: bool = False):
        """Flash-RS of rank r: out [m, N] (and the send chunks [P*m, N], NaN in chunk r).

        partials[q] is peer q's fp32 [m, N] partial for chunk r (partials[r] is ignored)."""
        x_shard, W = _c(x_shard), _c(W)
        M, K = x_shard.shape
        N = W.shape[1]
        if M % P:
            raise ValueError("rows of x_shard must split into P chunks")
        m = M // P
        ps = []
        for q in range(P):
            if q == r:
                ps.append(None)
                continue
            p = _c(partials[q])
            if p.dtype != np.float32 or p.shape != (m, N):
                raise ValueError("partials are float32 [m, N]")
            ps.append(p)
        out = np.empty((m, N), dtype=np.float64)
        send = np.full((M, N), np.nan, dtype=np.float64) if want_send else None
        rc = self.lib.oracle_rs(_ptr(x_shard), _dt(x_shard), _ptr(W), _dt(W), _ptr_array(ps),
                                _ptr(out), _ptr(send) if send is not None else None, P, r, m, K,
                                N)
        _check(rc, "rs")
        return (out, send) if want_send else out

    def ag_sampled(self, x_slices, W: np.ndarray, rows, cols) -> np.ndarray:
        """Entries Y[rows[t], cols[t]] of the Flash-AG output (the same for every rank)."""
        xs = [_c(x) for x in x_slices]
        W = _c(W)
        P = len(xs)
        m, K = xs[0].shape
        N = W.shape[1]
        rows, cols = _idx(rows, cols)
        out = np.empty(rows.shape[0], dtype=np.float64)
        rc = self.lib.oracle_ag_sampled(_ptr_array(xs), _dt(xs[0]), _ptr(W), _dt(W), P, m, K, N,
                                        _ptr(rows), _ptr(cols), rows.shape[0], _ptr(out))
        _check(rc, "ag_sampled")
        return out

    def rs_sampled(self, x_shard, W, partials, P: int, r: int, rows, cols) -> np.ndarray:
        """Entries out[rows[t], cols[t]] of rank r's Flash-RS own chunk."""
        x_shard, W = _c(x_shard), _c(W)
        M, K = x_shard.shape
        N = W.shape[1]
        m = M // P
        ps = [None if q == r else _c(partials[q]) for q in range(P)]
        rows, cols = _idx(rows, cols)
        out = np.empty(rows.shape[0], dtype=np.float64)
        rc = self.lib.oracle_rs_sampled(_ptr(x_shard), _dt(x_shard), _ptr(W), _dt(W),
                                        _ptr_array(ps), P, r, m, K, N, _ptr(rows), _ptr(cols),
                                        rows.shape[0], _ptr(out))
        _check(rc, "rs_sampled")
        return out

    def rs_send_sampled(self, x_shard, W, P: int, d: int, rows, cols) -> np.ndarray:
        """Entries of send chunk d (rows index the [m, N] chunk)."""
        x_shard, W = _c(x_shard), _c(W)
        M, K = x_shard.shape
        N = W.shape[1]
        m = M // P
        rows, cols = _idx(rows, cols)
        out = np.empty(rows.shape[0], dtype=np.float64)
        rc = self.lib.oracle_rs_send_sampled(_ptr(x_shard), _dt(x_shard), _ptr(W), _dt(W), d, m,
                                             K, N, _ptr(rows), _ptr(cols), rows.shape[0],
                                             _ptr(out))
        _check(rc, "rs_send_sampled")
        return out

    # ---- the MLP block ------------------------------------------------------------------

    def swiglu(self, y: np.ndarray) -> np.ndarray:
        """h = silu(y[:, :inter]) * y[:, inter:] in fp64; y bf16 bits (uint16) or fp64
        [rows, 2*inter]."""
        y = _c(y)
        if y.dtype not in (np.uint16, np.float64) or y.ndim != 2 or y.shape[1] % 2:
            raise ValueError("y is bf16 bits or fp64 [rows, 2*inter]")
        rows, inter = y.shape[0], y.shape[1] // 2
        h = np.empty((rows, inter), dtype=np.float64)
        fn = self.lib.oracle_swiglu if y.dtype == np.uint16 else self.lib.oracle_swiglu_f64
        _check(fn(_ptr(y), rows, inter, _ptr(h)), "swiglu")
        return h

    def attn(self, qkv: np.ndarray, hq: int, hkv: int, causal: bool = True, rows=None,
             d: int = 128) -> np.ndarray:
        """Scaled dot-product attention in fp64 of one sequence: qkv bf16 bits [S, (hq+2hkv)*d]
        (token row = [query heads | key heads | value heads]); returns [len(rows) or S, hq*d] for
        the query positions `rows` (default all)."""
        qkv = _c(qkv)
        if qkv.dtype != np.uint16 or qkv.ndim != 2 or qkv.shape[1] != (hq + 2 * hkv) * d:
            raise ValueError("qkv is bf16 bits [S, (hq + 2 hkv) * d]")
        S = qkv.shape[0]
        r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
        n = S if r is None else len(r)
        out = np.empty((n, hq * d), dtype=np.float64)
        _check(self.lib.oracle_attn(_ptr(qkv), S, hq, hkv, d, int(causal),
                                    None if r is None else _ptr(r), n, _ptr(out)), "attn")
        return out

    def round_bf16(self, x: np.ndarray) -> np.ndarray:
        """x (fp64) rounded to the nearest bf16, ties to even, as bf16 bits (same shape)."""
        x = np.ascontiguousarray(x, dtype=np.float64)
        out = np.empty(x.shape, dtype=np.uint16)
        _check(self.lib.oracle_round_bf16(_ptr(x), x.size, _ptr(out)), "round_bf16")
        return out

    def mlp_block(self, x_slices, w_gu: np.ndarray, w_down: np.ndarray, partials, P: int,
                  r: int, fused: bool = False) -> np.ndarray:
        """Rank r's output of the MLP block: Y = Flash-AG(x_slices, w_gu) rounded to bf16,
        H = swiglu(Y) rounded to bf16, then Flash-RS(H, w_down, partials) (fp64 [m, N]).
        fused: the activation reads Y before any rounding (H is still rounded to bf16)."""
        y = self.ag(x_slices, w_gu, P, r)
        if not fused:
            y = self.round_bf16(y)
        h = self.round_bf16(self.swiglu(y))
        return self.rs(h, w_down, partials, P, r)


_default = None


def default() -> Oracle:
    """The oracle built from oracle.c in this directory."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def __getattr__(name):
    # module-level shortcuts: oracle.gemm(...), oracle.ag(...), ...
    if name in ("num_threads", "ag_order", "rs_order", "gemm", "ag", "rs", "ag_sampled",
                "rs_sampled", "rs_send_sampled", "swiglu", "round_bf16", "mlp_block", "attn"):
        return getattr(default(), name)
    raise AttributeError(name)
