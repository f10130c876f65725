"""Pins of the CPU oracle against what the FlashOverlap page and plain mathematics fix.

Each pin takes an ``oracle.Oracle`` so that the same checks can be run on deliberately broken
builds of the oracle (see test_oracle.py) to show that they catch the mistakes they target.
Nothing here calls the HIP library.

What the page fixes (FlashOverlap, gist.science paper 2604.24013, technical summary):
  * section 2, Flash-AG: the slice already on the rank is computed first; ring transfers bring
    the others.
  * section 2, Flash-RS: the chunk that stays on the rank is computed last.
  * section 2, architectural instantiations: column-parallel (All-Gather then GEMM) and
    row-parallel (GEMM then Reduce-Scatter) projections.
  * section 3: the algorithm is exact, so slicing never changes the result.
The pins below are closed forms, invariants and brute force derived from those statements.
"""
from __future__ import annotations

import itertools
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
if os.path.dirname(HERE) not in sys.path:
    sys.path.insert(0, os.path.dirname(HERE))

from comm_overlapped_sliced_amd import inputs  # noqa: E402


def _ints(rng, shape, lo=-3, hi=3):
    return rng.integers(lo, hi + 1, size=shape).astype(np.float32)


def _brute(A, B):
    """Pure-Python integer product (exact)."""
    A = [[int(v) for v in row] for row in np.asarray(A, dtype=np.float64)]
    B = [[int(v) for v in row] for row in np.asarray(B, dtype=np.float64)]
    M, K, N = len(A), len(B), len(B[0])
    return np.array([[sum(A[i][k] * B[k][j] for k in range(K)) for j in range(N)]
                     for i in range(M)], dtype=np.float64)


# ---- slice orders (section 2: local slice first for AG, own chunk last for RS) -------------

def pin_ag_order(orc):
    for P in range(1, 17):
        for r in range(P):
            o = orc.ag_order(P, r)
            assert o[0] == r, "Flash-AG computes the local slice first"
            assert sorted(o) == list(range(P)), "every slice exactly once"
            # ring from rank r-1: at step t the slice of rank r-t arrives
            assert o == [(r - t) % P for t in range(P)]


def pin_rs_order(orc):
    for P in range(1, 17):
        for r in range(P):
            o = orc.rs_order(P, r)
            assert o[-1] == r, "Flash-RS computes the chunk that stays on the rank last"
            assert sorted(o) == list(range(P))
        # at every step before the last, the ranks target pairwise distinct peers (no incast)
        for i in range(P - 1):
            targets = [orc.rs_order(P, r)[i] for r in range(P)]
            assert sorted(targets) == list(range(P))
            assert all(t != r for r, t in enumerate(targets)), "a step never targets itself"


# ---- the GEMM core ------------------------------------------------------------------------

def pin_gemm_bruteforce(orc):
    rng = np.random.default_rng(11)
    for (M, K, N) in [(1, 1, 1), (3, 5, 2), (7, 13, 6), (9, 4, 11), (16, 17, 5)]:
        A = _ints(rng, (M, K))
        B = _ints(rng, (K, N))
        ref = _brute(A, B)
        assert np.array_equal(orc.gemm(A, B), ref)
        # the same integers as bf16 operands (all of -3..3 are exact in bf16)
        Ab, Bb = inputs.f32_to_bf16_bits(A), inputs.f32_to_bf16_bits(B)
        assert np.array_equal(orc.gemm(Ab, Bb), ref)
        assert np.array_equal(orc.gemm(Ab, B), ref)


def pin_gemm_wide_integers(orc):
    """Larger integer magnitudes, still exact in fp64: any dropped/duplicated term shows."""
    rng = np.random.default_rng(12)
    A = rng.integers(-1000, 1001, size=(12, 37)).astype(np.float32)
    B = rng.integers(-1000, 1001, size=(37, 9)).astype(np.float32)
    assert np.array_equal(orc.gemm(A, B), _brute(A, B))


def pin_gemm_matches_numpy_f64(orc):
    """Non-integer operands: numpy's fp64 product (a library routine) agrees to rounding."""
    rng = np.random.default_rng(13)
    A = rng.standard_normal((48, 96)).astype(np.float32)
    B = rng.standard_normal((96, 40)).astype(np.float32)
    ref = A.astype(np.float64) @ B.astype(np.float64)
    got = orc.gemm(A, B)
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))
    # bf16 decoding of non-integer values: widen exactly, then compare the same way
    Ab = inputs.normal(99, (20, 64), 1.0, "bf16")
    Bb = inputs.normal(98, (64, 24), 0.02, "bf16")
    ref = inputs.bf16_bits_to_f32(Ab).astype(np.float64) @ inputs.bf16_bits_to_f32(Bb).astype(
        np.float64)
    got = orc.gemm(Ab, Bb)
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))


def pin_gemm_special_weights(orc):
    rng = np.random.default_rng(14)
    X = rng.standard_normal((10, 12)).astype(np.float32)
    eye = np.eye(12, dtype=np.float32)
    assert np.array_equal(orc.gemm(X, eye), X.astype(np.float64)), "W = I gives Y = X"
    perm = rng.permutation(12)
    Pm = np.zeros((12, 12), dtype=np.float32)
    Pm[perm, np.arange(12)] = 1.0  # column j of X.P is column perm[j] of X
    assert np.array_equal(orc.gemm(X, Pm), X[:, perm].astype(np.float64))


# ---- Flash-AG: slicing never changes the result --------------------------------------------

def pin_ag_any_order_is_monolithic(orc):
    rng = np.random.default_rng(21)
    P, m, K, N = 4, 3, 7, 5
    X = rng.standard_normal((P * m, K)).astype(np.float32)
    W = rng.standard_normal((K, N)).astype(np.float32)
    slices = [X[s * m:(s + 1) * m].copy() for s in range(P)]
    mono = orc.gemm(X, W)
    for order in itertools.permutations(range(P)):
        for r in range(P):
            assert np.array_equal(orc.ag(slices, W, P, r, order=list(order)), mono)
    P = 8
    X = rng.standard_normal((P * m, K)).astype(np.float32)
    slices = [X[s * m:(s + 1) * m] for s in range(P)]
    mono = orc.gemm(X, W)
    for r in range(P):
        assert np.array_equal(orc.ag(slices, W, P, r), mono)
        assert np.array_equal(orc.ag(slices, W, P, r, order=list(rng.permutation(P))), mono)


def pin_ag_column_parallel(orc):
    """P ranks, each with its own column shard W^(r): concatenating their outputs along N gives
    X_full . W_full (the column-parallel projection)."""
    rng = np.random.default_rng(22)
    P, m, K, n = 4, 2, 6, 3
    X = _ints(rng, (P * m, K))
    Wfull = _ints(rng, (K, P * n))
    slices = [X[s * m:(s + 1) * m] for s in range(P)]
    parts = [orc.ag(slices, Wfull[:, r * n:(r + 1) * n].copy(), P, r) for r in range(P)]
    assert np.array_equal(np.concatenate(parts, axis=1), _brute(X, Wfull))


def pin_ag_slices_land_in_place(orc):
    """Slice s must produce rows s*m.. of Y, whichever position it has in the order."""
    P, m, K, N = 4, 2, 3, 2
    slices = [np.full((m, K), float(s + 1), dtype=np.float32) for s in range(P)]
    W = np.ones((K, N), dtype=np.float32)
    for r in range(P):
        Y = orc.ag(slices, W, P, r)
        for s in range(P):
            assert np.all(Y[s * m:(s + 1) * m] == 3.0 * (s + 1))


# ---- Flash-RS: the reduce-scatter closed form ------------------------------------------------

def pin_rs_closed_form(orc):
    """P ranks each hold X^(q) [M, K_q] and W^(q) [K_q, N] (row-parallel). Rank r's output,
    fed the true partials of the other ranks, equals rows r*m.. of X_full . W_full."""
    rng = np.random.default_rng(31)
    for P, m, kq, N in [(4, 3, 5, 6), (3, 2, 4, 7), (8, 1, 2, 3)]:
        M = P * m
        Xq = [_ints(rng, (M, kq)) for _ in range(P)]
        Wq = [_ints(rng, (kq, N)) for _ in range(P)]
        full = _brute(np.concatenate(Xq, axis=1), np.concatenate(Wq, axis=0))
        dummy = [np.zeros((m, N), np.float32) for _ in range(P)]
        sends = [orc.rs(Xq[q], Wq[q], dummy, P, q, want_send=True)[1] for q in range(P)]
        for r in range(P):
            partials = [None if q == r else sends[q][r * m:(r + 1) * m].astype(np.float32)
                        for q in range(P)]
            out = orc.rs(Xq[r], Wq[r], partials, P, r)
            assert np.array_equal(out, full[r * m:(r + 1) * m])


def pin_rs_adds_every_peer_once(orc):
    """With X = 0 the own chunk is the sum of the incoming partials; powers of two make every
    dropped, doubled, negated or misplaced term visible."""
    P, m, K, N = 5, 2, 3, 4
    X = np.zeros((P * m, K), np.float32)
    W = np.ones((K, N), np.float32)
    for r in range(P):
        partials = [np.full((m, N), float(2 ** q), np.float32) for q in range(P)]
        out = orc.rs(X, W, partials, P, r)
        assert np.all(out == float(sum(2 ** q for q in range(P) if q != r)))


def pin_rs_send_chunks(orc):
    """Chunk d != r of the send buffer is rows d*m.. of X_shard . W; the own chunk is not sent."""
    rng = np.random.default_rng(32)
    P, m, K, N = 4, 3, 5, 2
    X = _ints(rng, (P * m, K))
    W = _ints(rng, (K, N))
    full = _brute(X, W)
    partials = [_ints(rng, (m, N)) for _ in range(P)]
    for r in range(P):
        out, send = orc.rs(X, W, partials, P, r, want_send=True)
        for d in range(P):
            blk = send[d * m:(d + 1) * m]
            if d == r:
                assert np.all(np.isnan(blk))
            else:
                assert np.array_equal(blk, full[d * m:(d + 1) * m])
        expect = full[r * m:(r + 1) * m] + sum(partials[q].astype(np.float64)
                                               for q in range(P) if q != r)
        assert np.array_equal(out, expect)


def pin_single_rank(orc):
    """P = 1: both calls reduce to a plain GEMM with nothing to receive."""
    rng = np.random.default_rng(33)
    X = _ints(rng, (4, 6))
    W = _ints(rng, (6, 3))
    ref = _brute(X, W)
    assert np.array_equal(orc.ag([X], W, 1, 0), ref)
    assert np.array_equal(orc.rs(X, W, [None], 1, 0), ref)


# ---- sampled entries agree with the full oracle ----------------------------------------------

def pin_sampled_entries(orc):
    P, m, K, N = 4, 5, 33, 7
    X = inputs.normal(41, (P * m, K), 1.0, "bf16")
    W = inputs.normal(42, (K, N), 0.02, "bf16")
    slices = [X[s * m:(s + 1) * m].copy() for s in range(P)]  # separate buffers
    rng = np.random.default_rng(43)
    rows = rng.integers(0, P * m, 50)
    cols = rng.integers(0, N, 50)
    full = orc.ag(slices, W, P, 2)
    assert np.array_equal(orc.ag_sampled(slices, W, rows, cols), full[rows, cols])
    partials = [inputs.normal(50 + q, (m, N), 1.0, "f32") for q in range(P)]
    out, send = orc.rs(X, W, partials, P, 1, want_send=True)
    r2, c2 = rng.integers(0, m, 30), rng.integers(0, N, 30)
    assert np.array_equal(orc.rs_sampled(X, W, partials, P, 1, r2, c2), out[r2, c2])
    for d in (0, 2, 3):
        got = orc.rs_send_sampled(X, W, P, d, r2, c2)
        assert np.array_equal(got, send[d * m + r2, c2])


# ---- a worked example computed by hand ------------------------------------------------------

def _read_golden(name):
    vals = {}
    with open(os.path.join(HERE, "golden", name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, rest = line.split("=", 1)
            rows = [[float(v) for v in r.split()] for r in rest.split(";")]
            vals[key.strip()] = np.array(rows, dtype=np.float32)
    return vals


def pin_hand_worked_example(orc):
    g = _read_golden("hand_worked_p2.txt")
    slices = [g["X0"], g["X1"]]
    for r in (0, 1):
        assert np.array_equal(orc.ag(slices, g["W"], 2, r), np.concatenate([g["Y0"], g["Y1"]]))
    xs = np.concatenate([g["X0"], g["X1"]])
    out, send = orc.rs(xs, g["W"], [None, g["PART_FROM_1"]], 2, 0, want_send=True)
    assert np.array_equal(out, g["OUT_RANK0"])
    assert np.array_equal(send[1:2], g["SEND_TO_1"])


ALL_PINS = [
    pin_ag_order, pin_rs_order, pin_gemm_bruteforce, pin_gemm_wide_integers,
    pin_gemm_matches_numpy_f64, pin_gemm_special_weights, pin_ag_any_order_is_monolithic,
    pin_ag_column_parallel, pin_ag_slices_land_in_place, pin_rs_closed_form,
    pin_rs_adds_every_peer_once, pin_rs_send_chunks, pin_single_rank, pin_sampled_entries,
    pin_hand_worked_example,
]


def run_all(orc) -> None:
    for pin in ALL_PINS:
        pin(orc)


if __name__ == "__main__":
    # used by the mutation check: `python tests/oracle_pins.py <liboracle path>`; exit 1 on a
    # failed pin
    import oracle as _o
    try:
        run_all(_o.Oracle(sys.argv[1]))
    except (AssertionError, ValueError) as e:
        print("PIN FAILED:", type(e).__name__, e)
        sys.exit(1)
    print("all pins hold")
