"""Shared helpers of the GPU tests: moving seeded numpy operands to the device and back, and the
relative Frobenius error used as the parity measure."""
from __future__ import annotations

import numpy as np

import oracle
from comm_overlapped_sliced_amd import flashovl as fo, inputs

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


# Per-element bounds of the full-size parity checks, on top of the relative Frobenius error:
#   bf16 output: |got - ref| <= 2^-8 |ref| + 2^-12 rms(ref). Rounding an fp32 value to the nearest
#     bf16 moves it by at most half a bf16 ulp, 2^-8 of its magnitude; fp32 accumulation over
#     K <= 16384 adds a few 1e-6 of rms(ref) (about sqrt(K/16) roundings of 2^-24).
#   fp32 output: |got - ref| <= 2^-14 (|ref| + rms(ref)): only fp32 accumulation and, for the own
#     chunk of Flash-RS, P-1 fp32 adds of the partials (a few 1e-7 of rms(ref)).
# A wrong tile, a dropped partial or a misplaced slice moves entries by about rms(ref), thousands
# of times these bounds, and the failure names the entry and its tile.
BOUND_BF16 = (2.0 ** -8, 2.0 ** -12)
BOUND_F32 = (2.0 ** -14, 2.0 ** -14)


def assert_parity(got, ref, out="bf16", tile=None, rows=None, cols=None, tol=TOL_BF16, what="",
                  bound=None):
    """got and ref are 2-D (fp64); rows/cols map their row/column indices back to the output
    matrix (for sub-blocks of full rows or columns). Checks relF <= tol over the whole block
    and the per-element bound for the output dtype (or bound = (rel, abs): |got - ref| <=
    rel |ref| + abs rms(ref)); on failure names the worst entry and the tile (row // bm,
    col // bn) that holds it."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} != {ref.shape}"
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    rel, ab = bound or (BOUND_BF16 if out == "bf16" else BOUND_F32)
    lim = rel * np.abs(ref) + ab * rms
    err = np.abs(got - ref)
    bad = ~(err <= lim)  # NaN counts as bad
    e = rel_frobenius(got, ref)
    if bad.any() or not e <= tol:
        if bad.any():
            i, j = np.unravel_index(np.argmax(np.where(np.isnan(err), np.inf, err - lim)), err.shape)
        else:
            i, j = np.unravel_index(np.argmax(err), err.shape)
        r = int(rows[i]) if rows is not None else int(i)
        c = int(cols[j]) if cols is not None else int(j)
        where = f" tile ({r // tile[0]}, {c // tile[1]})" if tile else ""
        raise AssertionError(
            f"{what}: relF {e:.3e} (bound {tol:g}), {int(bad.sum())} of {bad.size} entries past "
            f"the per-element bound; worst at ({r}, {c}){where}: got {got[i, j]!r} ref "
            f"{ref[i, j]!r} limit {lim[i, j]:.3e}")


def tile_rows(rows: int, block: int, bm: int, seed: int) -> np.ndarray:
    """Row indices of a matrix cut into blocks (slices or chunks) of `block` rows, each cut into
    tile rows of bm: the first and the last row of every tile row of every block, and one more
    drawn at random inside it."""
    rng = np.random.default_rng(seed)
    out = []
    for b0 in range(0, rows, block):
        b1 = min(rows, b0 + block)
        for t0 in range(b0, b1, bm):
            t1 = min(b1, t0 + bm)
            out += [t0, t1 - 1, int(rng.integers(t0, t1))]
    return np.unique(np.array(out, dtype=np.int64))


def tile_cols(cols: int, bn: int, seed: int) -> np.ndarray:
    """Column indices: the first and last column of every tile column and one drawn inside it."""
    return tile_rows(cols, cols, bn, seed)


_FULL = {}


def oracle_cached(key, fn, keep: int = 4):
    """fn() (an oracle call), kept for the rest of the session under `key` so that several tests
    of one workload pay for the fp64 product once; at most `keep` results are held."""
    if key not in _FULL:
        while len(_FULL) >= keep:
            _FULL.pop(next(iter(_FULL)))
        _FULL[key] = fn()
    return _FULL[key]


# ---- full-size oracle references of the Flash-AG and Flash-RS workloads --------------------
#
# The 70B shares (and the 1K-8K sweep) are compared entry by entry with the full oracle output.
# For the largest products (16K tokens, 405B) every tile is checked on whole rows (the first,
# the last and one random row of every tile row of every slice, all N columns) and whole
# columns (the first, the last and one random column of every tile column, all rows): the
# oracle computes those rows and columns as a smaller problem of the same definition (each
# output entry depends only on its row of X, its column of W and its partials).

FULL_ORACLE_MAX_FLOP = 1.0e12   # larger products are checked on whole rows and columns


def ag_oracle_blocks(case, rank=0, full_max=None):
    """(row_idx, col_idx, ref) blocks of the Flash-AG output that the oracle checks: the whole
    output, or whole rows and whole columns of every tile. The AG output is the same for every
    rank; the oracle is called once per workload and session."""
    x, w = case.x(), case.w()
    m, P = case.m, case.P
    slices = [x[s * m:(s + 1) * m] for s in range(P)]
    if case.flops <= (FULL_ORACLE_MAX_FLOP if full_max is None else full_max):
        ref = oracle_cached(("ag", case.name, case.M),
                            lambda: oracle.ag(slices, w, P, rank))
        return [(None, None, ref)]
    bm, bn, _ = fo.tile_info(P, m, case.K, case.N)

    def blocks():
        rows = tile_rows(case.M, m, bm, seed=case.M)
        cols = tile_cols(case.N, bn, seed=case.N)
        # whole rows: the rows picked in every slice form a smaller Flash-AG problem when every
        # slice contributes as many (else each slice's rows are a problem of their own)
        sub = [np.ascontiguousarray(x[rows[(rows >= s * m) & (rows < (s + 1) * m)]])
               for s in range(P)]
        if len({len(t) for t in sub}) == 1:
            ref_rows = oracle.ag(sub, w, P, rank)
        else:
            ref_rows = np.concatenate([oracle.ag([t], w, 1, 0) for t in sub])
        ref_cols = oracle.ag(slices, np.ascontiguousarray(w[:, cols]), P, rank)
        return [(rows, None, ref_rows), (None, cols, ref_cols)]

    return oracle_cached(("ag", case.name, case.M), blocks)


def check_ag_blocks(got, blocks, tile, what):
    for rows, cols, ref in blocks:
        g = got
        if rows is not None:
            g = g[rows]
        if cols is not None:
            g = g[:, cols]
        assert_parity(g, ref, "bf16", tile, rows, cols, what=what)


def rs_oracle(case, r, full_max=None):
    """(row_idx, col_idx, out_ref, send_ref) blocks of rank r's Flash-RS results checked against
    the oracle: the own chunk and every send chunk whole, or whole rows and columns of every
    tile. Rows index the [m, N] chunk; send_ref is [P*len(rows), len(cols)] (NaN in chunk r)."""
    x, w = case.x(), case.w()
    P, m = case.P, case.m
    parts = [case.partial(q) for q in range(P)]
    if case.flops <= (FULL_ORACLE_MAX_FLOP if full_max is None else full_max):
        out, send = oracle.rs(x, w, parts, P, r, want_send=True)
        return [(None, None, out, send)]
    bm, bn, _ = fo.tile_info(P, m, case.K, case.N, out_dt=fo.F32)
    rows = tile_rows(m, m, bm, seed=m + r)
    cols = tile_cols(case.N, bn, seed=case.N + r)
    res = []
    # whole rows: the same rows of every chunk, and their partials, form a smaller problem
    xs = np.concatenate([x[d * m + rows] for d in range(P)])
    ps = [None if q == r else np.ascontiguousarray(parts[q][rows]) for q in range(P)]
    out, send = oracle.rs(xs, w, ps, P, r, want_send=True)
    res.append((rows, None, out, send))
    wc = np.ascontiguousarray(w[:, cols])
    ps = [None if q == r else np.ascontiguousarray(parts[q][:, cols]) for q in range(P)]
    out, send = oracle.rs(x, wc, ps, P, r, want_send=True)
    res.append((None, cols, out, send))
    return res


def check_rs(out, send, blocks, case, r, tile):
    P, m = case.P, case.m
    for rows, cols, ref_out, ref_send in blocks:
        sel = lambda a: (a if rows is None else a[rows])[:, slice(None) if cols is None else cols]
        assert_parity(sel(out), ref_out, "f32", tile, rows, cols,
                      what=f"{case.name}: rank {r} own chunk")
        n = m if rows is None else len(rows)
        for d in range(P):
            if d == r:
                continue
            assert_parity(sel(send[d * m:(d + 1) * m]), ref_send[d * n:(d + 1) * n], "f32",
                          tile, rows, cols, what=f"{case.name}: rank {r} send chunk {d}")


