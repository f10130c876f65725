"""CPU checks of the full-size parity machinery used by the GPU tests: the oracle's rows and
columns computed as smaller problems equal the same rows and columns of the full oracle output
(every output entry of Flash-AG and Flash-RS depends only on its row of X, its column of W and,
for the own chunk, its entries of the partials), and the per-element check passes a correctly
rounded output and names the tile of a planted wrong entry."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from comm_overlapped_sliced_amd import configs
from tests.gpu_helpers import ag_oracle_blocks, assert_parity, rs_oracle, tile_cols, tile_rows

AG = configs.scaled(configs.L70B_AG, config=90, P=4, M=4 * 96, K=256, N=160,
                    name="small AG for the parity helpers")
RS = configs.scaled(configs.L70B_RS, config=91, P=4, M=4 * 96, K=192, N=136,
                    name="small RS for the parity helpers")


def test_tile_rows_cover_every_tile_row():
    rows = tile_rows(8 * 100, 100, 32, seed=1)
    for b0 in range(0, 800, 100):
        for t0 in range(b0, b0 + 100, 32):
            t1 = min(b0 + 100, t0 + 32)
            inside = rows[(rows >= t0) & (rows < t1)]
            assert t0 in inside and t1 - 1 in inside and len(inside) >= 2
    cols = tile_cols(136, 64, seed=2)
    assert {0, 63, 64, 127, 128, 135} <= set(cols.tolist())


@pytest.mark.parametrize("rank", [0, 3])
def test_ag_blocks_equal_full_oracle(rank):
    full = oracle.ag([AG.x()[s * AG.m:(s + 1) * AG.m] for s in range(AG.P)], AG.w(), AG.P, rank)
    blocks = ag_oracle_blocks(AG, rank, full_max=0)
    assert len(blocks) == 2
    for rows, cols, ref in blocks:
        want = full if rows is None else full[rows]
        want = want if cols is None else want[:, cols]
        assert np.array_equal(ref, want)


@pytest.mark.parametrize("rank", [0, 2])
def test_rs_blocks_equal_full_oracle(rank):
    parts = [RS.partial(q) for q in range(RS.P)]
    out, send = oracle.rs(RS.x(), RS.w(), parts, RS.P, rank, want_send=True)
    m = RS.m
    blocks = rs_oracle(RS, rank, full_max=0)
    assert len(blocks) == 2
    for rows, cols, ref_out, ref_send in blocks:
        sel = lambda a: (a if rows is None else a[rows])[:, slice(None) if cols is None else cols]
        assert np.array_equal(ref_out, sel(out))
        n = m if rows is None else len(rows)
        for d in range(RS.P):
            got = ref_send[d * n:(d + 1) * n]
            if d == rank:
                assert np.isnan(got).all()
            else:
                assert np.array_equal(got, sel(send[d * m:(d + 1) * m]))


def _round_bf16(a):
    return oracle.round_bf16(a).astype(np.uint32) << 16


def test_assert_parity_accepts_rounded_and_names_a_wrong_tile():
    rng = np.random.default_rng(5)
    ref = rng.normal(0.0, 1.3, (96, 160))
    got = (_round_bf16(ref)).view(np.float32).astype(np.float64)
    assert_parity(got, ref, "bf16", (32, 64), what="rounded")
    bad = got.copy()
    bad[40, 130] += 0.05  # one entry of tile (1, 2) off by ~4% of rms
    with pytest.raises(AssertionError, match=r"tile \(1, 2\)"):
        assert_parity(bad, ref, "bf16", (32, 64), what="planted")
    f32 = ref.astype(np.float32).astype(np.float64)
    assert_parity(f32, ref, "f32", (32, 64), what="fp32")
    f32[95, 0] = np.nan
    with pytest.raises(AssertionError, match=r"\(95, 0\) tile \(2, 0\)"):
        assert_parity(f32, ref, "f32", (32, 64), what="nan")
