"""Host checks of the GEMM's dispatch order (fo_tile_order runs the kernels' own mapping code on
the host): every workgroup gets a distinct tile inside the grid, every tile is covered, row
groups are whole tile rows, and the order is the schedule: Flash-AG's local slice first and whole,
Flash-RS's own chunk last and whole, the other slices group by group across slices."""
from __future__ import annotations

import itertools

import pytest

from comm_overlapped_sliced_amd import flashovl as fo

SHAPES = [  # (P, m, K, N)
    (8, 512, 8192, 7168), (8, 512, 3584, 8192), (8, 1024, 6656, 16384), (8, 128, 8192, 7168),
    (4, 200, 520, 392), (3, 256, 576, 512), (2, 37, 72, 136), (1, 300, 64, 1000), (5, 1000, 64, 96),
]
TILES = [fo.TILE_AUTO, fo.TILE_256x256, fo.TILE_256x128, fo.TILE_128x256, fo.TILE_128x128,
         fo.TILE_64x64]


def _grid(kind, P, m, K, N, tile):
    out_dt = fo.F32 if kind == "rs" else fo.BF16
    bm, bn, wg = fo.tile_info(P, m, K, N, fo.BF16, tile, out_dt=out_dt)
    return (m + bm - 1) // bm, (N + bn - 1) // bn, wg


@pytest.mark.parametrize("kind", ["ag", "rs"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "P%d_m%d_N%d" % (s[0], s[1], s[3]))
def test_every_tile_once(kind, shape):
    P, m, K, N = shape
    for tile, groups in itertools.product(TILES, [0, 1, 2, 3, 8]):
        tm_n, tn_n, wg = _grid(kind, P, m, K, N, tile)
        order = fo.tile_order(kind, P, m, K, N, o=fo.opts(tile=tile, row_groups=groups),
                              out_dt=fo.F32 if kind == "rs" else fo.BF16)
        assert len(order) == wg == P * tm_n * tn_n
        seen = {(p, tm, tn) for p, _, tm, tn in order}
        assert len(seen) == wg, "a tile is computed twice"
        assert all(0 <= p < P and 0 <= tm < tm_n and 0 <= tn < tn_n for p, tm, tn in seen)


@pytest.mark.parametrize("kind", ["ag", "rs"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "P%d_m%d_N%d" % (s[0], s[1], s[3]))
def test_groups_and_layout(kind, shape):
    P, m, K, N = shape
    for tile, req in itertools.product(TILES, [0, 1, 2, 3, 8]):
        tm_n, tn_n, _ = _grid(kind, P, m, K, N, tile)
        G = min(tm_n if req == 0 else req, 8, tm_n)
        gr = -(-tm_n // G)
        order = fo.tile_order(kind, P, m, K, N, o=fo.opts(tile=tile, row_groups=req),
                              out_dt=fo.F32 if kind == "rs" else fo.BF16)
        assert all(g == tm // gr for _, g, tm, _ in order), "group is not its tile row's group"
        T = tm_n * tn_n
        lead = 1 if kind == "ag" else 0
        trail = 1 if kind == "rs" else 0
        head, mid, tail = order[:lead * T], order[lead * T:(P - trail) * T], order[(P - trail) * T:]
        assert all(p == 0 for p, *_ in head), "AG: the local slice is not first and whole"
        assert all(p == P - 1 for p, *_ in tail), "RS: the own chunk is not last and whole"
        keys = [(g, p) for p, g, _, _ in mid]
        assert keys == sorted(keys), "the middle positions are not dispatched group by group"
        if req == 1:  # one group: the page's slice-by-slice order
            assert [p for p, *_ in order] == sorted(p for p, *_ in order)


@pytest.mark.parametrize("kind", ["ag", "rs"])
def test_natural_order_is_group_major_over_every_slice(kind):
    order = fo.tile_order(kind, 4, 512, 256, 512, o=fo.opts(order=fo.ORDER_NATURAL, row_groups=2,
                                                            tile=fo.TILE_128x256),
                          out_dt=fo.F32 if kind == "rs" else fo.BF16)
    keys = [(g, p) for p, g, _, _ in order]
    assert keys == sorted(keys)
    assert {p for p, *_ in order[:len(order) // 2]} == {0, 1, 2, 3}  # no slice is held back


@pytest.mark.parametrize("chunks,groups", [(2, 0), (4, 0), (4, 8), (8, 0), (8, 2), (3, 0)])
def test_k_chunks_cap_the_row_groups(chunks, groups):
    """K-chunk-major Flash-AG: each row group of a received slice travels as `chunks` transfers,
    so the row groups per slice are capped at FO_MAX_GROUPS / chunks (8 arrival units)."""
    P, m, K, N = 8, 1024, 16384, 13312
    order = fo.tile_order("ag", P, m, K, N, o=fo.opts(tile=fo.TILE_128x256, row_groups=groups,
                                                      k_chunks=chunks))
    G = len({g for _, g, _, _ in order})
    want = min(8 if groups == 0 else groups, 8 // chunks)
    assert G == want and G * chunks <= 8
    assert len({(p, tm, tn) for p, _, tm, tn in order}) == P * 8 * 52


def test_rejects():
    lib = fo.load()
    import ctypes
    cnt = ctypes.c_int64()
    B = fo.BF16
    assert lib.fo_tile_order(2, 4, 64, 64, 64, B, B, None, None, 0, ctypes.byref(cnt)) == \
        fo.FO_ERR_INVALID_ARG
    assert lib.fo_tile_order(0, 4, 64, 64, 64, B, B, None, None, 5, ctypes.byref(cnt)) == \
        fo.FO_ERR_INVALID_ARG
    assert lib.fo_tile_order(0, 4, 64, 64, 64, B, 7, None, None, 0, ctypes.byref(cnt)) == \
        fo.FO_ERR_INVALID_ARG
    o = fo.opts(row_groups=9)
    assert lib.fo_tile_order(0, 4, 64, 64, 64, B, B, ctypes.byref(o), None, 0,
                             ctypes.byref(cnt)) == fo.FO_ERR_INVALID_ARG
