"""CPU checks of the causal attention's work lists (fo_attn_schedule, host logic only): every
(slice, query tile, head) item is computed exactly once, whole or as the two halves of one
pair; only items longer than a workgroup slot's share are cut; each CU's load stays within one
item of the average; the lists are a function of the shape."""
from __future__ import annotations

import collections

import pytest

from comm_overlapped_sliced_amd import flashovl as fo

COST = 4  # the fixed cost the builder counts per item, in key tiles


def _walk_tiles(s, qt, m):
    """Key tiles a causal item walks: the s whole slices before it and its own slice up to the
    tile's last query."""
    q1 = min(m, (qt + 1) * 128)
    return s * ((m + 63) // 64) + (q1 + 63) // 64


SHAPES = [(8, 1024, 8, 256), (1, 8192, 8, 256), (8, 2048, 8, 256), (3, 200, 2, 256),
          (8, 256, 8, 256), (1, 64, 8, 256), (4, 1000, 4, 7), (2, 512, 3, 5), (32, 128, 2, 16)]


@pytest.mark.parametrize("P,m,hq,n_cu", SHAPES)
def test_every_item_once(P, m, hq, n_cu):
    entries, wgs = fo.attn_schedule(P, m, hq, n_cu)
    assert 1 <= wgs <= 2 * n_cu
    qtiles = (m + 127) // 128
    whole = collections.Counter()
    halves = collections.defaultdict(list)
    last_wg = -1
    for wg, s, qt, h, w in entries:
        assert last_wg <= wg < wgs  # each workgroup's entries are contiguous
        last_wg = wg
        assert 0 <= s < P and 0 <= qt < qtiles and 0 <= h < hq
        if w < 0:
            whole[(s, qt, h)] += 1
        else:
            halves[w >> 1].append((w & 1, s, qt, h))
    for k, parts in halves.items():
        assert sorted(p[0] for p in parts) == [0, 1], f"pair {k}"
        assert parts[0][1:] == parts[1][1:], f"pair {k} halves of different items"
    assert sorted(halves) == list(range(len(halves)))
    split = collections.Counter(p[0][1:] for p in halves.values())
    for s in range(P):
        for qt in range(qtiles):
            for h in range(hq):
                assert whole[(s, qt, h)] + split[(s, qt, h)] == 1, (s, qt, h)


@pytest.mark.parametrize("P,m,hq,n_cu", SHAPES)
def test_split_rule_and_balance(P, m, hq, n_cu):
    entries, wgs = fo.attn_schedule(P, m, hq, n_cu)
    qtiles = (m + 127) // 128
    total = sum(hq * (_walk_tiles(s, qt, m) + COST) for s in range(P) for qt in range(qtiles))
    share = -(-total // (2 * n_cu))
    cost = {}
    for wg, s, qt, h, w in entries:
        t = _walk_tiles(s, qt, m)
        if w < 0:
            assert t < 2 or t + COST <= share
            c = t + COST
        else:
            assert t >= 2 and t + COST > share
            c = ((t + 1) // 2 if (w & 1) == 0 else t - (t + 1) // 2) + COST
        cost.setdefault(wg, 0)
        cost[wg] += c
    if len(entries) <= n_cu:
        assert sorted(cost) == list(range(len(entries)))  # one item per workgroup
        return
    per_cu = collections.Counter()
    for wg, c in cost.items():
        per_cu[wg % n_cu] += c
    avg = sum(per_cu.values()) / n_cu
    item_max = max(((_walk_tiles(s, qt, m) + 1) // 2 if w >= 0 else _walk_tiles(s, qt, m)) + COST
                   for _, s, qt, _, w in entries)
    assert max(per_cu.values()) <= avg + item_max, (max(per_cu.values()), avg, item_max)


def test_lists_depend_on_the_shape_alone():
    a = fo.attn_schedule(8, 1024, 8, 256)
    b = fo.attn_schedule(8, 1024, 8, 256)
    assert a == b
    entries, wgs = a
    # the 70B Ulysses share at 8K tokens: 512 items, the 256 longest cut in two, two lists a CU
    assert wgs == 512
    assert sum(1 for e in entries if e[4] < 0) == 256
    assert sum(1 for e in entries if e[4] >= 0) == 512


def test_rejects_bad_shapes():
    import ctypes
    lib = fo.load()
    cnt, wgs = ctypes.c_int64(), ctypes.c_int32()
    assert lib.fo_attn_schedule(0, 64, 8, 256, None, 0, ctypes.byref(cnt), ctypes.byref(wgs)) \
        == fo.FO_ERR_INVALID_ARG
    assert lib.fo_attn_schedule(8, 64, 8, 0, None, 0, ctypes.byref(cnt), ctypes.byref(wgs)) \
        == fo.FO_ERR_INVALID_ARG
    assert lib.fo_attn_schedule(8, 64, 8, 256, None, 4, ctypes.byref(cnt), ctypes.byref(wgs)) \
        == fo.FO_ERR_INVALID_ARG
