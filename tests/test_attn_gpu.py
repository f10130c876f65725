"""GPU parity of the query-split attention behind a Flash All-to-All (fo_attn) and of its
resident form (fo_attn_ref), against the CPU oracle on the same seeded inputs, through the C ABI.

Tolerance: the kernel rounds the probabilities to bf16 before the value product (relative error
at most 2^-9 on each term p_j v_j, while the normalizing sum uses the unrounded p_j) and the
output to bf16 once (at most 2^-9 of the value). So each element is within
2^-9 (sum_j p_j |v_j| / sum_j p_j + |out|), up to fp32 sums; the oracle gives the first term as
the attention of the same scores over |V|. The check allows twice that, and a relative Frobenius
error of 3e-3 (two roundings; the output rounding alone is about 1.5e-3 on these inputs)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from comm_overlapped_sliced_amd import configs, flashovl as fo, inputs
from tests.gpu_helpers import from_dev, oracle_cached, rel_frobenius, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

TOL_ATTN = 3e-3
D = 128


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    fo.load()
    return torch.device("cuda:0")


def _abs_values(qkv, hq, hkv):
    """qkv with every value entry replaced by its magnitude (sign bit cleared)."""
    a = qkv.copy()
    a[:, (hq + hkv) * D:] &= np.uint16(0x7FFF)
    return a


def _check(got, qkv, hq, hkv, causal, what, rows=None, refs=None):
    ref = oracle.attn(qkv, hq, hkv, causal, rows=rows) if refs is None else refs[0]
    err = rel_frobenius(got, ref)
    print(f"{what}: relF {err:.2e}", flush=True)
    assert err <= TOL_ATTN, f"{what}: relF {err:.3e}"
    mag = (oracle.attn(_abs_values(qkv, hq, hkv), hq, hkv, causal, rows=rows) if refs is None
           else refs[1])
    bad = np.abs(got - ref) > 2.0 ** -8 * (mag + np.abs(ref)) + 1e-6
    assert not bad.any(), f"{what}: {bad.sum()} elements off, e.g. {np.argwhere(bad)[:3]}"


@pytest.mark.parametrize("S,hq,hkv,causal", [(200, 4, 2, True), (200, 4, 2, False),
                                             (1, 2, 1, True), (64, 8, 1, True),
                                             (300, 2, 2, False), (129, 8, 8, True)])
def test_attn_ref_against_oracle(dev, S, hq, hkv, causal):
    qkv = inputs.normal(8000 + S + hq, (S, (hq + 2 * hkv) * D), 1.0, "bf16")
    out = torch.full((S, hq * D), float("nan"), dtype=torch.bfloat16, device=dev)
    fo.attn_ref(to_dev(qkv, dev), out, hq, hkv, causal, stream=torch.cuda.current_stream())
    fo.check(torch.cuda.current_stream())
    _check(from_dev(out), qkv, hq, hkv, causal, f"S{S} hq{hq} hkv{hkv} causal{causal}")


def _sliced(dev, qkv, P, rank, hq, hkv, causal, o=None, arrivals=True, send=True):
    """fo_attn with both exchanges (send=True: the output rows of every slice but the rank's own
    go back to their owner): checks that every sent slice equals the rank's output rows bit for
    bit and that the own slice's buffer is untouched, and returns the output."""
    S, row = qkv.shape
    m = S // P
    slices = [to_dev(qkv[s * m:(s + 1) * m], dev) for s in range(P)]
    recv = torch.empty((S, row), dtype=torch.bfloat16, device=dev)
    if not arrivals:  # the slices already in place
        for s in range(P):
            recv[s * m:(s + 1) * m] = slices[s]
    out = torch.full((S, hq * D), float("nan"), dtype=torch.bfloat16, device=dev)
    back = [torch.full((m, hq * D), float("nan"), dtype=torch.bfloat16, device=dev)
            for _ in range(P)] if send else None
    st = torch.cuda.current_stream()
    o = o or fo.opts()
    if not arrivals:
        o.arrival = fo.ARR_NONE
    fo.attn(slices[rank], slices if arrivals else None, recv, out, P, rank, hq, hkv, causal,
            compute_stream=st, o=o, out_peer=back)
    fo.check(st)
    assert not torch.isnan(out).any().item()
    if send:
        for s in range(P):
            if s == rank:
                assert torch.isnan(back[s]).all().item(), "the own slice is not sent"
            else:
                assert torch.equal(back[s], out[s * m:(s + 1) * m]), f"slice {s} sent to rank {s}"
    return out


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("order", [fo.ORDER_FLASH, fo.ORDER_NATURAL], ids=["flash", "natural"])
def test_attn_sliced_against_oracle(dev, causal, order):
    # P = 4 slices of 72 tokens: ragged query tiles (72 of 128) and key tiles (72 = 64 + 8)
    P, m, hq, hkv = 4, 72, 4, 1
    qkv = inputs.normal(8100 + causal, (P * m, (hq + 2 * hkv) * D), 1.0, "bf16")
    for rank in (0, P - 1):
        out = _sliced(dev, qkv, P, rank, hq, hkv, causal, fo.opts(order=order))
        _check(from_dev(out), qkv, hq, hkv, causal, f"rank {rank} order {order} causal {causal}")


@pytest.mark.parametrize("groups", [1, 2, 3, 8])
def test_attn_row_group_arrivals(dev, groups):
    """Slices sent in row groups (each a whole number of 128-row query tiles; m = 200 leaves a
    short last group): every query and key tile waits for its own group."""
    P, m, hq, hkv = 3, 200 if groups < 8 else 1024, 2, 1
    qkv = inputs.normal(8150 + groups, (P * m, (hq + 2 * hkv) * D), 1.0, "bf16")
    for rank in (0, P - 1):
        out = _sliced(dev, qkv, P, rank, hq, hkv, True, fo.opts(row_groups=groups))
        if m <= 256:
            _check(from_dev(out), qkv, hq, hkv, True, f"groups {groups} rank {rank}")
        else:
            rows = np.arange(0, P * m, 37)
            _check(from_dev(out[torch.from_numpy(rows).to(dev)]), qkv, hq, hkv, True,
                   f"groups {groups} rank {rank}", rows=rows)


@pytest.mark.parametrize("epl", [1, 2, 3], ids=["one_engine", "engine_pair", "pair_split"])
@pytest.mark.parametrize("groups", [1, 2])
@pytest.mark.parametrize("order", [fo.ORDER_FLASH, fo.ORDER_NATURAL], ids=["flash", "natural"])
def test_attn_return_exchange_every_rank(dev, groups, order, epl):
    """The return All-to-All at every rank, whole slices and two row groups per slice (the second
    one short: m = 200 rows), against the oracle: each slice's rows reach its owner (checked in
    _sliced), and the output, including the own slice computed last, is the attention."""
    P, m, hq, hkv = 4, 200, 2, 1
    qkv = inputs.normal(8170 + groups, (P * m, (hq + 2 * hkv) * D), 1.0, "bf16")
    for rank in range(P):
        out = _sliced(dev, qkv, P, rank, hq, hkv, True,
                      fo.opts(row_groups=groups, order=order, engines_per_link=epl))
        _check(from_dev(out), qkv, hq, hkv, True, f"return exchange rank {rank} groups {groups}")
    # without the return exchange the output is the same, bit for bit
    a = _sliced(dev, qkv, P, 1, hq, hkv, True, fo.opts(row_groups=groups, order=order))
    b = _sliced(dev, qkv, P, 1, hq, hkv, True, fo.opts(row_groups=groups, order=order), send=False)
    assert torch.equal(a, b)


def test_attn_arrivals_match_resident_slices(dev):
    """Gating changes when a key slice is read, not what is computed: the call with arrivals
    equals the same call on slices already in place, bit for bit."""
    P, m, hq, hkv = 4, 200, 2, 1
    qkv = inputs.normal(8200, (P * m, (hq + 2 * hkv) * D), 1.0, "bf16")
    for rank in (1, 3):
        a = _sliced(dev, qkv, P, rank, hq, hkv, True)
        b = _sliced(dev, qkv, P, rank, hq, hkv, True, arrivals=False)
        assert torch.equal(a, b), f"rank {rank}"


def test_attn_sliced_equals_resident_in_natural_order(dev):
    """With the slices walked in index order the sliced call visits the keys in the order of the
    resident call, so the two agree bit for bit."""
    P, m, hq, hkv = 4, 128, 2, 2
    qkv = inputs.normal(8300, (P * m, (hq + 2 * hkv) * D), 1.0, "bf16")
    sl = _sliced(dev, qkv, P, 2, hq, hkv, True, fo.opts(order=fo.ORDER_NATURAL))
    ref = torch.empty_like(sl)
    fo.attn_ref(to_dev(qkv, dev), ref, hq, hkv, True, stream=torch.cuda.current_stream())
    fo.check(torch.cuda.current_stream())
    assert torch.equal(sl, ref)


@pytest.mark.parametrize("rank", [0, 7])
def test_attn_l70b(dev, rank):
    """The Llama-3.1-70B Ulysses share (8 slices of 1024 tokens, 8 query heads, 1 key/value head,
    causal) with both exchanges: every query row and head against the oracle (the result does
    not depend on the rank, so the oracle runs once), and every sent slice equal to those rows."""
    c = configs.L70B_ATTN
    qkv = c.qkv()
    out = _sliced(dev, qkv, c.P, rank, c.hq, c.hkv, c.causal)
    ref, mag = oracle_cached(("attn", c.name), lambda: (
        oracle.attn(qkv, c.hq, c.hkv, c.causal),
        oracle.attn(_abs_values(qkv, c.hq, c.hkv), c.hq, c.hkv, c.causal)))
    _check(from_dev(out), qkv, c.hq, c.hkv, c.causal, f"L70B rank {rank}", refs=(ref, mag))


def test_attn_back_to_back_calls_see_new_arrivals(dev):
    """Calls enqueued back to back with no other kernel between them, the peers' rows
    alternating between two sets and landing in the same receive buffer (rows of 2560 bytes,
    cache-line aligned, so the arrival waits take no cache invalidation): each call must equal
    the resident attention of its own set, bit for bit (index order walks the keys as the
    resident call does)."""
    P, m, hq, hkv = 4, 256, 8, 1
    row = (hq + 2 * hkv) * D
    sets = [inputs.normal(8400 + i, (P * m, row), 1.0, "bf16") for i in range(2)]
    st = torch.cuda.current_stream()
    refs, slices = [], []
    for q in sets:
        qd = to_dev(q, dev)
        ref = torch.empty((P * m, hq * D), dtype=torch.bfloat16, device=dev)
        fo.attn_ref(qd, ref, hq, hkv, True, stream=st)
        refs.append(ref)
        slices.append([qd[s * m:(s + 1) * m].contiguous() for s in range(P)])
    recv = torch.empty((P * m, row), dtype=torch.bfloat16, device=dev)
    outs = [torch.empty((P * m, hq * D), dtype=torch.bfloat16, device=dev) for _ in range(6)]
    # the return exchange into the same receive buffers every call: each call's sent rows must
    # be its own (calls in a row, one kernel after the other)
    backs = [[torch.empty((m, hq * D), dtype=torch.bfloat16, device=dev) for _ in range(P)]
             for _ in range(6)]
    for it in range(6):
        i, rank = it % 2, (it * 3) % P
        fo.attn(slices[i][rank], slices[i], recv, outs[it], P, rank, hq, hkv, True,
                compute_stream=st, o=fo.opts(order=fo.ORDER_NATURAL), out_peer=backs[it])
    fo.check(st)
    for it in range(6):
        rank = (it * 3) % P
        assert torch.equal(outs[it], refs[it % 2]), f"call {it}"
        for s in range(P):
            if s != rank:
                assert torch.equal(backs[it][s], refs[it % 2][s * m:(s + 1) * m]), f"call {it} slice {s}"


def test_attn_split_items_same_bits_every_call(dev):
    """Causal items longer than a workgroup's share are cut in two along their keys and the two
    halves combined in a fixed order: whichever half ends last, every call gives the same bits
    (resident form and the sliced call with both exchanges), within the tolerance of the oracle."""
    S, hq, hkv = 2048, 8, 1
    qkv = inputs.normal(8190, (S, (hq + 2 * hkv) * D), 1.0, "bf16")
    qd = to_dev(qkv, dev)
    st = torch.cuda.current_stream()
    outs = []
    for _ in range(4):
        out = torch.full((S, hq * D), float("nan"), dtype=torch.bfloat16, device=dev)
        fo.attn_ref(qd, out, hq, hkv, True, stream=st)
        fo.check(st)
        outs.append(out)
    for o in outs[1:]:
        assert torch.equal(o, outs[0])
    _check(from_dev(outs[0]), qkv, hq, hkv, True, "split items, resident")
    P = 8
    a = _sliced(dev, qkv, P, 5, hq, hkv, True)
    b = _sliced(dev, qkv, P, 5, hq, hkv, True)
    assert torch.equal(a, b)
    _check(from_dev(a), qkv, hq, hkv, True, "split items, sliced")


def test_attn_many_shapes_rebuild_tables(dev):
    """More causal shapes than the device keeps tables for: the tables are dropped and built
    again, and a shape seen before gives the same bits after the rebuild."""
    hq, hkv = 2, 1
    st = torch.cuda.current_stream()
    sizes = [64 + 8 * k for k in range(70)]
    qkvs = {S: inputs.normal(8300 + S, (S, (hq + 2 * hkv) * D), 1.0, "bf16") for S in (sizes[0], sizes[-1])}
    first = None
    for S in sizes + [sizes[0]]:
        qkv = qkvs.get(S)
        if qkv is None:
            qkv = inputs.normal(8300 + S, (S, (hq + 2 * hkv) * D), 1.0, "bf16")
        out = torch.full((S, hq * D), float("nan"), dtype=torch.bfloat16, device=dev)
        fo.attn_ref(to_dev(qkv, dev), out, hq, hkv, True, stream=st)
        fo.check(st)
        assert not torch.isnan(out).any().item(), f"S={S}"
        if S == sizes[0]:
            if first is None:
                first = out
            else:
                assert torch.equal(out, first)
    _check(from_dev(first), qkvs[sizes[0]], hq, hkv, True, "after the table rebuild")


@pytest.mark.parametrize("std", [3.0, 0.05], ids=["peaked", "flat"])
def test_attn_split_items_extreme_softmax(dev, std):
    """Split items under a peaked softmax (queries and keys with standard deviation 3: scores of
    several hundred, so the two halves' maxima differ widely and one half's weight underflows)
    and a flat one (std 0.05: every key nearly equal), resident and sliced, against the oracle."""
    S, hq, hkv, P = 2048, 8, 1, 8
    qkv = inputs.normal(8400 + int(std * 100), (S, (hq + 2 * hkv) * D), 1.0, "bf16")
    scaled = inputs.normal(8401 + int(std * 100), (S, (hq + hkv) * D), std, "bf16")
    qkv[:, :(hq + hkv) * D] = scaled  # queries and keys at `std`, values at 1
    st = torch.cuda.current_stream()
    out = torch.full((S, hq * D), float("nan"), dtype=torch.bfloat16, device=dev)
    fo.attn_ref(to_dev(qkv, dev), out, hq, hkv, True, stream=st)
    fo.check(st)
    _check(from_dev(out), qkv, hq, hkv, True, f"split items, std {std}, resident")
    a = _sliced(dev, qkv, P, 3, hq, hkv, True)
    _check(from_dev(a), qkv, hq, hkv, True, f"split items, std {std}, sliced")


@pytest.mark.parametrize("P,m", [(1, 8000), (8, 1000)], ids=["resident_8000", "sliced_8x1000"])
def test_attn_split_items_ragged_length(dev, P, m):
    """Split items at lengths that are not a multiple of the 128-query tile or the 64-key tile
    (the last query tile of a slice holds 64 or 104 rows, the last key tile of the diagonal is
    partly past the slice): the resident call (P = 1, 8000 tokens) or the sliced one with both
    exchanges (P = 8, m = 1000, rank 6), twice with the same bits, against the oracle on rows at
    the start, around a split item of the middle and at the ragged end of every slice."""
    hq, hkv = 8, 1
    S = P * m
    sched, _ = fo.attn_schedule(P, m, hq, torch.cuda.get_device_properties(dev).multi_processor_count)
    assert sum(1 for e in sched if e[4] >= 0) > 0, "the shape has split items"
    qkv = inputs.normal(8600 + m, (S, (hq + 2 * hkv) * D), 1.0, "bf16")
    st = torch.cuda.current_stream()
    if P == 1:
        qd = to_dev(qkv, dev)
        outs = []
        for _ in range(2):
            out = torch.full((S, hq * D), float("nan"), dtype=torch.bfloat16, device=dev)
            fo.attn_ref(qd, out, hq, hkv, True, stream=st)
            fo.check(st)
            outs.append(out)
    else:
        outs = [_sliced(dev, qkv, P, 6, hq, hkv, True) for _ in range(2)]
    assert torch.equal(outs[0], outs[1])
    rows = sorted({r for s in range(P) for r in
                   [*range(s * m, s * m + 16), *range(s * m + m // 2 - 8, s * m + m // 2 + 8),
                    *range(s * m + m - 40, s * m + m)]})
    _check(from_dev(outs[0])[rows], qkv, hq, hkv, True, f"split items, ragged, P={P} m={m}",
           rows=rows)


def test_attn_missed_arrival_times_out_then_recovers(dev):
    """Causal attention with split items whose arrival waits have a 1 us bound against transfers
    over one link: the call reports FO_ERR_TIMEOUT and every kernel still finishes (both halves of
    every pair reach their combine), and the next calls, with split items again, are correct and
    give the same bits as before the timeout."""
    P, m, hq, hkv = 8, 256, 8, 1
    qkv = inputs.normal(8500, (P * m, (hq + 2 * hkv) * D), 1.0, "bf16")
    before = _sliced(dev, qkv, P, 2, hq, hkv, True)
    slices = [to_dev(qkv[s * m:(s + 1) * m], dev) for s in range(P)]
    recv = torch.empty((P * m, qkv.shape[1]), dtype=torch.bfloat16, device=dev)
    out = torch.empty((P * m, hq * D), dtype=torch.bfloat16, device=dev)
    st = torch.cuda.current_stream()
    s = fo.attn(slices[2], slices, recv, out, P, 2, hq, hkv, True, compute_stream=st,
                o=fo.opts(spin_timeout_us=1, links=1), raw=True)
    assert s == fo.FO_OK
    with pytest.raises(fo.FoError) as ei:
        fo.check(st)
    assert ei.value.status == fo.FO_ERR_TIMEOUT
    fo.check(st)
    after = _sliced(dev, qkv, P, 2, hq, hkv, True)
    assert torch.equal(after, before)
    _check(from_dev(after), qkv, hq, hkv, True, "after a timed-out call")
