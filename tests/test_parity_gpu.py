"""GPU parity: fo_ag_gemm / fo_gemm_rs / fo_gemm_ref against the CPU oracle on the same seeded
inputs, called through the C ABI.

Bar: bit-exact on integer-valued fp32 inputs; relative Frobenius error <= 2e-3 for bf16 operands
with fp32 accumulation and <= 1e-6 for fp32 operands. Small cases compare every element with
the full oracle; the full-size workloads compare sampled entries (plus the slice-edge corners)
with the oracle's sampled products and check the exactness invariant of the FlashOverlap page
(technical summary section 3: slicing never changes the result) bit for bit against the
unsliced fo_gemm_ref.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from comm_overlapped_sliced_amd import configs, flashovl as fo, inputs
from tests.gpu_helpers import (TOL_BF16, TOL_F32, ag_oracle_blocks, check_ag_blocks, check_rs,
                               from_dev, rel_frobenius, rs_oracle, to_dev)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    fo.load()
    for name in ("libamdhip64", "libhsa-runtime64"):
        assert len(fo.runtimes_mapped(name)) == 1, fo.runtimes_mapped(name)
    return torch.device("cuda:0")


def _stream():
    return torch.cuda.current_stream()


class AG:
    """Device buffers of one Flash-AG problem."""

    def __init__(self, x: np.ndarray, w: np.ndarray, P: int, dev, out_dt="bf16"):
        self.P = P
        self.M, self.K = x.shape
        self.m = self.M // P
        self.N = w.shape[1]
        self.x, self.w = x, w
        self.slices = [x[s * self.m:(s + 1) * self.m] for s in range(P)]
        self.peer = [to_dev(s, dev) for s in self.slices]
        self.w_d = to_dev(w, dev)
        dt = torch.bfloat16 if x.dtype == np.uint16 else torch.float32
        self.x_recv = torch.empty((self.M, self.K), dtype=dt, device=dev)
        ot = torch.bfloat16 if out_dt == "bf16" else torch.float32
        self.y = torch.empty((self.M, self.N), dtype=ot, device=dev)
        self.dev = dev

    def run(self, r, o=None, resident=False):
        if resident:  # arrivals NONE: the slices are already in x_recv
            for s in range(self.P):
                if s != r:
                    self.x_recv[s * self.m:(s + 1) * self.m].copy_(self.peer[s])
            fo.ag_gemm(self.peer[r], None, self.x_recv, self.w_d, self.y, self.P, r,
                       compute_stream=_stream(), o=o)
        else:
            fo.ag_gemm(self.peer[r], self.peer, self.x_recv, self.w_d, self.y, self.P, r,
                       compute_stream=_stream(), o=o)
        fo.check(_stream())
        return from_dev(self.y)


class RS:
    """Device buffers of one Flash-RS problem."""

    def __init__(self, x: np.ndarray, w: np.ndarray, partials, P: int, dev):
        self.P = P
        self.M, self.K = x.shape
        self.m = self.M // P
        self.N = w.shape[1]
        self.x, self.w, self.partials = x, w, partials
        self.x_d = to_dev(x, dev)
        self.w_d = to_dev(w, dev)
        self.peer = [to_dev(p, dev) for p in partials]
        self.send = torch.empty((self.M, self.N), dtype=torch.float32, device=dev)
        self.out = torch.empty((self.m, self.N), dtype=torch.float32, device=dev)
        self.recv = torch.empty((self.M, self.N), dtype=torch.float32, device=dev)

    def run(self, r, o=None, resident=False):
        self.send.fill_(float("nan"))
        if resident:
            for q in range(self.P):
                if q != r:
                    self.recv[q * self.m:(q + 1) * self.m].copy_(self.peer[q])
            fo.gemm_rs(self.x_d, self.w_d, self.send, self.out, None, self.recv, self.P, r,
                       compute_stream=_stream(), o=o)
        else:
            fo.gemm_rs(self.x_d, self.w_d, self.send, self.out, self.peer, self.recv, self.P, r,
                       compute_stream=_stream(), o=o)
        fo.check(_stream())
        return from_dev(self.out), from_dev(self.send)


# emulated link topologies: one DMA engine per peer (default), and every transfer over one link
LINKS = [("mesh", 0), ("onelink", 1)]


# ---- config 1: integer-valued fp32, bit-exact ----------------------------------------------

@pytest.mark.parametrize("links", LINKS, ids=lambda e: e[0])
@pytest.mark.parametrize("mode", ["eager", "resident"])
def test_tiny_fp32_ag_bit_exact(dev, links, mode):
    c = configs.TINY_AG
    prob = AG(c.x(), c.w(), c.P, dev, out_dt="f32")
    for r in range(c.P):
        got = prob.run(r, o=fo.opts(links=links[1]), resident=(mode == "resident"))
        ref = oracle.ag(prob.slices, c.w(), c.P, r)
        assert np.array_equal(got, ref), f"rank {r}"


@pytest.mark.parametrize("links", LINKS, ids=lambda e: e[0])
@pytest.mark.parametrize("arrival", [("lockstep", fo.ARR_LOCKSTEP), ("eager", fo.ARR_EAGER),
                                     ("resident", None)], ids=lambda a: a[0])
def test_tiny_fp32_rs_bit_exact(dev, links, arrival):
    c = configs.TINY_RS
    parts = [c.partial(q) for q in range(c.P)]
    prob = RS(c.x(), c.w(), parts, c.P, dev)
    for r in range(c.P):
        o = fo.opts(links=links[1], arrival=arrival[1] or fo.ARR_DEFAULT)
        out, send = prob.run(r, o=o, resident=arrival[1] is None)
        ref_out, ref_send = oracle.rs(c.x(), c.w(), parts, c.P, r, want_send=True)
        assert np.array_equal(out, ref_out), f"rank {r}"
        m = c.m
        for d in range(c.P):
            if d == r:
                assert np.all(np.isnan(send[d * m:(d + 1) * m])), "own chunk is not sent"
            else:
                assert np.array_equal(send[d * m:(d + 1) * m], ref_send[d * m:(d + 1) * m])


@pytest.mark.parametrize("arrival", [("lockstep", fo.ARR_LOCKSTEP), ("eager", fo.ARR_EAGER),
                                     ("resident", None)], ids=lambda a: a[0])
def test_tiny_fp32_natural_order_bit_exact(dev, arrival):
    """The data-slicing order (NATURAL): slices in index order; for RS the own chunk is written
    where it falls and the partials are added after the GEMM. Exact on integers, every rank."""
    c = configs.TINY_AG
    prob = AG(c.x(), c.w(), c.P, dev, out_dt="f32")
    cr = configs.TINY_RS
    parts = [cr.partial(q) for q in range(cr.P)]
    rs = RS(cr.x(), cr.w(), parts, cr.P, dev)
    for r in range(c.P):
        if arrival[1] != fo.ARR_LOCKSTEP:
            got = prob.run(r, o=fo.opts(order=fo.ORDER_NATURAL,
                                        arrival=arrival[1] or fo.ARR_DEFAULT),
                           resident=arrival[1] is None)
            assert np.array_equal(got, oracle.ag(prob.slices, c.w(), c.P, r)), f"AG rank {r}"
        out, send = rs.run(r, o=fo.opts(order=fo.ORDER_NATURAL,
                                        arrival=arrival[1] or fo.ARR_DEFAULT),
                           resident=arrival[1] is None)
        ref_out, ref_send = oracle.rs(cr.x(), cr.w(), parts, cr.P, r, want_send=True)
        assert np.array_equal(out, ref_out), f"RS rank {r}"
        keep = ~np.isnan(ref_send)
        assert np.array_equal(send[keep], ref_send[keep])


def test_natural_rs_matches_flash_bitwise(dev):
    """Both orders add the same partials in the same order onto the same fp32 accumulator."""
    P, m, K, N = 4, 520, 264, 392
    x = inputs.normal(7380, (P * m, K), 1.0, "bf16")
    w = inputs.normal(7381, (K, N), 0.02, "bf16")
    parts = [inputs.normal(7390 + q, (m, N), 1.0, "f32") for q in range(P)]
    rs = RS(x, w, parts, P, dev)
    for r in (0, 3):
        flash, _ = rs.run(r, o=fo.opts(tile=fo.TILE_128x128))
        nat, _ = rs.run(r, o=fo.opts(tile=fo.TILE_128x128, order=fo.ORDER_NATURAL, row_groups=1))
        assert np.array_equal(flash, nat), f"rank {r}"
        assert rel_frobenius(nat, oracle.rs(x, w, parts, P, r)) <= TOL_BF16


def test_fp32_non_integer_tolerance(dev):
    """Non-integer fp32 operands pin the fp32 path itself (integers are exact in bf16 too)."""
    P, M, K, N = 4, 256, 256, 512
    x = inputs.normal(7001, (M, K), 1.0, "f32")
    w = inputs.normal(7002, (K, N), 1.0, "f32")
    prob = AG(x, w, P, dev, out_dt="f32")
    got = prob.run(2)
    assert rel_frobenius(got, oracle.ag(prob.slices, w, P, 2)) <= TOL_F32
    parts = [inputs.normal(7010 + q, (M // P, N), 1.0, "f32") for q in range(P)]
    rs = RS(x, w, parts, P, dev)
    out, send = rs.run(1)
    ref_out, ref_send = oracle.rs(x, w, parts, P, 1, want_send=True)
    assert rel_frobenius(out, ref_out) <= TOL_F32
    keep = ~np.isnan(ref_send)
    assert rel_frobenius(send[keep], ref_send[keep]) <= TOL_F32


# ---- bf16: several tiles, ragged tails, every tile shape -----------------------------------

TILES = [("256x256", fo.TILE_256x256), ("256x128", fo.TILE_256x128),
         ("128x256", fo.TILE_128x256), ("128x128", fo.TILE_128x128), ("64x64", fo.TILE_64x64)]


@pytest.mark.parametrize("tile", TILES, ids=lambda t: t[0])
@pytest.mark.parametrize("shape", [(4, 200, 520, 392), (3, 256, 576, 512), (2, 37, 72, 136)],
                         ids=lambda s: "P%d_m%d_K%d_N%d" % s)
def test_bf16_ragged_all_tiles(dev, tile, shape):
    P, m, K, N = shape
    x = inputs.normal(7100 + m, (P * m, K), 1.0, "bf16")
    w = inputs.normal(7200 + N, (K, N), 0.02, "bf16")
    prob = AG(x, w, P, dev)
    ref = oracle.gemm(x, w)
    y_ref = torch.empty_like(prob.y)
    fo.gemm_ref(to_dev(x, dev), prob.w_d, y_ref, tile=tile[1], stream=_stream())
    outs = {}
    for r in sorted({0, P - 1}):
        got = outs[r] = prob.run(r, o=fo.opts(tile=tile[1]))
        assert rel_frobenius(got, ref) <= TOL_BF16, f"rank {r}"
        # exactness of slicing: the sliced product equals the unsliced one bit for bit
        assert np.array_equal(got, from_dev(y_ref)), f"rank {r}"
    # fp32 output of the same product; the bf16 output is that fp32 sum rounded to nearest even
    prob32 = AG(x, w, P, dev, out_dt="f32")
    got32 = prob32.run(0, o=fo.opts(tile=tile[1]))
    assert rel_frobenius(got32, ref) <= 1e-5
    assert np.array_equal(_round_bf16(got32), outs[0])


def _round_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 values rounded to the nearest bf16, ties to even (finite inputs), as fp64."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("tile", TILES, ids=lambda t: t[0])
def test_bf16_rs_ragged(dev, tile):
    P, m, K, N = 4, 200, 520, 392
    x = inputs.normal(7300, (P * m, K), 1.0, "bf16")
    w = inputs.normal(7301, (K, N), 0.02, "bf16")
    parts = [inputs.normal(7310 + q, (m, N), 1.0, "f32") for q in range(P)]
    prob = RS(x, w, parts, P, dev)
    for r in (0, 3):
        out, send = prob.run(r, o=fo.opts(tile=tile[1]))
        ref_out, ref_send = oracle.rs(x, w, parts, P, r, want_send=True)
        assert rel_frobenius(out, ref_out) <= TOL_BF16
        keep = ~np.isnan(ref_send)
        assert np.all(np.isnan(send[~keep]))
        assert rel_frobenius(send[keep], ref_send[keep]) <= TOL_BF16


@pytest.mark.parametrize("groups", [1, 2, 3, 0], ids=lambda g: f"groups{g}")
def test_row_groups(dev, groups):
    """Slices cut into row groups (each its own transfer, gate and release): ragged slices of five
    128-row tile rows, every arrival mode and both link layouts, against the oracle."""
    P, m, K, N = 4, 520, 264, 392
    x = inputs.normal(7350, (P * m, K), 1.0, "bf16")
    w = inputs.normal(7351, (K, N), 0.02, "bf16")
    ref = oracle.gemm(x, w)
    ag = AG(x, w, P, dev)
    parts = [inputs.normal(7360 + q, (m, N), 1.0, "f32") for q in range(P)]
    rs = RS(x, w, parts, P, dev)
    for r, links in ((1, 0), (2, 1)):
        ag.x_recv.view(torch.int16).fill_(-1)
        got = ag.run(r, o=fo.opts(tile=fo.TILE_128x128, row_groups=groups, links=links))
        assert not np.isnan(got).any()
        assert rel_frobenius(got, ref) <= TOL_BF16, f"AG rank {r} links {links}"
        for arrival in (fo.ARR_LOCKSTEP, fo.ARR_EAGER):
            rs.recv.fill_(float("nan"))
            out, send = rs.run(r, o=fo.opts(tile=fo.TILE_128x128, row_groups=groups, links=links,
                                             arrival=arrival))
            ref_out, ref_send = oracle.rs(x, w, parts, P, r, want_send=True)
            assert rel_frobenius(out, ref_out) <= TOL_BF16, f"RS rank {r} arrival {arrival}"
            keep = ~np.isnan(ref_send)
            assert rel_frobenius(send[keep], ref_send[keep]) <= TOL_BF16


# ---- degenerate cases ------------------------------------------------------------------------

def test_single_rank_and_tiny_shapes(dev):
    """Degenerate shapes. The AG output is taken in fp32 here: with only a handful of entries,
    the bf16 rounding of the output alone can push the relative error past 2e-3 by chance; the
    rounded output is instead held to half a bf16 ulp (plus fp32 accumulation error) per entry."""
    for (P, m, K, N) in [(1, 64, 128, 64), (2, 1, 8, 8), (1, 1, 8, 8), (5, 3, 16, 24)]:
        x = inputs.normal(7400 + m, (P * m, K), 1.0, "bf16")
        w = inputs.normal(7401 + K, (K, N), 0.02, "bf16")
        ref = oracle.gemm(x, w)
        prob32 = AG(x, w, P, dev, out_dt="f32")
        assert rel_frobenius(prob32.run(P - 1), ref) <= 1e-5
        prob = AG(x, w, P, dev)
        got = prob.run(P - 1)
        assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6)
        parts = [inputs.normal(7410 + q, (m, N), 1.0, "f32") for q in range(P)]
        rs = RS(x, w, parts, P, dev)
        out, _ = rs.run(0)
        assert rel_frobenius(out, oracle.rs(x, w, parts, P, 0)) <= TOL_BF16


def test_empty_reduction(dev):
    """K = 0: the products are empty sums (zeros); RS returns just the sum of the partials."""
    P, m, N = 4, 64, 128
    dt = torch.bfloat16
    x_local = torch.empty((m, 8), dtype=dt, device=dev)
    w = torch.empty((8, N), dtype=dt, device=dev)
    y = torch.full((P * m, N), 7.0, dtype=dt, device=dev)
    x_recv = torch.empty((P * m, 8), dtype=dt, device=dev)
    st = fo.load().fo_ag_gemm(x_local.data_ptr(), None, x_recv.data_ptr(), w.data_ptr(),
                              y.data_ptr(), P, 0, m, 0, N, fo.BF16, fo.BF16, None, None, None)
    assert st == fo.FO_OK
    fo.check(None)
    assert torch.all(y == 0)
    parts = [inputs.integers(7500 + q, (m, N), -3, 3, "f32") for q in range(P)]
    peer = [to_dev(p, dev) for p in parts]
    out = torch.full((m, N), 5.0, device=dev)
    send = torch.empty((P * m, N), device=dev)
    recv = torch.empty((P * m, N), device=dev)
    import ctypes
    arr = (ctypes.c_void_p * P)(*[p.data_ptr() for p in peer])
    st = fo.load().fo_gemm_rs(x_local.data_ptr(), w.data_ptr(), send.data_ptr(), out.data_ptr(),
                              ctypes.cast(arr, ctypes.c_void_p), recv.data_ptr(), P, 2, m, 0, N,
                              fo.BF16, None, None, None)
    assert st == fo.FO_OK
    fo.check(None)
    expect = sum(parts[q].astype(np.float64) for q in range(P) if q != 2)
    assert np.array_equal(from_dev(out), expect)


# ---- the full-size workloads: every entry, or whole rows and columns of every tile ----------
#
# The 70B shares (and the 1K-8K sweep) are compared entry by entry with the full oracle output.
# For the largest products (16K tokens, 405B) every tile is checked on whole rows (the first,
# the last and one random row of every tile row of every slice, all N columns) and whole
# columns (the first, the last and one random column of every tile column, all rows): the
# oracle computes those rows and columns as a smaller problem of the same definition (each
# output entry depends only on its row of X, its column of W and its partials). Every rank's
# output must also equal the unsliced fo_gemm_ref bit for bit (the page's exactness claim,
# technical summary section 3).

def _ag_full(case, dev, ranks):
    x, w = case.x(), case.w()
    prob = AG(x, w, case.P, dev)
    y_ref = torch.empty_like(prob.y)
    fo.gemm_ref(to_dev(x, dev), prob.w_d, y_ref, stream=_stream())
    torch.cuda.synchronize()
    mono = from_dev(y_ref)
    blocks = ag_oracle_blocks(case)
    tile = fo.tile_info(case.P, case.m, case.K, case.N)[:2]
    check_ag_blocks(mono, blocks, fo.tile_info(1, case.M, case.K, case.N)[:2],
                    f"{case.name}: fo_gemm_ref")
    for r in ranks:
        got = prob.run(r)
        check_ag_blocks(got, blocks, tile, f"{case.name}: rank {r}")
        assert np.array_equal(got, mono), f"rank {r}: sliced != unsliced"


def test_l70b_ag_every_rank(dev):
    _ag_full(configs.L70B_AG, dev, ranks=range(8))


@pytest.mark.parametrize("case", configs.SWEEP_AG, ids=lambda c: f"M{c.M}")
def test_sweep_ag(dev, case):
    _ag_full(case, dev, ranks=(0, 5))


def test_l405b_ag(dev):
    _ag_full(configs.L405B_AG, dev, ranks=(0, 3))


def _rs_full(case, dev, ranks):
    x, w = case.x(), case.w()
    parts = [case.partial(q) for q in range(case.P)]
    prob = RS(x, w, parts, case.P, dev)
    y_ref = torch.empty((case.M, case.N), dtype=torch.float32, device=dev)
    fo.gemm_ref(prob.x_d, prob.w_d, y_ref, stream=_stream())
    torch.cuda.synchronize()
    mono = from_dev(y_ref)
    m = case.m
    tile = fo.tile_info(case.P, m, case.K, case.N, out_dt=fo.F32)[:2]
    for r in ranks:
        out, send = prob.run(r)
        check_rs(out, send, rs_oracle(case, r), case, r, tile)
        for d in range(case.P):
            blk = send[d * m:(d + 1) * m]
            if d == r:
                assert np.all(np.isnan(blk))
                continue
            # chunks for other ranks are rows of the unsliced product, bit for bit
            assert np.array_equal(blk, mono[d * m:(d + 1) * m]), f"rank {r} chunk {d}"


def test_l70b_rs_every_rank(dev):
    _rs_full(configs.L70B_RS, dev, ranks=range(8))


def test_l405b_rs(dev):
    _rs_full(configs.L405B_RS, dev, ranks=(0, 6))
