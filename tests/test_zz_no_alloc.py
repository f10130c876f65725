"""fo_gemm_rs_noalloc (Flash-RS with resident partials, scratch in a static device array)
against fo_gemm_rs with the same resident partials, through the C ABI: every bit of the own
chunk and of every send chunk, on calls in a row whose second input is smaller (the array keeps
the previous call's counters and words), in both orders, and against the oracle."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

import oracle
from comm_overlapped_sliced_amd import flashovl as fo, inputs
from tests.gpu_helpers import TOL_BF16, from_dev, rel_frobenius, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    fo.load()
    return torch.device("cuda:0")


def _problem(dev, P, m, K, N, seed):
    x = inputs.normal(seed, (P * m, K), 1.0, "bf16")
    w = inputs.normal(seed + 1, (K, N), 0.02, "bf16")
    parts = [inputs.normal(seed + 10 + q, (m, N), 1.0, "f32") for q in range(P)]
    recv = torch.empty((P * m, N), dtype=torch.float32, device=dev)
    for q in range(P):
        recv[q * m:(q + 1) * m] = to_dev(parts[q], dev)
    return x, w, parts, to_dev(x, dev), to_dev(w, dev), recv


def _run(fn, dev, xd, wd, recv, P, r, m, N, o):
    send = torch.full((P * m, N), float("nan"), dtype=torch.float32, device=dev)
    out = torch.full((m, N), float("nan"), dtype=torch.float32, device=dev)
    s = torch.cuda.current_stream()
    fn(xd, wd, send, out, recv, P, r, s, o)
    fo.check(s)
    return from_dev(out), from_dev(send)


def _noalloc(xd, wd, send, out, recv, P, r, s, o):
    fo.gemm_rs_noalloc(xd, wd, send, out, recv, P, r, compute_stream=s, o=o)


def _regular(xd, wd, send, out, recv, P, r, s, o):
    fo.gemm_rs(xd, wd, send, out, None, recv, P, r, compute_stream=s, o=o)


@pytest.mark.parametrize("order", [fo.ORDER_FLASH, fo.ORDER_NATURAL], ids=["flash", "natural"])
def test_noalloc_equals_gemm_rs_on_calls_in_a_row(dev, order):
    # the 70B down-projection share first, then a smaller ragged problem on the same array
    cases = [(8, 512, 3584, 8192, 3, 9100), (4, 200, 520, 392, 1, 9200), (3, 64, 256, 136, 2, 9300)]
    for P, m, K, N, r, seed in cases:
        print(f"noalloc case P={P} m={m} K={K} N={N} rank={r} order={order}", flush=True)
        x, w, parts, xd, wd, recv = _problem(dev, P, m, K, N, seed)
        o = fo.opts(order=order)
        out_a, send_a = _run(_noalloc, dev, xd, wd, recv, P, r, m, N, o)
        out_b, send_b = _run(_regular, dev, xd, wd, recv, P, r, m, N, fo.opts(order=order,
                                                                               arrival=fo.ARR_NONE))
        assert not np.isnan(out_a).any()
        assert np.array_equal(out_a, out_b), f"own chunk P={P} m={m}"
        for d in range(P):
            blk_a, blk_b = send_a[d * m:(d + 1) * m], send_b[d * m:(d + 1) * m]
            if d == r:
                assert np.isnan(blk_a).all()
            else:
                assert np.array_equal(blk_a, blk_b), f"send chunk {d} P={P} m={m}"
        if P * m * K * N <= 8 * 512 * 3584 * 8192:
            ref = oracle.rs(x, w, parts, P, r)
            assert rel_frobenius(out_a, ref) <= TOL_BF16


def test_noalloc_rejects_arrivals_and_bad_args(dev):
    lib = fo.load()
    P, m, K, N = 4, 64, 256, 512
    t = [torch.empty(n, dtype=torch.float32, device=dev) for n in (P * m * N, m * N, P * m * N)]
    xd = torch.empty((P * m, K), dtype=torch.bfloat16, device=dev)
    wd = torch.empty((K, N), dtype=torch.bfloat16, device=dev)
    o = fo.opts(arrival=fo.ARR_EAGER)
    st = lib.fo_gemm_rs_noalloc(xd.data_ptr(), wd.data_ptr(), t[0].data_ptr(), t[1].data_ptr(),
                                t[2].data_ptr(), P, 0, m, K, N, fo.BF16, None, ctypes.byref(o))
    assert st == fo.FO_ERR_INVALID_ARG
    st = lib.fo_gemm_rs_noalloc(xd.data_ptr(), wd.data_ptr(), t[0].data_ptr(), t[0].data_ptr(),
                                t[2].data_ptr(), P, 0, m, K, N, fo.BF16, None, None)
    assert st == fo.FO_ERR_INVALID_ARG  # out overlaps send_buf


@pytest.mark.parametrize("order", [fo.ORDER_FLASH, fo.ORDER_NATURAL], ids=["flash", "natural"])
def test_noalloc_captured_in_a_graph(dev, order):
    """The call captured in a HIP graph (torch.cuda.graph) and replayed four times, with eager
    work between the replays (the outputs poisoned, another problem run eagerly through the same
    static array): every replay equals the eager call bit for bit."""
    P, m, K, N, r, seed = 4, 200, 520, 392, 1, 9400
    print(f"noalloc graph P={P} m={m} K={K} N={N} rank={r} order={order}", flush=True)
    x, w, parts, xd, wd, recv = _problem(dev, P, m, K, N, seed)
    o = fo.opts(order=order)
    out_e, send_e = _run(_noalloc, dev, xd, wd, recv, P, r, m, N, o)
    other = _problem(dev, 3, 64, 256, 136, seed + 50)

    send = torch.full((P * m, N), float("nan"), dtype=torch.float32, device=dev)
    out = torch.full((m, N), float("nan"), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st = fo.gemm_rs_noalloc(xd, wd, send, out, recv, P, r,
                                compute_stream=torch.cuda.current_stream(), o=o, raw=True)
    assert st == fo.FO_OK, fo.load().fo_last_error().decode()
    for rep in range(4):
        out.fill_(float("nan"))
        send.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        fo.check(torch.cuda.current_stream())
        assert np.array_equal(from_dev(out), out_e), f"replay {rep}: own chunk"
        got = from_dev(send)
        for d in range(P):
            if d != r:
                assert np.array_equal(got[d * m:(d + 1) * m], send_e[d * m:(d + 1) * m]), \
                    f"replay {rep}: send chunk {d}"
        # eager work on the same static array between replays
        _, _, _, oxd, owd, orecv = other
        _run(_noalloc, dev, oxd, owd, orecv, 3, 2, 64, 136, fo.opts(order=order))
    del g
