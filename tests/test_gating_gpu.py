"""GPU tests of per-slice gating: a slice is read only after it has arrived, stale data in the
receive buffers is never used, late arrivals only delay the result, and an arrival that does not
come within the bound is reported as FO_ERR_TIMEOUT while every kernel still finishes.

Late arrivals are forced by the sizes: large slices carried one after the other over a single
emulated link (one DMA engine) against a GEMM whose N is small, so the GEMM reaches every slice
long before it lands. A missed arrival is forced from the host with a 1 us bound on the
kernel's own waits; the transfers still land and fo_check() waits for them."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from comm_overlapped_sliced_amd import flashovl as fo, inputs
from tests.gpu_helpers import TOL_BF16, from_dev, rel_frobenius, to_dev
from tests.test_parity_gpu import AG, RS

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    fo.load()
    return torch.device("cuda:0")


def test_poisoned_rerun_ag(dev):
    """Receive buffer filled with NaN before every call and the peers' data alternated between
    calls: any early or stale read shows up as a wrong or NaN result."""
    P, m, K, N = 8, 256, 1024, 512
    xs = [inputs.normal(7600 + i, (P * m, K), 1.0, "bf16") for i in range(2)]
    w = inputs.normal(7602, (K, N), 0.02, "bf16")
    probs = [AG(x, w, P, dev) for x in xs]
    refs = [oracle.gemm(x, w) for x in xs]
    for it in range(6):
        i = it % 2
        prob = probs[i]
        # share one receive buffer between both problems, poisoned each time
        prob.x_recv = probs[0].x_recv
        prob.x_recv.view(torch.int16).fill_(-1)  # 0xffff: a bf16 NaN
        for links in (0, 1):
            prob.x_recv.view(torch.int16).fill_(-1)
            got = prob.run(it % P, o=fo.opts(links=links))
            assert not np.isnan(got).any()
            assert rel_frobenius(got, refs[i]) <= TOL_BF16, f"iteration {it} links {links}"


def test_poisoned_rerun_rs(dev):
    P, m, K, N = 8, 128, 512, 256
    x = inputs.normal(7700, (P * m, K), 1.0, "bf16")
    w = inputs.normal(7701, (K, N), 0.02, "bf16")
    part_sets = [[inputs.normal(7710 + 10 * i + q, (m, N), 1.0, "f32") for q in range(P)]
                 for i in range(2)]
    probs = [RS(x, w, ps, P, dev) for ps in part_sets]
    for it in range(6):
        i = it % 2
        prob = probs[i]
        prob.recv = probs[0].recv
        for arrival in (fo.ARR_LOCKSTEP, fo.ARR_EAGER):
            prob.recv.fill_(float("nan"))
            r = (3 * it) % P
            out, _ = prob.run(r, o=fo.opts(arrival=arrival))
            assert not np.isnan(out).any()
            ref = oracle.rs(x, w, part_sets[i], P, r)
            assert rel_frobenius(out, ref) <= TOL_BF16, f"iteration {it}"


def test_late_arrivals_only_delay(dev):
    """Seven 8 MiB slices over one link take about a millisecond; the GEMM (N = 128) needs a few
    microseconds per slice, so every received slice is waited for."""
    P, m, K, N = 8, 1024, 4096, 128
    x = inputs.normal(7800, (P * m, K), 1.0, "bf16")
    w = inputs.normal(7801, (K, N), 0.02, "bf16")
    prob = AG(x, w, P, dev)
    ref = oracle.gemm(x, w)
    for r in (2, 5):
        prob.x_recv.view(torch.int16).fill_(-1)
        got = prob.run(r, o=fo.opts(links=1))
        assert not np.isnan(got).any()
        assert rel_frobenius(got, ref) <= TOL_BF16
    # Flash-RS: seven 8 MiB partials over one link, K = 64
    Pr, mr, Kr, Nr = 8, 512, 64, 4096
    xr = inputs.normal(7802, (Pr * mr, Kr), 1.0, "bf16")
    wr = inputs.normal(7803, (Kr, Nr), 0.02, "bf16")
    parts = [inputs.normal(7810 + q, (mr, Nr), 1.0, "f32") for q in range(Pr)]
    rs = RS(xr, wr, parts, Pr, dev)
    for r, arrival in ((6, fo.ARR_LOCKSTEP), (1, fo.ARR_EAGER)):
        rs.recv.fill_(float("nan"))
        out, _ = rs.run(r, o=fo.opts(links=1, arrival=arrival))
        assert not np.isnan(out).any()
        assert rel_frobenius(out, oracle.rs(xr, wr, parts, Pr, r)) <= TOL_BF16


def test_missed_arrival_times_out(dev):
    """A 1 us bound on the in-kernel waits against transfers that take a millisecond: the call
    reports FO_ERR_TIMEOUT, the kernel finishes, fo_check() waits for the transfers, and the next
    call is correct again."""
    P, m, K, N = 8, 1024, 4096, 128
    x = inputs.normal(7900, (P * m, K), 1.0, "bf16")
    w = inputs.normal(7901, (K, N), 0.02, "bf16")
    prob = AG(x, w, P, dev)
    st = fo.ag_gemm(prob.peer[1], prob.peer, prob.x_recv, prob.w_d, prob.y, P, 1,
                    compute_stream=torch.cuda.current_stream(),
                    o=fo.opts(spin_timeout_us=1, links=1), raw=True)
    assert st == fo.FO_OK
    with pytest.raises(fo.FoError) as ei:
        fo.check(torch.cuda.current_stream())
    assert ei.value.status == fo.FO_ERR_TIMEOUT
    # the record is cleared and the path works again
    fo.check(torch.cuda.current_stream())
    got = prob.run(1)
    assert rel_frobenius(got, oracle.gemm(x, w)) <= TOL_BF16


@pytest.mark.parametrize("epl", [1, 2, 3], ids=["one_engine", "engine_pair", "pair_split"])
@pytest.mark.parametrize("chunks", [0, 4])
def test_back_to_back_calls_see_new_arrivals(dev, chunks, epl):
    """Calls enqueued back to back with no other kernel between them, the peers' data
    alternating between two sets and landing in the same receive buffer: each call's kernel
    reads the rows the previous call read, so a cached line of the previous data would show.
    Each result must equal the unsliced product of its own data bit for bit. (Rows of 8 KB and
    K blocks of 2 KB lie on 128-byte cache lines, so the arrival waits take no cache
    invalidation.)"""
    P, m, K, N = 8, 512, 4096, 512
    xs = [inputs.normal(7950 + i, (P * m, K), 1.0, "bf16") for i in range(2)]
    w = inputs.normal(7952, (K, N), 0.02, "bf16")
    w_d = to_dev(w, dev)
    refs = []
    for x in xs:
        y = torch.empty((P * m, N), dtype=torch.bfloat16, device=dev)
        fo.gemm_ref(to_dev(x, dev), w_d, y, stream=torch.cuda.current_stream())
        refs.append(y)

    def layout(t):
        if not chunks:
            return t.contiguous()
        return t.reshape(m, chunks, K // chunks).permute(1, 0, 2).contiguous().reshape(m, K)

    peers = [[layout(to_dev(x[s * m:(s + 1) * m], dev)) for s in range(P)] for x in xs]
    x_recv = torch.empty((P * m, K), dtype=torch.bfloat16, device=dev)
    ys = [torch.empty((P * m, N), dtype=torch.bfloat16, device=dev) for _ in range(8)]
    stream = torch.cuda.current_stream()
    for links in (0, 1):
        for it in range(8):
            i, r = it % 2, (3 * it) % P
            fo.ag_gemm(peers[i][r], peers[i], x_recv, w_d, ys[it], P, r, compute_stream=stream,
                       o=fo.opts(links=links, k_chunks=chunks, engines_per_link=epl))
        fo.check(stream)
        for it in range(8):
            assert torch.equal(ys[it].view(torch.int16), refs[it % 2].view(torch.int16)), \
                f"call {it} links {links} engines per link {epl}"
