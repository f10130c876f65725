"""GPU tests of per-slice gating: a slice is read only after it has arrived, stale data in the
receive buffers is never used, late arrivals only delay the result, and an arrival that never
comes within the bound is reported as FO_ERR_TIMEOUT while every kernel still finishes.

Late and missing arrivals are forced from the host: the caller's copy stream is held by a
sleeping kernel queued before the call, so the copies start late; the kernels' own bounded waits
guarantee termination."""
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


@pytest.fixture(scope="module")
def cycles_per_ms(dev):
    """Calibrates torch.cuda._sleep (a one-wave spin kernel) against event time."""
    s = torch.cuda.Stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(s):
        torch.cuda._sleep(1000)
        e0.record(s)
        torch.cuda._sleep(2_000_000)
        e1.record(s)
    s.synchronize()
    ms = e0.elapsed_time(e1)
    assert ms > 0
    return 2_000_000 / ms


def _delay(stream, cycles_per_ms, ms):
    with torch.cuda.stream(stream):
        torch.cuda._sleep(int(cycles_per_ms * ms))


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
        for engine in (fo.COPY_SDMA, fo.COPY_BLIT):
            prob.x_recv.view(torch.int16).fill_(-1)
            got = prob.run(it % P, o=fo.opts(copy_engine=engine))
            assert not np.isnan(got).any()
            assert rel_frobenius(got, refs[i]) <= TOL_BF16, f"iteration {it} engine {engine}"


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


@pytest.mark.parametrize("engine", [fo.COPY_SDMA, fo.COPY_BLIT], ids=["sdma", "blit"])
def test_late_arrivals_only_delay(dev, cycles_per_ms, engine):
    P, m, K, N = 8, 256, 1024, 512
    x = inputs.normal(7800, (P * m, K), 1.0, "bf16")
    w = inputs.normal(7801, (K, N), 0.02, "bf16")
    prob = AG(x, w, P, dev)
    ref = oracle.gemm(x, w)
    copy = torch.cuda.Stream()
    prob.x_recv.view(torch.int16).fill_(-1)
    _delay(copy, cycles_per_ms, 5.0)
    got = prob.run(2, o=fo.opts(copy_engine=engine), copy_stream=copy)
    assert rel_frobenius(got, ref) <= TOL_BF16
    parts = [inputs.normal(7810 + q, (m, N), 1.0, "f32") for q in range(P)]
    rs = RS(x, w, parts, P, dev)
    rs.recv.fill_(float("nan"))
    _delay(copy, cycles_per_ms, 5.0)
    out, _ = rs.run(6, o=fo.opts(copy_engine=engine), copy_stream=copy)
    assert rel_frobenius(out, oracle.rs(x, w, parts, P, 6)) <= TOL_BF16


def test_withheld_arrival_times_out(dev, cycles_per_ms):
    """Arrivals held back far beyond a 2 ms bound: the call reports FO_ERR_TIMEOUT, the kernel
    finishes, and the next call is correct again."""
    P, m, K, N = 4, 128, 256, 256
    x = inputs.normal(7900, (P * m, K), 1.0, "bf16")
    w = inputs.normal(7901, (K, N), 0.02, "bf16")
    prob = AG(x, w, P, dev)
    copy = torch.cuda.Stream()
    _delay(copy, cycles_per_ms, 60.0)
    st = fo.ag_gemm(prob.peer[1], prob.peer, prob.x_recv, prob.w_d, prob.y, P, 1,
                    compute_stream=torch.cuda.current_stream(), copy_stream=copy,
                    o=fo.opts(spin_timeout_us=2000), raw=True)
    assert st == fo.FO_OK
    with pytest.raises(fo.FoError) as ei:
        fo.check(torch.cuda.current_stream())
    assert ei.value.status == fo.FO_ERR_TIMEOUT
    # the record is cleared and the path works again
    fo.check(torch.cuda.current_stream())
    got = prob.run(1)
    assert rel_frobenius(got, oracle.gemm(x, w)) <= TOL_BF16
