"""GPU tests of the Flash-RS tail: with 16-byte aligned buffers the own chunk's tiles store their
fp32 sums and workgroups appended to the grid add the received partials onto them; otherwise the
own tiles add them in their epilogue. Both add the same partials in the same order onto the same
fp32 accumulator, so the results must be equal bit for bit: the fused epilogue is forced by an
output buffer that is 4-byte but not 16-byte aligned."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from comm_overlapped_sliced_amd import configs, flashovl as fo, inputs
from tests.gpu_helpers import TOL_BF16, check_rs, from_dev, rel_frobenius, rs_oracle, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    fo.load()
    return torch.device("cuda:0")


def _stream():
    return torch.cuda.current_stream()


class RSPair:
    """One Flash-RS problem with two outputs: aligned (tail workgroups) and offset by one float
    (the own tiles' fused epilogue)."""

    def __init__(self, x, w, parts, P, dev):
        self.P = P
        self.m = x.shape[0] // P
        self.N = w.shape[1]
        self.x_d, self.w_d = to_dev(x, dev), to_dev(w, dev)
        self.peer = [to_dev(p, dev) for p in parts]
        self.send = torch.empty((P * self.m, self.N), dtype=torch.float32, device=dev)
        self.recv = torch.empty((P * self.m, self.N), dtype=torch.float32, device=dev)
        self.out_a = torch.empty((self.m, self.N), dtype=torch.float32, device=dev)
        self.buf = torch.empty(self.m * self.N + 4, dtype=torch.float32, device=dev)
        self.out_u = self.buf[1:1 + self.m * self.N].view(self.m, self.N)  # 4 bytes past 16

    def run(self, r, out, o=None, resident=False):
        out.fill_(float("nan"))
        if resident:
            for q in range(self.P):
                if q != r:
                    self.recv[q * self.m:(q + 1) * self.m].copy_(self.peer[q])
        fo.gemm_rs(self.x_d, self.w_d, self.send, out, None if resident else self.peer,
                   self.recv, self.P, r, compute_stream=_stream(), o=o)
        fo.check(_stream())
        return from_dev(out)


@pytest.mark.parametrize("shape", [(4, 200, 520, 392), (8, 512, 512, 1024), (3, 300, 256, 136),
                                   (2, 64, 128, 64)], ids=lambda s: "P%d_m%d_K%d_N%d" % s)
@pytest.mark.parametrize("tile", [fo.TILE_AUTO, fo.TILE_128x256, fo.TILE_64x64, fo.TILE_256x256])
def test_tail_equals_fused_epilogue(dev, shape, tile):
    P, m, K, N = shape
    x = inputs.normal(8400 + m, (P * m, K), 1.0, "bf16")
    w = inputs.normal(8401, (K, N), 0.02, "bf16")
    parts = [inputs.normal(8410 + q, (m, N), 1.0, "f32") for q in range(P)]
    prob = RSPair(x, w, parts, P, dev)
    assert prob.out_u.data_ptr() % 16 == 4
    for r in sorted({0, P - 1, 1 % P}):
        ref = oracle.rs(x, w, parts, P, r)
        for arrival, groups, resident, epl in ((fo.ARR_LOCKSTEP, 0, False, 1),
                                               (fo.ARR_EAGER, 1, False, 1),
                                               (fo.ARR_NONE, 0, True, 1),
                                               (fo.ARR_LOCKSTEP, 2, False, 1),
                                               (fo.ARR_LOCKSTEP, 0, False, 2),
                                               (fo.ARR_LOCKSTEP, 0, False, 3)):
            o = fo.opts(tile=tile, arrival=arrival, row_groups=groups, engines_per_link=epl)
            a = prob.run(r, prob.out_a, o, resident)
            u = prob.run(r, prob.out_u, o, resident)
            assert not np.isnan(a).any()
            assert np.array_equal(a, u), f"rank {r} arrival {arrival} groups {groups}"
            assert rel_frobenius(a, ref) <= TOL_BF16


def test_tail_l70b_down(dev):
    """The 70B down projection at ranks 0 and 7: the tail equals the fused epilogue bit for bit,
    and the own chunk and every send chunk equal the full oracle output entry by entry."""
    c = configs.L70B_RS
    x, w = c.x(), c.w()
    parts = [c.partial(q) for q in range(c.P)]
    prob = RSPair(x, w, parts, c.P, dev)
    tile = fo.tile_info(c.P, c.m, c.K, c.N, out_dt=fo.F32)[:2]
    for r in (0, 7):
        a = prob.run(r, prob.out_a)
        send = from_dev(prob.send)
        u = prob.run(r, prob.out_u)
        assert np.array_equal(a, u), f"rank {r}"
        check_rs(a, send, rs_oracle(c, r), c, r, tile)


def test_back_to_back_calls_see_new_partials(dev):
    """Flash-RS calls enqueued back to back, the peers' partials alternating between two sets
    and landing in the same receive buffer: each call reads the rows the previous call read.
    Both forms of the adds (the tail workgroups, and the own tiles' epilogue with an output
    that is not 16-byte aligned) must give each set's result, bit for bit the same every time."""
    P, m, K, N = 8, 256, 512, 1024
    x = inputs.normal(8700, (P * m, K), 1.0, "bf16")
    w = inputs.normal(8701, (K, N), 0.02, "bf16")
    sets = [[inputs.normal(8710 + 10 * i + q, (m, N), 1.0, "f32") for q in range(P)]
            for i in range(2)]
    x_d, w_d = to_dev(x, dev), to_dev(w, dev)
    peers = [[to_dev(p, dev) for p in ps] for ps in sets]
    send = torch.empty((P * m, N), dtype=torch.float32, device=dev)
    recv = torch.empty((P * m, N), dtype=torch.float32, device=dev)
    n = 8
    buf = torch.empty(n * (m * N + 4), dtype=torch.float32, device=dev)
    stream = _stream()
    r = 3
    for aligned in (True, False):
        outs = []
        for it in range(n):
            base = it * (m * N + 4) + (0 if aligned else 1)
            out = buf[base:base + m * N].view(m, N)
            assert (out.data_ptr() % 16 == 0) == aligned
            fo.gemm_rs(x_d, w_d, send, out, peers[it % 2], recv, P, r, compute_stream=stream)
            outs.append(out)
        fo.check(stream)
        got = [from_dev(o) for o in outs]
        for i in range(2):
            ref = oracle.rs(x, w, sets[i], P, r)
            assert rel_frobenius(got[i], ref) <= TOL_BF16, f"set {i} aligned {aligned}"
            for it in range(i + 2, n, 2):
                assert np.array_equal(got[it], got[i]), f"call {it} aligned {aligned}"


def test_tail_missed_partial_times_out(dev):
    """A 1 us bound on the in-kernel waits against partials that take a millisecond over one
    link: the tail workgroups give up, the call reports FO_ERR_TIMEOUT, every kernel finishes,
    and the next call is correct again."""
    P, m, K, N = 8, 512, 64, 4096
    x = inputs.normal(8800, (P * m, K), 1.0, "bf16")
    w = inputs.normal(8801, (K, N), 0.02, "bf16")
    parts = [inputs.normal(8810 + q, (m, N), 1.0, "f32") for q in range(P)]
    prob = RSPair(x, w, parts, P, dev)
    st = fo.gemm_rs(prob.x_d, prob.w_d, prob.send, prob.out_a, prob.peer, prob.recv, P, 2,
                    compute_stream=_stream(), o=fo.opts(spin_timeout_us=1, links=1), raw=True)
    assert st == fo.FO_OK
    with pytest.raises(fo.FoError) as ei:
        fo.check(_stream())
    assert ei.value.status == fo.FO_ERR_TIMEOUT
    fo.check(_stream())
    got = prob.run(2, prob.out_a, fo.opts(links=1))
    assert rel_frobenius(got, oracle.rs(x, w, parts, P, 2)) <= TOL_BF16
