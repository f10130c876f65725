"""GPU test of the library's ordering of calls on different streams: a Flash-AG call and a
Flash-RS call that consumes its output, enqueued on two streams in turn with no event or host
synchronization between them. Each call waits for the previous call on the device, whichever
stream that was on, so every result equals that of the same calls on one stream, bit for bit;
an RS reading its input early would read the NaN the AG output starts with."""
from __future__ import annotations

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


def test_ag_then_rs_alternating_streams(dev):
    P, m, K, N1, N2, r = 4, 256, 512, 512, 384, 1
    print(f"streams P={P} m={m} K={K} N1={N1} N2={N2} rank={r}", flush=True)
    x = inputs.normal(8100, (P * m, K), 1.0, "bf16")
    w1 = inputs.normal(8101, (K, N1), 0.02, "bf16")
    w2 = inputs.normal(8102, (N1, N2), 0.02, "bf16")
    parts = [inputs.normal(8110 + q, (m, N2), 1.0, "f32") for q in range(P)]
    xd = to_dev(x, dev)
    slices = [xd[s * m:(s + 1) * m] for s in range(P)]
    w1d, w2d = to_dev(w1, dev), to_dev(w2, dev)
    peers = [to_dev(p, dev) for p in parts]
    x_recv = torch.empty((P * m, K), dtype=torch.bfloat16, device=dev)
    send = torch.empty((P * m, N2), dtype=torch.float32, device=dev)
    recv = torch.empty((P * m, N2), dtype=torch.float32, device=dev)

    def nan_y():
        return torch.full((P * m, N1), float("nan"), dtype=torch.bfloat16, device=dev)

    def nan_out():
        return torch.full((m, N2), float("nan"), dtype=torch.float32, device=dev)

    # the same two calls on one stream
    s0 = torch.cuda.current_stream()
    y_ref, out_ref = nan_y(), nan_out()
    fo.ag_gemm(slices[r], slices, x_recv, w1d, y_ref, P, r, compute_stream=s0)
    fo.gemm_rs(y_ref, w2d, send, out_ref, peers, recv, P, r, compute_stream=s0)
    fo.check(s0)
    y_host = from_dev(y_ref)
    assert rel_frobenius(y_host, oracle.gemm(x, w1)) <= TOL_BF16
    y_bits = y_ref.view(torch.int16).cpu().numpy().view(np.uint16)
    ref_out = oracle.rs(y_bits, w2, parts, P, r)
    out_host = from_dev(out_ref)
    assert rel_frobenius(out_host, ref_out) <= TOL_BF16

    reps = 6
    ys = [nan_y() for _ in range(reps)]
    outs = [nan_out() for _ in range(reps)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for k in range(reps):
        sa, sb = streams[k % 2], streams[(k + 1) % 2]
        fo.ag_gemm(slices[r], slices, x_recv, w1d, ys[k], P, r, compute_stream=sa)
        fo.gemm_rs(ys[k], w2d, send, outs[k], peers, recv, P, r, compute_stream=sb)
    for s in streams:
        fo.check(s)
    torch.cuda.synchronize()
    ref_y_bits = y_ref.view(torch.int16).cpu().numpy()
    for k in range(reps):
        assert np.array_equal(ys[k].view(torch.int16).cpu().numpy(), ref_y_bits), f"AG call {k}"
        assert np.array_equal(from_dev(outs[k]), out_host), f"RS call {k}"
