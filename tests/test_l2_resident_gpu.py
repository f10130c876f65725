"""Arrival waits without cache invalidation, on receive buffers small enough to stay in one XCD's
4 MB L2 between calls.

When every transfer starts and ends on a 128-byte line (the receive buffer 128-byte aligned and a
row, or a K block, a multiple of 128 bytes) the kernels take no acquire after an arrival wait:
the launch invalidates what earlier kernels cached, and no workgroup reads a row before its
transfer has landed. Calls enqueued back to back on one stream, the peers' data alternating
between two sets and landing in the same ~512 KB receive buffer, would show a stale line as a
result equal to the other set's. Each call must equal its own set's unsliced product bit for
bit: Flash-AG with row-major slices and with K blocks, Flash-RS with its partials added in the
own tiles' write-back (an output that is not 16-byte aligned), and the attention.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from comm_overlapped_sliced_amd import flashovl as fo, inputs
from tests.gpu_helpers import TOL_BF16, from_dev, rel_frobenius, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

P, CALLS = 8, 8


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    fo.load()
    return torch.device("cuda:0")


def _no_acquire(buf, row_bytes):
    """The condition under which the library takes no acquire after an arrival wait."""
    assert buf.data_ptr() % 128 == 0 and row_bytes % 128 == 0


@pytest.mark.parametrize("chunks", [0, 2])
def test_ag_l2_resident_alternating(dev, chunks):
    m, K, N = 64, 512, 256
    xs = [inputs.normal(9400 + i, (P * m, K), 1.0, "bf16") for i in range(2)]
    w = inputs.normal(9402, (K, N), 0.02, "bf16")
    w_d = to_dev(w, dev)
    stream = torch.cuda.current_stream()
    refs = []
    for x in xs:
        y = torch.empty((P * m, N), dtype=torch.bfloat16, device=dev)
        fo.gemm_ref(to_dev(x, dev), w_d, y, stream=stream)
        refs.append(y)

    def layout(t):
        if not chunks:
            return t.contiguous()
        return t.reshape(m, chunks, K // chunks).permute(1, 0, 2).contiguous().reshape(m, K)

    peers = [[layout(to_dev(x[s * m:(s + 1) * m], dev)) for s in range(P)] for x in xs]
    x_recv = torch.empty((P * m, K), dtype=torch.bfloat16, device=dev)
    assert x_recv.numel() * 2 <= 1 << 20
    _no_acquire(x_recv, (K // max(1, chunks)) * 2)
    ys = [torch.empty((P * m, N), dtype=torch.bfloat16, device=dev) for _ in range(CALLS)]
    for it in range(CALLS):
        i, r = it % 2, (5 * it) % P
        fo.ag_gemm(peers[i][r], peers[i], x_recv, w_d, ys[it], P, r, compute_stream=stream,
                   o=fo.opts(k_chunks=chunks))
    fo.check(stream)
    for it in range(CALLS):
        assert torch.equal(ys[it].view(torch.int16), refs[it % 2].view(torch.int16)), f"call {it}"


def test_rs_fused_writeback_l2_resident_alternating(dev):
    m, K, N = 64, 256, 256
    x = inputs.normal(9500, (P * m, K), 1.0, "bf16")
    w = inputs.normal(9501, (K, N), 0.02, "bf16")
    sets = [[inputs.normal(9510 + 10 * i + q, (m, N), 1.0, "f32") for q in range(P)]
            for i in range(2)]
    x_d, w_d = to_dev(x, dev), to_dev(w, dev)
    peers = [[to_dev(p, dev) for p in ps] for ps in sets]
    send = torch.empty((P * m, N), dtype=torch.float32, device=dev)
    recv = torch.empty((P * m, N), dtype=torch.float32, device=dev)
    assert recv.numel() * 4 <= 1 << 20
    _no_acquire(recv, N * 4)
    buf = torch.empty(CALLS * (m * N + 4), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    r = 6
    outs = []
    for it in range(CALLS):
        base = it * (m * N + 4) + 1   # 4 bytes past 16: the own tiles add the partials
        out = buf[base:base + m * N].view(m, N)
        assert out.data_ptr() % 16 == 4
        fo.gemm_rs(x_d, w_d, send, out, peers[it % 2], recv, P, r, compute_stream=stream)
        outs.append(out)
    fo.check(stream)
    got = [from_dev(o) for o in outs]
    for i in range(2):
        ref = oracle.rs(x, w, sets[i], P, r)
        assert rel_frobenius(got[i], ref) <= TOL_BF16, f"set {i}"
        for it in range(i + 2, CALLS, 2):
            assert np.array_equal(got[it], got[i]), f"call {it}"


def test_attn_l2_resident_alternating(dev):
    Pa, m, hq, hkv = 4, 128, 2, 1
    row = (hq + 2 * hkv) * 128
    sets = [inputs.normal(9600 + i, (Pa * m, row), 1.0, "bf16") for i in range(2)]
    stream = torch.cuda.current_stream()
    refs, slices = [], []
    for q in sets:
        qd = to_dev(q, dev)
        ref = torch.empty((Pa * m, hq * 128), dtype=torch.bfloat16, device=dev)
        fo.attn_ref(qd, ref, hq, hkv, True, stream=stream)
        refs.append(ref)
        slices.append([qd[s * m:(s + 1) * m].contiguous() for s in range(Pa)])
    recv = torch.empty((Pa * m, row), dtype=torch.bfloat16, device=dev)
    assert recv.numel() * 2 <= 1 << 20
    _no_acquire(recv, row * 2)
    outs = [torch.empty((Pa * m, hq * 128), dtype=torch.bfloat16, device=dev)
            for _ in range(CALLS)]
    for it in range(CALLS):
        i, rank = it % 2, (3 * it) % Pa
        # index order walks the keys as the resident call does, so the bits match
        fo.attn(slices[i][rank], slices[i], recv, outs[it], Pa, rank, hq, hkv, True,
                compute_stream=stream, o=fo.opts(order=fo.ORDER_NATURAL))
    fo.check(stream)
    for it in range(CALLS):
        assert torch.equal(outs[it], refs[it % 2]), f"call {it}"
