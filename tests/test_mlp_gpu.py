"""GPU parity of the MLP block (AG gate+up -> SwiGLU -> RS down, one rank's share) and of its
activation kernel fo_swiglu, against the CPU oracle on the same seeded inputs, through the C ABI.

The oracle rounds the activations between the kernels to bf16 as the kernels' bf16 tensors do
(Y after the gate+up projection, H after SwiGLU); the bar is the relative Frobenius error of
2e-3 of bf16 operands, and for fo_swiglu alone one bf16 rounding per element."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from comm_overlapped_sliced_amd import configs, flashovl as fo, inputs
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


def _stream():
    return torch.cuda.current_stream()


@pytest.mark.parametrize("shape", [(300, 264), (1, 8), (4096, 3584)], ids=lambda s: "%dx%d" % s)
def test_swiglu_against_oracle(dev, shape):
    rows, inter = shape
    y = inputs.normal(7700 + rows, (rows, 2 * inter), 2.0, "bf16")
    h = torch.full((rows, inter), float("nan"), dtype=torch.bfloat16, device=dev)
    fo.swiglu(to_dev(y, dev), h, stream=_stream())
    torch.cuda.synchronize()
    got, ref = from_dev(h), oracle.swiglu(y)
    # fp32 arithmetic and one rounding to bf16: within one bf16 unit in the last place
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-30)
    assert rel_frobenius(got, ref) <= TOL_BF16


def _block(dev, x, w_gu, w_d, parts, P, r, o_ag=None, o_rs=None):
    """The block on the GPU: rank r's out [m, N] (fp32)."""
    M, K = x.shape
    m = M // P
    inter = w_gu.shape[1] // 2
    N = w_d.shape[1]
    slices = [to_dev(x[s * m:(s + 1) * m], dev) for s in range(P)]
    w_gu_d, w_d_d = to_dev(w_gu, dev), to_dev(w_d, dev)
    x_recv = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    y = torch.empty((M, 2 * inter), dtype=torch.bfloat16, device=dev)
    h = torch.empty((M, inter), dtype=torch.bfloat16, device=dev)
    peer = [to_dev(p, dev) for p in parts]
    send = torch.empty((M, N), device=dev)
    out = torch.empty((m, N), device=dev)
    recv = torch.empty((M, N), device=dev)
    s = _stream()
    fo.ag_gemm(slices[r], slices, x_recv, w_gu_d, y, P, r, compute_stream=s, o=o_ag)
    fo.swiglu(y, h, stream=s)
    fo.gemm_rs(h, w_d_d, send, out, peer, recv, P, r, compute_stream=s, o=o_rs)
    fo.check(s)
    return from_dev(out)


def test_mlp_block_against_oracle(dev):
    P, m, K, inter, N = 4, 72, 264, 256, 392
    x = inputs.normal(7750, (P * m, K), 1.0, "bf16")
    w_gu = inputs.normal(7751, (K, 2 * inter), 0.05, "bf16")
    w_d = inputs.normal(7752, (inter, N), 0.05, "bf16")
    parts = [inputs.normal(7760 + q, (m, N), 1.0, "f32") for q in range(P)]
    slices = [x[s * m:(s + 1) * m] for s in range(P)]
    for r in (0, P - 1):
        ref = oracle.mlp_block(slices, w_gu, w_d, parts, P, r)
        got = _block(dev, x, w_gu, w_d, parts, P, r)
        assert rel_frobenius(got, ref) <= TOL_BF16, f"rank {r}"
        # the page's data-slicing order gives the same block output
        nat = _block(dev, x, w_gu, w_d, parts, P, r, o_ag=fo.opts(order=fo.ORDER_NATURAL),
                     o_rs=fo.opts(order=fo.ORDER_NATURAL, row_groups=1))
        assert rel_frobenius(nat, ref) <= TOL_BF16, f"rank {r} natural"


def test_mlp_block_l70b(dev):
    """The Llama-3.1-70B block (gate+up of config 2, down of config 3, seven fp32 partials), rank
    0: every entry of the rank's output chunk against the oracle, which needs only slice 0 of X
    (the rows of H that the own chunk reads)."""
    ag, rs = configs.L70B_AG, configs.L70B_RS
    P, m, inter = ag.P, ag.m, rs.K
    x, w_gu, w_d = ag.x(), ag.w(), rs.w()
    parts = [rs.partial(q) for q in range(P)]
    r = 0
    got = _block(dev, x, w_gu, w_d, parts, P, r)
    y0 = oracle.round_bf16(oracle.gemm(x[r * m:(r + 1) * m], w_gu))
    h0 = oracle.round_bf16(oracle.swiglu(y0))
    ref = oracle.gemm(h0, w_d) + sum(parts[q].astype(np.float64) for q in range(P) if q != r)
    assert rel_frobenius(got, ref) <= TOL_BF16
