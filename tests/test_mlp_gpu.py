"""GPU parity of the MLP block (AG gate+up -> SwiGLU -> RS down, one rank's share) and of its
activation kernel fo_swiglu, against the CPU oracle on the same seeded inputs, through the C ABI.

The oracle rounds the activations between the kernels to bf16 as the kernels' bf16 tensors do
(Y after the gate+up projection, H after SwiGLU); the bar is the relative Frobenius error of
2e-3 of bf16 operands, and for fo_swiglu alone one bf16 rounding per element. With the SwiGLU
epilogue of fo_ag_gemm (fused) Y is never rounded: the oracle's fused block reads the fp64
projection."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from comm_overlapped_sliced_amd import configs, flashovl as fo, inputs
from tests.gpu_helpers import (TOL_BF16, ag_oracle_blocks, assert_parity, from_dev,
                               rel_frobenius, to_dev)

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


def _block(dev, x, w_gu, w_d, parts, P, r, o_ag=None, o_rs=None, fused=False):
    """The block on the GPU: rank r's out [m, N] (fp32). fused: the gate+up projection writes H
    through its SwiGLU epilogue (o_ag's other fields kept)."""
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
    if fused:
        o_ag = o_ag or fo.opts()
        o_ag.epilogue = fo.EPI_SWIGLU
        fo.ag_gemm(slices[r], slices, x_recv, w_gu_d, h, P, r, compute_stream=s, o=o_ag)
    else:
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
        ref_f = oracle.mlp_block(slices, w_gu, w_d, parts, P, r, fused=True)
        got_f = _block(dev, x, w_gu, w_d, parts, P, r, fused=True)
        assert rel_frobenius(got_f, ref_f) <= TOL_BF16, f"rank {r} fused"
        # the page's data-slicing order gives the same block output
        nat = _block(dev, x, w_gu, w_d, parts, P, r, o_ag=fo.opts(order=fo.ORDER_NATURAL),
                     o_rs=fo.opts(order=fo.ORDER_NATURAL, row_groups=1))
        assert rel_frobenius(nat, ref) <= TOL_BF16, f"rank {r} natural"


def test_mlp_block_l70b(dev):
    """The Llama-3.1-70B block (gate+up of config 2, down of config 3, seven fp32 partials), rank
    0: every entry of the rank's output chunk against the oracle's block.

    Per-element bound 2^-8 (|ref| + rms(ref)): Y and H are rounded to bf16 between the kernels,
    and where the GPU's fp32 sum and the oracle's exact sum fall on two sides of a rounding tie
    one entry of H differs by a bf16 ulp (2^-7 of it); the down projection weighs each such
    entry by a weight of about 0.02, so an output entry moves by a small fraction of rms(ref)
    (at most about 2e-3 of it measured), not by the 2^-14 of a single fp32 chain."""
    ag, rs = configs.L70B_AG, configs.L70B_RS
    P, m = ag.P, ag.m
    x, w_gu, w_d = ag.x(), ag.w(), rs.w()
    parts = [rs.partial(q) for q in range(P)]
    r = 0
    got = _block(dev, x, w_gu, w_d, parts, P, r)
    ref = oracle.mlp_block([x[q * m:(q + 1) * m] for q in range(P)], w_gu, w_d, parts, P, r)
    assert_parity(got, ref, "f32", what="70B MLP block, rank 0", bound=(2.0 ** -8, 2.0 ** -8))


def _ag_swiglu(dev, x, w_gu, P, r, o):
    """fo_ag_gemm with the SwiGLU epilogue: H [P*m, inter] (the bf16 device tensor)."""
    M, K = x.shape
    m = M // P
    inter = w_gu.shape[1] // 2
    slices = [to_dev(x[q * m:(q + 1) * m], dev) for q in range(P)]
    x_recv = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    h = torch.full((M, inter), float("nan"), dtype=torch.bfloat16, device=dev)
    o.epilogue = fo.EPI_SWIGLU
    s = _stream()
    fo.ag_gemm(slices[r], slices, x_recv, to_dev(w_gu, dev), h, P, r, compute_stream=s, o=o)
    fo.check(s)
    assert not torch.isnan(h).any().item()  # every element written
    return h


@pytest.mark.parametrize("tile", [fo.TILE_256x256, fo.TILE_256x128, fo.TILE_128x256,
                                  fo.TILE_128x128, fo.TILE_64x64],
                         ids=["256x256", "256x128", "128x256", "128x128", "64x64"])
def test_swiglu_epilogue_against_oracle(dev, tile):
    """H = silu(X.W_gate) * (X.W_up) from the fp32 accumulators, every tile shape: m = 72 and
    inter = 264 leave ragged row and column tiles (264 = 2 * 128 + 8)."""
    P, m, K, inter = 3, 72, 200, 264
    x = inputs.normal(7800 + tile, (P * m, K), 1.0, "bf16")
    w_gu = inputs.normal(7801 + tile, (K, 2 * inter), 0.1, "bf16")
    slices = [x[q * m:(q + 1) * m] for q in range(P)]
    for r in (0, P - 1):
        got = from_dev(_ag_swiglu(dev, x, w_gu, P, r, fo.opts(tile=tile)))
        ref = oracle.swiglu(oracle.ag(slices, w_gu, P, r))
        assert rel_frobenius(got, ref) <= TOL_BF16, f"rank {r}"
        # per element: one bf16 rounding of an fp32 result (fp32 sums over K = 200 terms)
        scale = np.sqrt(np.mean(ref ** 2))
        assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-4 * scale), f"rank {r}"


def test_swiglu_epilogue_beats_the_two_kernel_path(dev):
    """The fused H skips the rounding of Y to bf16 that the two-kernel path (fo_ag_gemm, then
    fo_swiglu) takes: both near the exact H, the fused one nearer."""
    P, m, K, inter = 2, 256, 512, 512
    x = inputs.normal(7820, (P * m, K), 1.0, "bf16")
    w_gu = inputs.normal(7821, (K, 2 * inter), 0.05, "bf16")
    r = 1
    fused = from_dev(_ag_swiglu(dev, x, w_gu, P, r, fo.opts()))
    slices = [to_dev(x[q * m:(q + 1) * m], dev) for q in range(P)]
    x_recv = torch.empty((P * m, K), dtype=torch.bfloat16, device=dev)
    y = torch.empty((P * m, 2 * inter), dtype=torch.bfloat16, device=dev)
    h = torch.empty((P * m, inter), dtype=torch.bfloat16, device=dev)
    s = _stream()
    fo.ag_gemm(slices[r], slices, x_recv, to_dev(w_gu, dev), y, P, r, compute_stream=s)
    fo.swiglu(y, h, stream=s)
    fo.check(s)
    exact = oracle.swiglu(oracle.ag([x[q * m:(q + 1) * m] for q in range(P)], w_gu, P, r))
    e_fused, e_two = rel_frobenius(fused, exact), rel_frobenius(from_dev(h), exact)
    assert e_fused <= TOL_BF16 and e_two <= 4 * TOL_BF16
    assert e_fused < e_two, (e_fused, e_two)


def test_swiglu_epilogue_l70b(dev):
    """The Llama-3.1-70B gate+up projection (8 slices of 512 x 8192, W 8192 x 7168) with the
    SwiGLU epilogue, rank 3: every entry of H against silu(gate) * up of the oracle's fp64
    projection."""
    ag = configs.L70B_AG
    P, m = ag.P, ag.m
    x, w_gu = ag.x(), ag.w()
    r = 3
    h = _ag_swiglu(dev, x, w_gu, P, r, fo.opts())
    (_, _, y), = ag_oracle_blocks(ag)
    ref = oracle.swiglu(y)
    bm, bn, _ = fo.tile_info(P, m, ag.K, ag.N)
    assert_parity(from_dev(h), ref, "bf16", (bm, bn // 2), what="70B gate+up SwiGLU, rank 3")
