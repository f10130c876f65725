"""GPU parity at the bounds of the calls, every output element against the oracle.

- P = 1: no peer, so Flash-AG and Flash-RS reduce to the plain GEMM (nothing to receive or add).
- P = FO_MAX_P = 32: 31 peers' slices or partials, their transfers shared out over the emulated
  links, with ragged slices (m a multiple of no tile edge), a K tail (K not a multiple of the
  64-deep K step) and ragged N.
- The attention at P = 1 (one slice: no exchange at all), at P = 32 (inbound exchange only) and
  at P = 16 with the return exchange (2P = FO_MAX_P signal sets).
The sliced results also equal the unsliced GEMM bit for bit (the exactness of slicing).
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from comm_overlapped_sliced_amd import flashovl as fo, inputs
from tests.gpu_helpers import assert_parity, from_dev, to_dev
from tests.test_attn_gpu import _check, _sliced
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


AG_CASES = [(1, 200, 520, 392), (32, 37, 200, 136), (32, 72, 72, 264)]


@pytest.mark.parametrize("case", AG_CASES, ids=lambda c: "P%d_m%d_K%d_N%d" % c)
def test_ag_bounds(dev, case):
    P, m, K, N = case
    x = inputs.normal(7600 + P + m, (P * m, K), 1.0, "bf16")
    w = inputs.normal(7601 + N, (K, N), 0.02, "bf16")
    ref = oracle.gemm(x, w)
    prob = AG(x, w, P, dev)
    y_ref = torch.empty_like(prob.y)
    fo.gemm_ref(to_dev(x, dev), prob.w_d, y_ref, stream=torch.cuda.current_stream())
    unsliced = from_dev(y_ref)
    for r in sorted({0, P // 2, P - 1}):
        for resident in (False, True):
            got = prob.run(r, resident=resident)
            what = f"P{P} rank {r} resident {resident}"
            assert_parity(got, ref, what=what)
            assert np.array_equal(got, unsliced), what


RS_CASES = [(1, 200, 520, 392), (32, 37, 200, 136), (32, 72, 72, 264)]


@pytest.mark.parametrize("case", RS_CASES, ids=lambda c: "P%d_m%d_K%d_N%d" % c)
def test_rs_bounds(dev, case):
    P, m, K, N = case
    x = inputs.normal(7700 + P + m, (P * m, K), 1.0, "bf16")
    w = inputs.normal(7701 + N, (K, N), 0.02, "bf16")
    parts = [inputs.normal(7710 + q, (m, N), 1.0, "f32") for q in range(P)]
    prob = RS(x, w, parts, P, dev)
    for r in sorted({0, P // 2, P - 1}):
        for resident in (False, True):
            out, send = prob.run(r, resident=resident)
            ref_out, ref_send = oracle.rs(x, w, parts, P, r, want_send=True)
            what = f"P{P} rank {r} resident {resident}"
            assert_parity(out, ref_out, out="f32", what=what + " own chunk")
            keep = ~np.isnan(ref_send)
            assert np.all(np.isnan(send[~keep])), what + ": the own chunk is not sent"
            rows = np.flatnonzero(keep.any(axis=1))
            if rows.size:
                assert_parity(send[rows], ref_send[rows], out="f32", what=what + " send chunks")


@pytest.mark.parametrize("P,m,send", [(1, 200, False), (32, 40, False), (16, 72, True)],
                         ids=["P1", "P32_inbound", "P16_both"])
def test_attn_bounds(dev, P, m, send):
    hq, hkv = 2, 1
    qkv = inputs.normal(8300 + P, (P * m, (hq + 2 * hkv) * 128), 1.0, "bf16")
    for rank in sorted({0, P - 1}):
        out = _sliced(dev, qkv, P, rank, hq, hkv, True, send=send)
        _check(from_dev(out), qkv, hq, hkv, True, f"P{P} rank {rank}")
