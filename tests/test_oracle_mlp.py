"""Pins of the oracle's MLP-block pieces (CPU): the bf16 rounding of the activations between the
kernels and the SwiGLU activation, checked against brute force and closed forms, not against
their own formulas."""
from __future__ import annotations

import numpy as np
import pytest

import oracle


def _all_bf16():
    """Every finite bf16 value (fp64) and its bit pattern."""
    bits = np.arange(1 << 16, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        vals = (bits << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    ok = np.isfinite(vals)
    return vals[ok], bits[ok].astype(np.uint16)


def _nearest_bf16_brute(x):
    """Nearest finite bf16 by exhaustive search; ties go to the even bit pattern."""
    vals, bits = _all_bf16()
    out = np.empty(len(x), dtype=np.uint16)
    for i, xi in enumerate(x):
        d = np.abs(vals - xi)
        best = np.flatnonzero(d == d.min())
        cand = bits[best]
        if len(cand) > 1:  # a tie (or +0/-0): the even pattern, the one matching x's sign
            cand = cand[(cand & 1) == 0] if (cand & 1).min() == 0 else cand
            sign = 0x8000 if np.signbit(xi) else 0
            same = cand[(cand & 0x8000) == sign]
            cand = same if len(same) else cand
        out[i] = cand[0]
    return out


def test_round_bf16_ties_and_simple_values():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties to the even pattern 0x3F80
    x = np.array([1 + 2**-8, 1 + 3 * 2**-8, -(1 + 2**-8), 1 + 2**-8 + 2**-30, 3.0, 0.0,
                  2.0**-100, 1.0 / 3.0])
    assert list(oracle.round_bf16(x)) == [0x3F80, 0x3F82, 0xBF80, 0x3F81, 0x4040, 0x0000,
                                          0x0D80, 0x3EAB]


def test_round_bf16_brute_force():
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.normal(0, 1, 300), rng.normal(0, 1e4, 100), rng.normal(0, 1e-3, 100)])
    # exact midpoints between neighbouring bf16 values (ties) and points just off them
    vals, _ = _all_bf16()
    pos = np.sort(vals[(vals > 1e-3) & (vals < 1e3)])
    mids = (pos[:-1] + pos[1:])[rng.integers(0, len(pos) - 1, 200)] / 2
    x = np.concatenate([x, mids, np.nextafter(mids, np.inf), -mids])
    assert np.array_equal(oracle.round_bf16(x), _nearest_bf16_brute(x))


def _bits(vals):
    return (np.asarray(vals, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _enc(vals, form):
    """A y row as bf16 bits or as fp64 (the two input forms of the activation)."""
    v = np.asarray(vals, dtype=np.float32)
    return _bits(v) if form == "bf16" else v.astype(np.float64)


@pytest.mark.parametrize("form", ["bf16", "f64"])
def test_swiglu_closed_forms(form):
    g = np.array([0.0, 1.0, -1.0, 2.5, -2.5, 30.0, -30.0, 0.125], dtype=np.float32)
    ones = np.ones_like(g)
    y = np.stack([_enc(np.concatenate([g, ones]), form)])     # gate = g, up = 1
    h = oracle.swiglu(y)[0]
    assert h[0] == 0.0                                          # silu(0) = 0
    assert h[1] == pytest.approx(1.0 / (1.0 + np.exp(-1.0)), rel=1e-15)
    assert h[1] - h[2] == pytest.approx(1.0, rel=1e-15)         # silu(g) - silu(-g) = g
    assert h[3] - h[4] == pytest.approx(2.5, rel=1e-15)
    assert h[5] == pytest.approx(30.0, rel=1e-12) and abs(h[6]) < 1e-11
    # the up half multiplies: gate = 1, up = v gives silu(1) * v
    v = np.array([3.0, -0.5, 0.0, 8.0], dtype=np.float32)
    y2 = np.stack([_enc(np.concatenate([np.ones(4, np.float32), v]), form)])
    assert np.allclose(oracle.swiglu(y2)[0], v / (1.0 + np.exp(-1.0)), rtol=1e-15, atol=0)


def test_swiglu_halves_are_gate_then_up():
    rng = np.random.default_rng(5)
    gate = rng.normal(0, 2, (3, 16)).astype(np.float32)
    up = rng.normal(0, 1, (3, 16)).astype(np.float32)
    y = _bits(np.concatenate([gate, up], axis=1))
    gd = (y[:, :16].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ud = (y[:, 16:].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    h = oracle.swiglu(y)
    assert np.allclose(h, gd * ud / (1 + np.exp(-gd)), rtol=1e-14, atol=0)
    swapped = np.concatenate([y[:, 16:], y[:, :16]], axis=1)
    assert not np.allclose(oracle.swiglu(swapped), h)


def test_mlp_block_is_the_three_steps():
    """P = 2, tiny shapes: the block equals Flash-AG, rounding, SwiGLU, rounding and Flash-RS done
    one after the other with plain numpy for the middle steps."""
    rng = np.random.default_rng(9)
    P, m, K, inter, N = 2, 3, 8, 4, 5
    xs = [_bits(rng.normal(0, 1, (m, K))) for _ in range(P)]
    w_gu = _bits(rng.normal(0, 0.3, (K, 2 * inter)))
    w_d = _bits(rng.normal(0, 0.3, (inter, N)))
    parts = [rng.normal(0, 1, (m, N)).astype(np.float32) for _ in range(P)]
    dec = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for r in range(P):
        y = np.concatenate([dec(x) for x in xs]) @ dec(w_gu)
        yb = _nearest_bf16_brute(y.ravel()).reshape(y.shape)
        g, u = dec(yb[:, :inter]), dec(yb[:, inter:])
        hb = _nearest_bf16_brute((g / (1 + np.exp(-g)) * u).ravel()).reshape(g.shape)
        full = dec(hb) @ dec(w_d)
        expect = full[r * m:(r + 1) * m] + sum(parts[q].astype(np.float64) for q in range(P) if q != r)
        assert np.allclose(oracle.mlp_block(xs, w_gu, w_d, parts, P, r), expect, rtol=1e-12, atol=1e-12)


def test_swiglu_f64_reads_unrounded_values():
    # 1 + 2^-10 has no bf16 form: the fp64 input keeps it (silu(g) * 1 with g = 1 + 2^-10)
    g = 1 + 2.0**-10
    h = oracle.swiglu(np.array([[g, 1.0]]))[0, 0]
    assert h == pytest.approx(g / (1 + np.exp(-g)), rel=1e-15)
    assert h != pytest.approx(1 / (1 + np.exp(-1.0)), rel=1e-6)


def test_mlp_block_fused_skips_the_y_rounding():
    """fused=True: SwiGLU reads the unrounded fp64 projection, only H is rounded to bf16."""
    rng = np.random.default_rng(19)
    P, m, K, inter, N = 2, 3, 8, 4, 5
    xs = [_bits(rng.normal(0, 1, (m, K))) for _ in range(P)]
    w_gu = _bits(rng.normal(0, 0.3, (K, 2 * inter)))
    w_d = _bits(rng.normal(0, 0.3, (inter, N)))
    parts = [rng.normal(0, 1, (m, N)).astype(np.float32) for _ in range(P)]
    dec = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for r in range(P):
        y = np.concatenate([dec(x) for x in xs]) @ dec(w_gu)
        g, u = y[:, :inter], y[:, inter:]
        hb = _nearest_bf16_brute((g / (1 + np.exp(-g)) * u).ravel()).reshape(g.shape)
        full = dec(hb) @ dec(w_d)
        expect = full[r * m:(r + 1) * m] + sum(parts[q].astype(np.float64) for q in range(P) if q != r)
        got = oracle.mlp_block(xs, w_gu, w_d, parts, P, r, fused=True)
        assert np.allclose(got, expect, rtol=1e-12, atol=1e-12)
