"""Pins of the oracle's attention (CPU): closed forms and invariants that fix what scaled
dot-product attention computes, so that a dropped scale, a wrong key-head mapping, a missing
causal mask or a softmax over the wrong axis fails one of them."""
from __future__ import annotations

import os

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

D = 128


def _bits(vals):
    return (np.asarray(vals, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _dec(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _qkv(q, k, v):
    """Token rows [query heads | key heads | value heads] from [S, hq, D], [S, hkv, D] arrays."""
    S = q.shape[0]
    return _bits(np.concatenate([q.reshape(S, -1), k.reshape(S, -1), v.reshape(S, -1)], axis=1))


def _rand(rng, S, hq, hkv, sd=1.0):
    return (rng.normal(0, sd, (S, hq, D)), rng.normal(0, sd, (S, hkv, D)),
            rng.normal(0, 1, (S, hkv, D)))


def pin_zero_queries_average_the_values(orc):
    # q = 0: every score is 0, the softmax is uniform over the keys a query sees
    rng = np.random.default_rng(1)
    S, hq, hkv = 9, 2, 1
    _, k, v = _rand(rng, S, hq, hkv)
    qkv = _qkv(np.zeros((S, hq, D)), k, v)
    vd = _dec(qkv[:, (hq + hkv) * D:]).reshape(S, hkv, D)[:, 0]
    for causal in (True, False):
        out = orc.attn(qkv, hq, hkv, causal)
        expect = np.cumsum(vd, axis=0) / np.arange(1, S + 1)[:, None] if causal else \
            np.broadcast_to(vd.mean(axis=0), (S, D))
        for h in range(hq):
            assert np.allclose(out[:, h * D:(h + 1) * D], expect, rtol=1e-13, atol=1e-13)


def pin_single_key_returns_its_value(orc):
    rng = np.random.default_rng(2)
    q, k, v = _rand(rng, 1, 4, 2)
    qkv = _qkv(q, k, v)
    out = orc.attn(qkv, 4, 2, True)
    vd = _dec(qkv[:, 6 * D:]).reshape(2, D)
    for h in range(4):
        assert np.array_equal(out[0, h * D:(h + 1) * D], vd[h // 2])


def pin_two_keys_are_a_logistic_of_the_scaled_score_gap(orc):
    # two keys: the weight of key 1 is sigmoid(s1 - s0), with s = q.k / sqrt(D)
    rng = np.random.default_rng(3)
    q, k, v = _rand(rng, 2, 1, 1)
    qkv = _qkv(q, k, v)
    qd, kd = _dec(qkv[1, :D]), _dec(qkv[:, D:2 * D])
    vd = _dec(qkv[:, 2 * D:])
    gap = (qd @ kd[1] - qd @ kd[0]) / np.sqrt(D)
    w1 = 1.0 / (1.0 + np.exp(-gap))
    out = orc.attn(qkv, 1, 1, True)
    assert np.allclose(out[1], (1 - w1) * vd[0] + w1 * vd[1], rtol=1e-12, atol=1e-12)
    assert np.array_equal(out[0], vd[0])  # causal: query 0 sees key 0 only


def pin_a_dominant_score_selects_its_value(orc):
    # every query is 64 e_0 and only key t has a non-zero first entry (64): its score is
    # 4096 / sqrt(128) = 362 against 0 for the others, so the softmax is one-hot on key t
    S, t = 6, 3
    q = np.zeros((S, 1, D)); q[:, 0, 0] = 64.0
    k = np.zeros((S, 1, D)); k[t, 0, 0] = 64.0   # scores 0 except key t: 4096/sqrt(128) = 362
    rng = np.random.default_rng(4)
    v = rng.normal(0, 1, (S, 1, D))
    qkv = _qkv(q, k, v)
    out = orc.attn(qkv, 1, 1, False)
    assert np.allclose(out, np.broadcast_to(_dec(qkv[t, 2 * D:]), (S, D)), rtol=0, atol=1e-12)


def pin_query_heads_map_to_their_key_head_group(orc):
    # hq = 6, hkv = 3: heads 2g and 2g+1 read key/value head g. Values of head g are all g + 1,
    # so any weights give g + 1.
    rng = np.random.default_rng(5)
    S, hq, hkv = 5, 6, 3
    q, k, _ = _rand(rng, S, hq, hkv)
    v = np.broadcast_to(np.arange(1, hkv + 1, dtype=np.float64)[None, :, None], (S, hkv, D))
    out = orc.attn(_qkv(q, k, v), hq, hkv, True)
    for h in range(hq):
        assert np.allclose(out[:, h * D:(h + 1) * D], h // 2 + 1, rtol=1e-14, atol=0)


def pin_scale_is_one_over_sqrt_head_dim(orc):
    # query 1 scores x = 8 * 1.5 = 12 against key 1 and 0 against key 0; with v_0 = 0 and v_1 = 1
    # the output is the weight of key 1, sigmoid(x / sqrt(128)): any other scale gives another value
    S = 2
    q = np.zeros((S, 1, D)); q[1, 0, 0] = 8.0
    k = np.zeros((S, 1, D)); k[1, 0, 0] = 1.5
    v = np.zeros((S, 1, D)); v[1, 0, :] = 1.0
    out = orc.attn(_qkv(q, k, v), 1, 1, True)
    x = 8.0 * 1.5
    assert out[1, 0] == pytest.approx(1.0 / (1.0 + np.exp(-x / np.sqrt(128))), rel=1e-14)


def pin_causal_rows_ignore_later_keys_and_noncausal_ignore_key_order(orc):
    rng = np.random.default_rng(6)
    S, hq, hkv = 8, 2, 2
    q, k, v = _rand(rng, S, hq, hkv)
    base = orc.attn(_qkv(q, k, v), hq, hkv, True)
    k2, v2 = k.copy(), v.copy()
    k2[5:] += 3.0
    v2[5:] -= 2.0
    changed = orc.attn(_qkv(q, k2, v2), hq, hkv, True)
    assert np.array_equal(base[:5], changed[:5]) and not np.allclose(base[5:], changed[5:])
    # non-causal: permuting the keys (with their values) leaves every row unchanged
    perm = rng.permutation(S)
    full = orc.attn(_qkv(q, k, v), hq, hkv, False)
    pq = orc.attn(_qkv(q, k[perm], v[perm]), hq, hkv, False)
    assert np.allclose(full, pq, rtol=1e-12, atol=1e-12)


def pin_selected_rows_equal_the_full_result(orc):
    rng = np.random.default_rng(7)
    S, hq, hkv = 11, 2, 1
    qkv = _qkv(*_rand(rng, S, hq, hkv))
    full = orc.attn(qkv, hq, hkv, True)
    rows = np.array([10, 0, 4])
    assert np.array_equal(orc.attn(qkv, hq, hkv, True, rows=rows), full[rows])


PINS = [pin_zero_queries_average_the_values, pin_single_key_returns_its_value,
        pin_two_keys_are_a_logistic_of_the_scaled_score_gap, pin_a_dominant_score_selects_its_value,
        pin_query_heads_map_to_their_key_head_group, pin_scale_is_one_over_sqrt_head_dim,
        pin_causal_rows_ignore_later_keys_and_noncausal_ignore_key_order,
        pin_selected_rows_equal_the_full_result]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__[4:])
def test_pin(pin):
    pin(oracle.default())


# planted mistakes in a patched copy of oracle.c: each must fail at least one pin
MUTANTS = [
    ("attn drops the 1/sqrt(d) scale", "const double scale = 1.0 / sqrt((double)d);",
     "const double scale = 1.0;"),
    ("attn maps query heads modulo the key heads", "const int g = h / (hq / hkv);",
     "const int g = h % hkv;"),
    ("attn causal mask lets a query see the next key", "const int64_t nk = causal ? i + 1 : S;",
     "const int64_t nk = causal ? (i + 2 < S ? i + 2 : S) : S;"),
    ("attn causal mask hides the query's own key", "const int64_t nk = causal ? i + 1 : S;",
     "const int64_t nk = causal ? (i > 0 ? i : 1) : S;"),
    ("attn reads values from the key heads", "qkv + j * W + (int64_t)(hq + hkv + g) * d;",
     "qkv + j * W + (int64_t)(hq + g) * d;"),
    ("attn skips the normalization", "for (int e = 0; e < d; ++e) o[e] /= den;", "(void)den;"),
    ("attn uses the wrong query row", "const uint16_t* q = qkv + i * W + (int64_t)h * d;",
     "const uint16_t* q = qkv + (i > 0 ? i - 1 : 0) * W + (int64_t)h * d;"),
]


@pytest.mark.parametrize("desc,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, desc, old, new):
    src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    assert src.count(old) == 1, f"mutation anchor for '{desc}' not found once in oracle.c"
    mutant_c = tmp_path / "mutant.c"
    mutant_c.write_text(src.replace(old, new))
    lib = str(tmp_path / "libmutant_attn.so")
    oracle.build(force=True, src=str(mutant_c), out=lib)
    orc = oracle.Oracle(lib)
    failed = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(orc)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin caught: {desc}"
