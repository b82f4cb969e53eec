"""Pins for the oracle's GEMV / expert FFN / routed layer / shard partials (CPU).

Pins used (none re-types the oracle's own code):
* exact rational arithmetic (fractions.Fraction) on tiny non-square shapes:
  fp9 values and float32 inputs are dyadic rationals, so W x is exact there;
* hand-worked closed forms for a sparse expert whose output is known by eye;
* special cases that reduce to something known: every routed expert equal to
  the shared one gives (1 + sum w) * expert(x); zero routing weights leave the
  shared expert; a permutation of (id, w) pairs changes nothing; tokens do not
  interact;
* the tensor-parallel identity: the shard partials add up to the full output
  (exact in real arithmetic, because silu acts on each intermediate index).
"""

import math
from fractions import Fraction

import numpy as np
import pytest

import oracle

RNG = np.random.default_rng(2024)
FINITE_CODES = np.array([c for c in range(512) if ((c >> 3) & 31) != 31])


def rand_codes(shape, rng=RNG, scale_exp=None):
    """Random finite fp9 codes (optionally near a given binade)."""
    if scale_exp is None:
        return rng.choice(FINITE_CODES, size=shape)
    e = np.clip(rng.integers(scale_exp - 3, scale_exp + 2, size=shape), 0, 30)
    m = rng.integers(0, 8, size=shape)
    s = rng.integers(0, 2, size=shape)
    return (s << 8) | (e << 3) | m


def exact_value(code):
    """fp9 code -> Fraction, from the layout (sign bit 8, exp bits 7..3 bias 15,
    mantissa bits 2..0), written with integer arithmetic only."""
    code = int(code)
    s, e, m = code >> 8, (code >> 3) & 31, code & 7
    if e == 0:
        v = Fraction(m, 8) * Fraction(1, 2 ** 14)
    else:
        v = Fraction(8 + m, 8) * (Fraction(2) ** (e - 15))
    return -v if s else v


def exact_gemv(codes, x):
    rows, cols = codes.shape
    xf = [Fraction(float(v)) for v in x]
    return [sum((exact_value(codes[r, k]) * xf[k] for k in range(cols)), Fraction(0))
            for r in range(rows)]


@pytest.mark.parametrize("shape", [(5, 16), (3, 24), (7, 8)])
def test_gemv_exact_rational(shape):
    codes = rand_codes(shape, scale_exp=12)
    x = RNG.standard_normal(shape[1]).astype(np.float32)
    got = oracle.gemv(codes, x)
    ref = exact_gemv(codes, x)
    for g, r, row in zip(got, ref, codes):
        bound = sum(abs(exact_value(c)) for c in row) * max(abs(float(v)) for v in x)
        assert abs(Fraction(float(g)) - r) <= Fraction(shape[1] * 2.0 ** -52) * bound


def test_gemv_one_hot_is_decode():
    codes = rand_codes((6, 24))
    for k in range(24):
        x = np.zeros(24, dtype=np.float32)
        x[k] = 1.0
        np.testing.assert_array_equal(oracle.gemv(codes, x), oracle.decode(codes[:, k]))


def _code(v):
    return int(oracle.quantize(np.array([v], dtype=np.float32))[0])


def test_expert_sparse_closed_form():
    """I=4, H=8.  gate[i, i] = 1, up[i, i+4] = 2, down[j, j % 4] = 1, rest 0:
    g_i = x_i, v_i = 2 x_{i+4}, h_i = silu(x_i) * 2 x_{i+4}, y_j = h_{j % 4}."""
    I, H = 4, 8
    gate = np.zeros((I, H), dtype=np.int64)
    up = np.zeros((I, H), dtype=np.int64)
    down = np.zeros((H, I), dtype=np.int64)
    for i in range(I):
        gate[i, i] = _code(1.0)
        up[i, i + 4] = _code(2.0)
    for j in range(H):
        down[j, j % 4] = _code(1.0)
    x = np.array([1.0, -1.0, 0.0, 2.0, 0.5, 3.0, -2.0, 1.0], dtype=np.float32)
    y = oracle.expert_ffn((gate, up, down), x[None, :])[0]
    for j in range(H):
        i = j % 4
        xi, xu = float(x[i]), float(x[i + 4])
        expect = xi / (1.0 + math.exp(-xi)) * 2.0 * xu
        assert y[j] == pytest.approx(expect, rel=1e-15, abs=1e-300)
    # literal values: silu(1) * 2 * 0.5, silu(-1) * 2 * 3
    assert y[0] == pytest.approx(0.7310585786300049, rel=1e-15)
    assert y[1] == pytest.approx(-1.6136485282199706, rel=1e-15)
    # exchanging gate and up changes the answer (silu is applied to the gate)
    y_sw = oracle.expert_ffn((up, gate, down), x[None, :])[0]
    assert abs(y_sw[1] - y[1]) > 1.0   # silu(6) * -1 vs silu(-1) * 6


def test_expert_exact_rational_small():
    I, H = 6, 16
    gate = rand_codes((I, H), scale_exp=12)
    up = rand_codes((I, H), scale_exp=12)
    down = rand_codes((H, I), scale_exp=12)
    x = RNG.standard_normal(H).astype(np.float32)
    g = exact_gemv(gate, x)
    v = exact_gemv(up, x)
    h = [Fraction(float(gi) / (1.0 + math.exp(-float(gi)))) * vi for gi, vi in zip(g, v)]
    ref = [sum((exact_value(down[j, i]) * h[i] for i in range(I)), Fraction(0)) for j in range(H)]
    got = oracle.expert_ffn((gate, up, down), x[None, :])[0]
    scale = max(abs(float(r)) for r in ref)
    for a, b in zip(got, ref):
        assert abs(a - float(b)) <= 1e-13 * scale


def _tiny_layer(n_routed=12, I=16, H=24, seed=5):
    rng = np.random.default_rng(seed)
    experts = [(rand_codes((I, H), rng, 10), rand_codes((I, H), rng, 10),
                rand_codes((H, I), rng, 10)) for _ in range(n_routed + 1)]
    return experts, (lambda e: experts[e])


def _route(T, n_routed, k, rng):
    ids = np.stack([rng.choice(n_routed, size=k, replace=False) for _ in range(T)])
    z = rng.standard_normal((T, k))
    w = np.exp(z) / np.exp(z).sum(axis=1, keepdims=True)
    return ids, w.astype(np.float32)


def test_moe_all_experts_equal_gives_scaled_expert():
    experts, _ = _tiny_layer()
    same = experts[0]
    x = RNG.standard_normal((2, 24)).astype(np.float32)
    ids, w = _route(2, 12, 4, RNG)
    out = oracle.moe_layer(lambda e: same, x, ids, w, 12)
    single = oracle.expert_ffn(same, x)
    scale = 1.0 + w.astype(np.float64).sum(axis=1)
    np.testing.assert_allclose(out, single * scale[:, None], rtol=1e-12, atol=1e-12)


def test_moe_zero_weights_leave_shared_only():
    experts, get = _tiny_layer()
    x = RNG.standard_normal((1, 24)).astype(np.float32)
    ids, _ = _route(1, 12, 4, RNG)
    out = oracle.moe_layer(get, x, ids, np.zeros_like(ids, dtype=np.float32), 12)
    np.testing.assert_array_equal(out, oracle.expert_ffn(experts[12], x))


def test_moe_one_hot_weight():
    experts, get = _tiny_layer()
    x = RNG.standard_normal((1, 24)).astype(np.float32)
    ids, _ = _route(1, 12, 4, RNG)
    w = np.zeros((1, 4), dtype=np.float32)
    w[0, 2] = 1.0
    out = oracle.moe_layer(get, x, ids, w, 12)
    ref = oracle.expert_ffn(experts[12], x) + oracle.expert_ffn(experts[int(ids[0, 2])], x)
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-13)


def test_moe_permutation_and_batch_independence():
    _, get = _tiny_layer()
    x = RNG.standard_normal((2, 24)).astype(np.float32)
    ids, w = _route(2, 12, 4, RNG)
    out = oracle.moe_layer(get, x, ids, w, 12)
    perm = RNG.permutation(4)
    out_p = oracle.moe_layer(get, x, ids[:, perm], w[:, perm], 12)
    np.testing.assert_allclose(out, out_p, rtol=1e-13, atol=1e-13)
    for t in range(2):
        one = oracle.moe_layer(get, x[t:t + 1], ids[t:t + 1], w[t:t + 1], 12)
        np.testing.assert_array_equal(one[0], out[t])


def test_moe_rejects_bad_ids():
    _, get = _tiny_layer()
    x = RNG.standard_normal((1, 24)).astype(np.float32)
    with pytest.raises(ValueError):
        oracle.moe_layer(get, x, np.array([[0, 12, 3, 4]]), np.ones((1, 4)), 12)


@pytest.mark.parametrize("n_shards", [1, 2, 4, 8, 16])
def test_partials_sum_to_full(n_shards):
    _, get = _tiny_layer()
    x = RNG.standard_normal((2, 24)).astype(np.float32)
    ids, w = _route(2, 12, 4, RNG)
    full = oracle.moe_layer(get, x, ids, w, 12)
    parts = oracle.moe_partials(get, x, ids, w, 12, n_shards)
    assert parts.shape == (n_shards, 2, 24)
    np.testing.assert_allclose(parts.sum(axis=0), full, rtol=1e-12, atol=1e-12 * np.abs(full).max())
    if n_shards == 1:
        np.testing.assert_array_equal(parts[0], full)


def test_partial_is_the_slice_computation():
    """Shard r of a single-expert 'layer' equals the expert computed with only
    the slice's gate/up rows and down columns (the slice taken by hand)."""
    experts, _ = _tiny_layer()
    e = experts[3]
    x = RNG.standard_normal((1, 24)).astype(np.float32)
    parts = oracle.moe_partials(lambda _: e, x, np.zeros((1, 0), dtype=np.int64),
                                np.zeros((1, 0)), 12, 4)
    for r in range(4):
        sl = slice(4 * r, 4 * r + 4)
        sub = (e[0][sl], e[1][sl], e[2][:, sl])
        np.testing.assert_allclose(parts[r], oracle.expert_ffn(sub, x), rtol=1e-14, atol=1e-300)


def test_plan_union_ascending_shared_last():
    ids = np.array([[5, 3, 9], [3, 7, 1]])
    assert oracle.moe_plan(ids, 10) == [1, 3, 5, 7, 9, 10]
    w = np.array([[0.5, 0.25, 0.25], [0.125, 0.375, 0.5]])
    sw = oracle.moe_slot_weights(ids, w, 10)
    assert sw.shape == (6, 2)
    np.testing.assert_array_equal(sw[:, 0], [0, 0.25, 0.5, 0, 0.25, 1])
    np.testing.assert_array_equal(sw[:, 1], [0.5, 0.125, 0, 0.375, 0, 1])
    # a token listing an id twice: weights add (the layer sums over the list)
    sw2 = oracle.moe_slot_weights(np.array([[2, 2]]), np.array([[0.25, 0.5]]), 4)
    np.testing.assert_array_equal(sw2[:, 0], [0.75, 1.0])


def test_rms_normalize():
    v = RNG.standard_normal((3, 50)) * 100
    r = oracle.rms_normalize(v)
    np.testing.assert_allclose(np.mean(r * r, axis=1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(r * np.sqrt(np.mean(v * v, axis=1, keepdims=True)), v, rtol=1e-14)


def test_rms_normalize_closed_forms():
    # (3, 4): mean square 12.5; with eps = 0.5 it becomes 13
    np.testing.assert_allclose(oracle.rms_normalize([3.0, 4.0]), [[3 / 12.5 ** 0.5, 4 / 12.5 ** 0.5]],
                               rtol=1e-15)
    np.testing.assert_allclose(oracle.rms_normalize([3.0, 4.0], eps=0.5),
                               [[3 / 13 ** 0.5, 4 / 13 ** 0.5]], rtol=1e-15)
    # a constant row c maps to c / sqrt(c^2 + eps): +-1 without eps
    np.testing.assert_array_equal(oracle.rms_normalize(np.full((1, 7), -2.5)), -np.ones((1, 7)))
    np.testing.assert_allclose(oracle.rms_normalize(np.full((1, 7), 2.0), eps=5.0), np.full((1, 7), 2 / 3),
                               rtol=1e-15)
    # invariant to a positive scale, odd in the sign, rows independent
    v = RNG.standard_normal((2, 33))
    np.testing.assert_allclose(oracle.rms_normalize(1024.0 * v), oracle.rms_normalize(v), rtol=1e-14)
    np.testing.assert_array_equal(oracle.rms_normalize(-v), -oracle.rms_normalize(v))
    np.testing.assert_array_equal(oracle.rms_normalize(v)[1], oracle.rms_normalize(v[1:])[0])
    # an all-zero row: 0/0 without eps, 0 with it
    with np.errstate(invalid="ignore"):
        assert np.all(np.isnan(oracle.rms_normalize(np.zeros((1, 4)))))
    np.testing.assert_array_equal(oracle.rms_normalize(np.zeros((1, 4)), eps=1e-6), np.zeros((1, 4)))
