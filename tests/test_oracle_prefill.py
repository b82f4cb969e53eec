"""Pins of the oracle's prefill plan (per-expert token lists).

What fixes it, independently of its own loops:
* a hand-worked example with a repeated id (tests/golden/prefill_plan_example.txt);
* brute force over the set of (expert, token) pairs: every pair the batch names
  is in exactly one entry of the right list, nothing else is, lists are in
  ascending token order and the entries of each token's weights add up to
  1 + sum_i w[t, i];
* a grouped evaluation of the layer through the lists (gather the tokens of an
  expert, one matrix product per expert, scatter through tok_entry) equals the
  per-token layer of the oracle, which never sees the lists;
* degenerate cases: one token, one routed expert, every token naming the same
  expert, no routed ids at all.
"""

import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "prefill_plan_example.txt")


def read_golden():
    rec = {}
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if not line:
            continue
        key, *vals = line.split()
        rec[key] = vals
    return rec


def test_hand_worked_example():
    g = read_golden()
    ids = np.array(g["ids"], dtype=np.int64).reshape(4, 2)
    w = np.array(g["w"], dtype=np.float64).reshape(4, 2)
    off, tok, wt, te = oracle.prefill_plan(ids, w, 3)
    np.testing.assert_array_equal(off, np.array(g["offsets"], dtype=np.int64))
    np.testing.assert_array_equal(tok, np.array(g["tokens"], dtype=np.int64))
    np.testing.assert_array_equal(wt, np.array(g["weights"], dtype=np.float64))
    np.testing.assert_array_equal(te, np.array(g["tok_entry"], dtype=np.int64).reshape(4, 3))


def brute_force_check(ids, w, n_routed):
    T, K = ids.shape
    off, tok, wt, te = oracle.prefill_plan(ids, w, n_routed)
    assert off[0] == 0 and np.all(np.diff(off) >= 0) and off[-1] == len(tok) == len(wt)
    pairs = {(n_routed, t) for t in range(T)} | {(int(ids[t, i]), t) for t in range(T)
                                                  for i in range(K)}
    got = []
    for p in range(n_routed + 1):
        e = n_routed if p == 0 else p - 1
        seg = tok[off[p]:off[p + 1]]
        assert np.all(np.diff(seg) > 0), "tokens ascending, each once"
        got += [(e, int(t)) for t in seg]
    assert len(got) == len(set(got)) and set(got) == pairs
    # weights: shared 1, routed the sum over the token's positions naming e
    for p in range(n_routed + 1):
        e = n_routed if p == 0 else p - 1
        for a in range(off[p], off[p + 1]):
            t = tok[a]
            ref = 1.0 if p == 0 else sum(w[t, i] for i in range(K) if ids[t, i] == e)
            assert wt[a] == pytest.approx(ref, rel=1e-15, abs=0)
    # tok_entry: the shared entry, then the first position of each distinct id
    for t in range(T):
        assert tok[te[t, 0]] == t and te[t, 0] < off[1]
        for i in range(K):
            a = te[t, 1 + i]
            if int(ids[t, i]) in [int(v) for v in ids[t, :i]]:
                assert a == -1
            else:
                p = int(ids[t, i]) + 1
                assert off[p] <= a < off[p + 1] and tok[a] == t
    tot = np.zeros(T)
    np.add.at(tot, tok, wt)
    np.testing.assert_allclose(tot, 1.0 + w.sum(axis=1), rtol=0,
                               atol=1e-14 * (1.0 + np.abs(w).sum(axis=1)).max())
    return off, tok, wt, te


@pytest.mark.parametrize("T,K,E,dups", [(1, 8, 256, False), (37, 8, 16, False),
                                         (64, 4, 5, True), (200, 2, 64, True),
                                         (9, 1, 1, False)])
def test_brute_force_invariants(T, K, E, dups):
    rng = np.random.default_rng(T * 1000 + K * 10 + E)
    if dups:
        ids = rng.integers(0, E, size=(T, K))
    else:
        ids = np.stack([rng.choice(E, size=K, replace=False) for _ in range(T)])
    w = rng.standard_normal((T, K))
    brute_force_check(ids, w, E)


def test_every_token_on_one_expert():
    ids = np.full((50, 3), 2)
    w = np.ones((50, 3))
    off, tok, wt, te = brute_force_check(ids, w, 4)
    np.testing.assert_array_equal(np.diff(off), [50, 0, 0, 50, 0])
    assert np.all(wt[50:] == 3.0) and np.all(te[:, 2:] == -1)


def test_no_routed_ids():
    off, tok, wt, te = oracle.prefill_plan(np.zeros((3, 0), np.int64), np.zeros((3, 0)), 0)
    np.testing.assert_array_equal(off, [0, 3])
    np.testing.assert_array_equal(tok, [0, 1, 2])
    np.testing.assert_array_equal(te, [[0], [1], [2]])


def test_out_of_range_rejected():
    with pytest.raises(ValueError):
        oracle.prefill_plan(np.array([[0, 5]]), np.ones((1, 2)), 5)
    with pytest.raises(ValueError):
        oracle.prefill_plan(np.array([[-1]]), np.ones((1, 1)), 5)


def test_grouped_evaluation_equals_per_token_layer():
    """Layer output through the lists (one GEMM per expert) == per-token oracle."""
    rng = np.random.default_rng(11)
    H, I, E, K, T = 24, 16, 6, 3, 29
    finite = np.array([c for c in range(512) if ((c >> 3) & 31) != 31])
    experts = {}
    for e in range(E + 1):
        # small codes keep the products tame
        experts[e] = tuple(rng.choice(finite[(finite & 0xFF) < 0x70], size=shp)
                           for shp in ((I, H), (I, H), (H, I)))
    x = rng.standard_normal((T, H))
    ids = rng.integers(0, E, size=(T, K))          # repeats included
    w = rng.random((T, K))
    ref = oracle.moe_layer(lambda e: experts[e], x, ids, w, E)

    off, tok, wt, te = oracle.prefill_plan(ids, w, E)
    dec = lambda c: oracle.decode(c).astype(np.float64)
    y = np.zeros((len(tok), H))
    for p in range(E + 1):
        e = E if p == 0 else p - 1
        a0, a1 = off[p], off[p + 1]
        if a0 == a1:
            continue
        g, u, d = (dec(m) for m in experts[e])
        X = x[tok[a0:a1]]                          # gathered [n, H]
        G, U = X @ g.T, X @ u.T
        h = wt[a0:a1, None] * (G / (1 + np.exp(-G))) * U
        y[a0:a1] = h @ d.T
    out = np.zeros((T, H))
    for t in range(T):
        for a in te[t]:
            if a >= 0:
                out[t] += y[a]
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
