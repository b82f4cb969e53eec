"""GPU parity of the prefill path (per-expert token lists + grouped GEMMs on the
matrix cores) against the float64 oracle.

Bars: the token lists bit-exact against oracle.prefill_plan (entries, tokens,
tok_entry; weights bit-exact where a token names an id at most twice, since one
float32 addition is correctly rounded); f32 outputs within relative L2 <= 1e-5
and max-abs <= 1e-4 * max|ref| of oracle.moe_layer, the per-token definition
that never sees the lists.  Sizes span several 64-token tiles with ragged
tails, ragged hidden and intermediate units (1040 = 8 * 128 + 16, 336 =
2 * 128 + 80) and more than one 256-row block.  The full-size case (7168/2048,
256 routed + 1 shared, T = 2048) is in test_gpu_parity.py next to the layer
it shares.
"""

import numpy as np
import pytest

import oracle
from gpu_util import OracleExperts, check_close, say
from lib_util import ensure_built

import bit_moe_expert_fp9_amd as dm
from bit_moe_expert_fp9_amd import synth

pytestmark = pytest.mark.gpu

SEED = 0


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a GPU (deselect with -m 'not gpu')")
    ensure_built()
    return torch


def to_dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


# ------------------------------------------------------------------- plan --

def check_plan(torch, ids, w, E, ref_ids=None, ref_w=None, status=0):
    T, k = ids.shape
    say("prefill plan T =", T, "k =", k, "E =", E)
    off, tok, wt, te, st = dm.prefill_plan(to_dev(torch, ids.astype(np.int32)),
                                           to_dev(torch, w.astype(np.float32)), E)
    ro, rt, rw, rte = oracle.prefill_plan(ids if ref_ids is None else ref_ids,
                                          w if ref_w is None else ref_w, E)
    np.testing.assert_array_equal(off, ro)
    np.testing.assert_array_equal(tok, rt)
    np.testing.assert_array_equal(te, rte)
    np.testing.assert_array_equal(wt, rw.astype(np.float32))
    assert st == status


def test_plan_bit_exact(torch_dev):
    torch = torch_dev
    rng = np.random.default_rng(41)
    for T, k, E in [(1, 8, 256), (7, 8, 256), (300, 8, 256), (2048, 8, 256), (517, 3, 9),
                    (64, 1, 1), (1000, 32, 1024), (5, 8, 1024), (200, 12, 64), (33, 16, 16),
                    (90, 17, 40)]:
        ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])
        w = rng.random((T, k)).astype(np.float32)
        check_plan(torch, ids, w, E)


@pytest.mark.parametrize("T,k,E,rep", [(333, 6, 11, (4, 1)), (150, 20, 40, (19, 17))])
def test_plan_repeats_and_bad_ids(torch_dev, T, k, E, rep):
    torch = torch_dev
    rng = np.random.default_rng(42)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])
    w = rng.random((T, k)).astype(np.float32)
    dup = ids.copy()
    dup[::7, rep[0]] = dup[::7, rep[1]]          # a repeat: weights add (one f32 add)
    check_plan(torch, dup, w, E, status=dm.duckmoe.STATUS_DUP_ID)
    bad = ids.copy()
    bad[5, 2], bad[100, k - 1] = -3, E + 4       # skipped: for the oracle a zero-weight
    ref_ids, ref_w = bad.copy(), w.copy()        # repeat of the token's first id
    for t, i in ((5, 2), (100, k - 1)):
        ref_ids[t, i] = ids[t, 0]
        ref_w[t, i] = 0.0
    check_plan(torch, bad, w, E, ref_ids, ref_w, status=dm.duckmoe.STATUS_BAD_ID)


def test_plan_without_ids(torch_dev):
    torch = torch_dev
    say("prefill plan, no routed ids")
    z = torch.zeros((5, 0), dtype=torch.int32, device="cuda")
    off, tok, wt, te, st = dm.prefill_plan(z, z.float(), 3)
    np.testing.assert_array_equal(off, [0, 5, 5, 5, 5])
    np.testing.assert_array_equal(tok, np.arange(5))
    assert np.all(wt == 1.0) and st == 0
    np.testing.assert_array_equal(te[:, 0], np.arange(5))


# ------------------------------------------------------------------ layers --

LAYERS = {  # workload: (H, I, n_routed, top_k)
    180: (1040, 336, 24, 8),    # ragged units in both GEMMs, 2 row blocks of gate/up
    181: (2064, 1536, 16, 4),   # 6 row blocks of gate/up, 9 of down
    182: (256, 128, 3, 2),      # every expert gets many tiles
}


@pytest.fixture(scope="module")
def layers(torch_dev):
    out = {}
    for wl, (H, I, E, K) in LAYERS.items():
        say("build prefill layer", wl, (H, I, E, K))
        out[wl] = (dm.Layer(H, I, E, K).fill_synthetic(SEED, wl, 0),
                   OracleExperts(SEED, wl, 0, H, I))
    return out


def run_prefill(torch, lay, ox, wl, step, T, ids=None, w=None, ws=None):
    x = synth.activations(SEED, wl, 0, step, T, lay.hidden)
    if ids is None:
        ids, w = synth.routing(SEED, wl, 0, step, T, lay.n_routed, lay.top_k)
    if ws is None:
        ws = lay.prefill_workspace(T)
    out = dm.moe_prefill(lay, to_dev(torch, x), to_dev(torch, ids.astype(np.int32)),
                         to_dev(torch, w.astype(np.float32)), ws=ws)
    torch.cuda.synchronize()
    return x, ids, w, out.cpu().numpy(), ws


@pytest.mark.parametrize("wl", sorted(LAYERS))
@pytest.mark.parametrize("T", [1, 9, 64, 65, 200, 333])
def test_prefill_layer(torch_dev, layers, wl, T):
    torch = torch_dev
    lay, ox = layers[wl]
    say("prefill layer", wl, "T =", T)
    x, ids, w, got, ws = run_prefill(torch, lay, ox, wl, 300 + T, T)
    assert dm.status(ws) == 0
    ox.prefetch(list(np.unique(ids)) + [lay.n_routed])
    ref = oracle.moe_layer(ox, x, ids, w, lay.n_routed)
    for t in range(T):
        check_close(got[t], ref[t], "prefill wl %d T=%d token %d" % (wl, T, t))


def test_prefill_repeats_bad_ids_and_zero_weights(torch_dev, layers):
    torch = torch_dev
    lay, ox = layers[180]
    E, T = lay.n_routed, 150
    ids, w = synth.routing(SEED, 180, 0, 9, T, E, lay.top_k)
    w = w.astype(np.float32)
    ids[::5, 6] = ids[::5, 2]                    # repeats
    ids[3, 1], ids[77, 7], ids[120, 0] = E, -1, E + 9   # out of range
    w[10] = 0.0                                  # a token with zero routing weights
    say("prefill with repeats, bad ids, zero weights")
    x, _, _, got, ws = run_prefill(torch, lay, ox, 180, 9, T, ids, w)
    assert dm.status(ws) == dm.duckmoe.STATUS_BAD_ID | dm.duckmoe.STATUS_DUP_ID
    ref_ids, ref_w = ids.copy(), w.astype(np.float64)
    for t, i, r in ((3, 1, 0), (77, 7, 0), (120, 0, 1)):
        ref_ids[t, i] = ids[t, r]
        ref_w[t, i] = 0.0
    ox.prefetch(list(np.unique(ref_ids)) + [E])
    ref = oracle.moe_layer(ox, x, ref_ids, ref_w, E)
    for t in range(T):
        check_close(got[t], ref[t], "prefill repeats/bad token %d" % t)
    # a clean call on the same workspace clears the status word
    run_prefill(torch, lay, ox, 180, 10, T, ws=ws)
    assert dm.status(ws) == 0


def test_prefill_shared_only_and_dense(torch_dev, layers):
    """ids None: the shared expert alone (routed layer) and a dense MLP
    (n_routed = 0); both equal oracle.expert_ffn of that expert."""
    torch = torch_dev
    lay, ox = layers[181]
    T = 77
    x = synth.activations(SEED, 181, 0, 21, T, lay.hidden)
    say("prefill shared expert only")
    got = dm.moe_prefill(lay, to_dev(torch, x), None, None).cpu().numpy()
    ox.prefetch([lay.n_routed])
    ref = oracle.expert_ffn(ox(lay.n_routed), x)
    for t in range(T):
        check_close(got[t], ref[t], "shared only token %d" % t)
    H, I = 1040, 2064
    dense = dm.Layer(H, I, 0, 1).fill_synthetic(SEED, 183, 0)
    odx = OracleExperts(SEED, 183, 0, H, I)
    xd = synth.activations(SEED, 183, 0, 1, 100, H)
    say("prefill dense MLP", H, I)
    got = dm.moe_prefill(dense, to_dev(torch, xd), None, None).cpu().numpy()
    ref = oracle.expert_ffn(odx(0), xd)
    for t in range(100):
        check_close(got[t], ref[t], "dense token %d" % t)


def test_prefill_repeat_calls_bit_identical(torch_dev, layers):
    torch = torch_dev
    lay, _ = layers[181]
    T = 300
    x = to_dev(torch, synth.activations(SEED, 181, 0, 5, T, lay.hidden))
    ids, w = synth.routing(SEED, 181, 0, 5, T, lay.n_routed, lay.top_k)
    idd, wd = to_dev(torch, ids.astype(np.int32)), to_dev(torch, w.astype(np.float32))
    say("prefill repeat calls")
    ws = lay.prefill_workspace(T)
    first = dm.moe_prefill(lay, x, idd, wd, ws=ws).cpu().numpy()
    for _ in range(10):
        np.testing.assert_array_equal(first, dm.moe_prefill(lay, x, idd, wd, ws=ws).cpu().numpy())


def test_prefill_matches_decode_path(torch_dev, layers):
    """At T <= 8 both paths run: they agree within the f32 bar."""
    torch = torch_dev
    lay, _ = layers[180]
    for T in (1, 2, 8):
        say("prefill vs decode T =", T)
        x = to_dev(torch, synth.activations(SEED, 180, 0, 40 + T, T, lay.hidden))
        ids, w = synth.routing(SEED, 180, 0, 40 + T, T, lay.n_routed, lay.top_k)
        idd, wd = to_dev(torch, ids.astype(np.int32)), to_dev(torch, w.astype(np.float32))
        a = dm.moe_prefill(lay, x, idd, wd).cpu().numpy()
        b = dm.moe_layer(lay, x, idd, wd).cpu().numpy()
        for t in range(T):
            check_close(a[t], b[t], "prefill vs decode T=%d token %d" % (T, t))


@pytest.mark.parametrize("T", [144, 147, 216, 219])
def test_prefill_tile_size_boundaries(torch_dev, layers, T):
    """The call cuts its lists into 96-entry tiles when the routed lists average
    49 to 72 entries, else 64: with 24 experts and top-8 that is T = 147 .. 218.
    Both sides of both boundaries against the oracle (every 7th token and the
    last)."""
    torch = torch_dev
    lay, ox = layers[180]
    say("prefill tile-size boundary T =", T)
    x, ids, w, got, ws = run_prefill(torch, lay, ox, 180, 500 + T, T)
    assert dm.status(ws) == 0
    toks = sorted(set(range(0, T, 7)) | {T - 1})
    ox.prefetch(list(np.unique(ids[toks])) + [lay.n_routed])
    ref = oracle.moe_layer(ox, x[toks], ids[toks], w[toks], lay.n_routed)
    for i, t in enumerate(toks):
        check_close(got[t], ref[i], "tile boundary T=%d token %d" % (T, t))


def test_prefill_largest_batch(torch_dev):
    """T = 32768 (the call's limit) on a small layer: sampled tokens against the
    oracle (tokens at tile edges, the first and the last)."""
    torch = torch_dev
    H, I, E, K, T = 128, 64, 6, 2, 32768
    lay = dm.Layer(H, I, E, K).fill_synthetic(SEED, 184, 0)
    ox = OracleExperts(SEED, 184, 0, H, I)
    x = synth.activations(SEED, 184, 0, 0, T, H)
    ids, w = synth.routing(SEED, 184, 0, 0, T, E, K)
    say("prefill T = 32768")
    got = dm.moe_prefill(lay, to_dev(torch, x), to_dev(torch, ids.astype(np.int32)),
                         to_dev(torch, w.astype(np.float32))).cpu().numpy()
    assert np.all(np.isfinite(got))
    toks = [0, 1, 63, 64, 4097, 20000, T - 1]
    ox.prefetch(list(range(E + 1)))
    ref = oracle.moe_layer(ox, x[toks], ids[toks], w[toks], E)
    for i, t in enumerate(toks):
        check_close(got[t], ref[i], "T=32768 token %d" % t)
