"""GPU parity of the matrix-core decode path (3 <= T <= 8 tokens) on the cases
the random draws of test_gpu_parity.py do not reach: invalid and repeated ids,
zero routing weights, every token naming the same experts (few slots), every
id distinct (65 slots at T = 8, top-8: the largest plan, whose last slot the
down kernel finds in its second word of slot experts), the stage split and
repeated calls, each of the three ways the weight tiles load their sign bytes,
and sign planes moved off 8-byte alignment (the same outputs, bit for bit).

Bars as everywhere: f32 outputs within relative L2 <= 1e-5 and max-abs <=
1e-4 * max|ref| of the float64 oracle; the status word exact; repeated calls
bit-identical.  The layer has ragged units in both contractions (1040 =
8 * 128 + 16 hidden, 336 = 2 * 128 + 80 intermediate) and 72 routed experts so
that 64 distinct ids fit.
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
WL, H, I, E, K = 104, 1040, 336, 72, 8


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a GPU (deselect with -m 'not gpu')")
    ensure_built()
    return torch


@pytest.fixture(scope="module")
def layer(torch_dev):
    say("build matrix-core test layer", WL, H, I, E, K)
    return dm.Layer(H, I, E, K).fill_synthetic(SEED, WL, 0), OracleExperts(SEED, WL, 0, H, I)


def to_dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def call(torch, lay, x, ids, w, ws=None):
    if ws is None:
        ws = lay.workspace(x.shape[0])
    out = dm.moe_layer(lay, to_dev(torch, x), to_dev(torch, ids.astype(np.int32)),
                       to_dev(torch, w.astype(np.float32)), ws=ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), dm.status(ws)


def reference(ox, x, ids, w):
    ox.prefetch([int(i) for i in np.unique(ids) if 0 <= i < E] + [E])
    return oracle.moe_layer(ox, x, ids, w, E)


@pytest.mark.parametrize("T", [3, 8])
def test_bad_repeated_ids_and_zero_weights(torch_dev, layer, T):
    torch = torch_dev
    lay, ox = layer
    x = synth.activations(SEED, WL, 0, 10 + T, T, H)
    ids, w = synth.routing(SEED, WL, 0, 10 + T, T, E, K)
    w = w.astype(np.float32)
    ids[0, 5] = ids[0, 1]              # a repeat: the two weights add
    ids[1, 2], ids[2, 7] = -1, E + 3   # out of range: skipped
    w[T - 1] = 0.0                     # a token with zero weights: shared expert only
    say("matrix-core path T =", T, "bad, repeated ids, zero weights")
    got, st = call(torch, lay, x, ids, w)
    assert st == dm.duckmoe.STATUS_BAD_ID | dm.duckmoe.STATUS_DUP_ID
    # for the oracle a skipped id is a zero-weight repeat of the token's first id
    ref_ids, ref_w = ids.copy(), w.astype(np.float64)
    for t, i in ((1, 2), (2, 7)):
        ref_ids[t, i] = ids[t, 0]
        ref_w[t, i] = 0.0
    ref = reference(ox, x, ref_ids, ref_w)
    for t in range(T):
        check_close(got[t], ref[t], "T=%d token %d" % (T, t))


def test_every_token_same_experts(torch_dev, layer):
    torch = torch_dev
    lay, ox = layer
    T = 8
    x = synth.activations(SEED, WL, 0, 30, T, H)
    _, w = synth.routing(SEED, WL, 0, 30, T, E, K)
    ids = np.tile(np.array([3, 70, 11, 0, 45, 9, 64, 27], dtype=np.int32), (T, 1))
    say("matrix-core path, 9 slots for 8 tokens")
    got, st = call(torch, lay, x, ids, w)
    assert st == 0
    check_close(got, reference(ox, x, ids, w), "same experts")
    assert dm.moe_plan(to_dev(torch, ids), E) == [E, 3, 70, 11, 0, 45, 9, 64, 27]


def test_sixty_four_distinct_ids(torch_dev, layer):
    torch = torch_dev
    lay, ox = layer
    T = 8
    rng = np.random.default_rng(7)
    ids = rng.permutation(E)[:T * K].reshape(T, K).astype(np.int32)
    w = rng.random((T, K)).astype(np.float32)
    x = synth.activations(SEED, WL, 0, 31, T, H)
    say("matrix-core path, 65 slots")
    got, st = call(torch, lay, x, ids, w)
    assert st == 0
    plan = dm.moe_plan(to_dev(torch, ids), E)
    assert len(plan) == 65 and plan[0] == E and plan[1:] == list(ids.ravel())
    ref = reference(ox, x, ids, w)
    for t in range(T):
        check_close(got[t], ref[t], "65 slots token %d" % t)


# Sign-load modes of the unit-pair loads, by column count: 1056 and 352 have
# sign rows of whole dwords but not of 8-byte words (one dword per lane and
# unit); 1088 and 320 have 8-byte rows (one 8-byte load per lane and pair) and
# a last unit only half inside the matrix; 1152 and 640 have 8-byte rows and
# an odd number of whole units, so each row's last pair has an empty second
# unit.  (The module's 1040 / 336 layer takes two 2-byte loads per unit.)
MODE_LAYERS = {  # workload: (H, I, n_routed, top_k)
    105: (1056, 352, 24, 8),
    106: (1088, 320, 24, 8),
    107: (1152, 640, 20, 6),
}


@pytest.fixture(scope="module")
def mode_layers(torch_dev):
    out = {}
    for wl, (h, i, e, k) in MODE_LAYERS.items():
        say("build sign-mode layer", wl, (h, i, e, k))
        out[wl] = (dm.Layer(h, i, e, k).fill_synthetic(SEED, wl, 0), OracleExperts(SEED, wl, 0, h, i))
    return out


@pytest.mark.parametrize("wl", sorted(MODE_LAYERS))
@pytest.mark.parametrize("T", [3, 6, 8])
def test_sign_load_modes(torch_dev, mode_layers, wl, T):
    torch = torch_dev
    lay, ox = mode_layers[wl]
    h, _, e, k = MODE_LAYERS[wl]
    x = synth.activations(SEED, wl, 0, 40 + T, T, h)
    ids, w = synth.routing(SEED, wl, 0, 40 + T, T, e, k)
    say("matrix-core path, layer", wl, "T =", T)
    got, st = call(torch, lay, x, ids, w)
    assert st == 0
    ox.prefetch([int(i) for i in np.unique(ids)] + [e])
    ref = oracle.moe_layer(ox, x, ids, w, e)
    for t in range(T):
        check_close(got[t], ref[t], "layer %d T=%d token %d" % (wl, T, t))


def test_stage_split_and_repeat_calls(torch_dev, layer):
    torch = torch_dev
    lay, ox = layer
    T = 5
    x = synth.activations(SEED, WL, 0, 32, T, H)
    ids, w = synth.routing(SEED, WL, 0, 32, T, E, K)
    xd, idd, wd = to_dev(torch, x), to_dev(torch, ids), to_dev(torch, w.astype(np.float32))
    say("matrix-core path, stage split and repeat calls")
    ws = lay.workspace(T)
    first = dm.moe_layer(lay, xd, idd, wd, ws=ws).cpu().numpy()
    for _ in range(10):
        np.testing.assert_array_equal(first, dm.moe_layer(lay, xd, idd, wd, ws=ws).cpu().numpy())
    ws2 = lay.workspace(T)
    dm.moe_gate_up(lay, xd, idd, wd, ws2)
    split = dm.moe_down(lay, xd, idd, wd, ws2).cpu().numpy()
    np.testing.assert_array_equal(split, first)
    # down again on the same workspace: the same bits
    np.testing.assert_array_equal(dm.moe_down(lay, xd, idd, wd, ws2).cpu().numpy(), first)
    check_close(first, reference(ox, x, ids, w), "T=5")


@pytest.mark.parametrize("offset", [2, 4])
def test_sign_plane_alignment(torch_dev, offset):
    """The same layer with its sign planes moved 2 or 4 bytes past an 8-byte
    boundary: the kernels then load the sign bytes as 2-byte or dword words
    instead of 8-byte pairs, in the bsz 3-8 path and in prefill.  The decoded
    weights and the arithmetic are the same, so the outputs must be too, bit
    for bit; the aligned layer is checked against the oracle."""
    torch = torch_dev
    wl, H, I, E, K, T = 108, 1024, 512, 16, 4, 6   # even unit counts: 8-byte pairs when aligned
    say("sign-plane alignment, offset", offset)
    lay = dm.Layer(H, I, E, K).fill_synthetic(SEED, wl, 0)
    ox = OracleExperts(SEED, wl, 0, H, I)
    x = synth.activations(SEED, wl, 0, 50, T, H)
    ids, w = synth.routing(SEED, wl, 0, 50, T, E, K)
    xp = synth.activations(SEED, wl, 0, 51, 70, H)
    idp, wp = synth.routing(SEED, wl, 0, 51, 70, E, K)

    def run():
        got = dm.moe_layer(lay, to_dev(torch, x), to_dev(torch, ids), to_dev(torch, w)).cpu().numpy()
        pf = dm.moe_prefill(lay, to_dev(torch, xp), to_dev(torch, idp), to_dev(torch, wp)).cpu().numpy()
        return got, pf

    aligned = run()
    planes = []
    for name in ("gu_sign", "dn_sign"):
        src = getattr(lay, name)
        buf = torch.zeros(src.numel() + 16, dtype=torch.uint8, device="cuda")
        buf[offset:offset + src.numel()].copy_(src)
        planes.append(buf)
    saved = (lay.struct.gu_sign, lay.struct.dn_sign)
    lay.struct.gu_sign = planes[0].data_ptr() + offset
    lay.struct.dn_sign = planes[1].data_ptr() + offset
    try:
        moved = run()
    finally:
        lay.struct.gu_sign, lay.struct.dn_sign = saved
    np.testing.assert_array_equal(moved[0], aligned[0])
    np.testing.assert_array_equal(moved[1], aligned[1])
    ox.prefetch([int(i) for i in np.unique(np.concatenate([ids.ravel(), idp.ravel()]))] + [E])
    check_close(aligned[0], oracle.moe_layer(ox, x, ids, w, E), "aligned layer T=%d" % T)
    for t in (0, 35, 69):
        check_close(aligned[1][t], oracle.moe_layer(ox, xp[t:t + 1], idp[t:t + 1], wp[t:t + 1], E)[0],
                    "aligned prefill token %d" % t)


# Blocks of 32 gate/up rows scaled apart: h' is scaled per (slot, token, block
# of 32 rows) and the down pass brings the four blocks of each 128-row unit to
# the unit's common scale.  Gate and up rows scaled by s give h' near s^2 times
# the others, so within one unit blocks sit 2^-12 (exact step), 2^-18 (a
# subnormal fp16 step) and 2^-24 or less (flushed, far below the bar) under the
# largest; one block is all zero (its exponent must not set the unit's scale);
# the ragged last unit is uniformly small (the unit's own scale is large), and
# its blocks past I carry the all-zero exponent.  Token rows of x are scaled
# 2^12 and 2^-12 apart.
MIX_BLOCK_SCALE = {1: 2.0 ** -6, 2: 2.0 ** -9, 4: 0.0, 5: 2.0 ** -12, 7: 2.0 ** -3,
                   8: 2.0 ** -6, 9: 2.0 ** -6, 10: 2.0 ** -6}


@pytest.mark.parametrize("T", [3, 6, 8])
def test_h_blocks_of_mixed_magnitude(torch_dev, T):
    torch = torch_dev
    wl, E2, K2 = 105, 6, 4
    say("matrix-core path T =", T, "h' blocks of mixed magnitude")
    lay = dm.Layer(H, I, E2, K2)
    codes = {}
    for e in range(E2 + 1):
        g, u, d = (synth.weights(SEED, wl, 0, e, m, shp)
                   for m, shp in enumerate(synth.expert_shapes(H, I)))
        for b, s in MIX_BLOCK_SCALE.items():
            g[32 * b:32 * (b + 1)] *= s
            u[32 * b:32 * (b + 1)] *= s
        lay.set_expert(e, g, u, d)
        codes[e] = (oracle.quantize(g), oracle.quantize(u), oracle.quantize(d))
    x = synth.activations(SEED, wl, 0, 30 + T, T, H)
    x[0] *= 2.0 ** 12
    x[1] *= 2.0 ** -12
    ids, w = synth.routing(SEED, wl, 0, 30 + T, T, E2, K2)
    got, st = call(torch, lay, x, ids, w)
    assert st == 0
    ref = oracle.moe_layer(lambda e: codes[int(e)], x, ids, w, E2)
    for t in range(T):
        check_close(got[t], ref[t], "mixed h' blocks T=%d token %d" % (T, t))
