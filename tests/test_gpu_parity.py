"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bars: bit-exact for decode, packing and the expert-selection plan; relative
L2 <= 1e-5 and max-abs <= 1e-4 * max|ref| for f32 outputs.  Inputs are the
seeded synthetic draws of bit_moe_expert_fp9_amd.synth; the oracle quantizes
them itself.  Workloads: 1 = single fp9 GEMV 256x512; 2 = one SwiGLU expert
(7168/2048); 3 = routed layer, 256 experts + shared, bsz 1; 4 = the same layer
at bsz 2 plus 32 shard partials; small layers (ragged chunks, all T) use
workload ids >= 100.
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


# ------------------------------------------------------------ decode / gemv --

def test_decode_all_codes_bit_exact(torch_dev):
    torch = torch_dev
    say("decode all 512 codes")
    codes = np.arange(512).reshape(1, 512)
    body, sign = oracle.pack(codes)
    out = dm.decode_fp9(to_dev(torch, body.reshape(-1)), to_dev(torch, sign.reshape(-1)), 512)
    got = out.cpu().numpy()
    ref = oracle.decode(codes.reshape(-1))
    fin = np.isfinite(ref)
    # bit-exact for every finite code and the infinities (sign of zero included)
    np.testing.assert_array_equal(got[fin].view(np.uint32),
                                  ref[fin].astype(np.float32).view(np.uint32))
    inf = np.isinf(ref)
    np.testing.assert_array_equal(got[inf], ref[inf].astype(np.float32))
    assert np.all(np.isnan(got[np.isnan(ref)]))


def test_decode_ragged_length(torch_dev):
    torch = torch_dev
    rng = np.random.default_rng(3)
    for n in (1, 7, 9, 1000, 4093):
        say("decode ragged n =", n)
        codes = rng.integers(0, 512, size=((n + 7) // 8) * 8)
        codes[n:] = 0
        codes = np.where(((codes >> 3) & 31) == 31, codes & ~0x80, codes)  # finite codes
        body, sign = oracle.pack(codes.reshape(1, -1))
        out = torch.full((n + 5,), 7.0, device="cuda")
        dm.decode_fp9(to_dev(torch, body.reshape(-1)[:n]), to_dev(torch, sign.reshape(-1)),
                      n, out=out)
        got = out.cpu().numpy()
        np.testing.assert_array_equal(got[:n].view(np.uint32),
                                      oracle.decode(codes[:n]).astype(np.float32).view(np.uint32))
        assert np.all(got[n:] == 7.0)  # nothing written past n


def test_gemv_single_fp9_matrix(torch_dev):
    """One fp9 GEMV: W 256x512 ~ N(0, 0.02) in fp9, x ~ N(0, 1)."""
    torch = torch_dev
    say("gemv 256x512")
    W = synth.weights(SEED, 1, 0, 0, 0, (256, 512))
    x = synth.activations(SEED, 1, 0, 0, 1, 512)[0]
    body, sign = dm.quantize_fp9(W)
    codes = oracle.quantize(W)
    ob, os_ = oracle.pack(codes)
    np.testing.assert_array_equal(body, ob)       # packing bit-exact
    np.testing.assert_array_equal(sign, os_)
    y = dm.gemv_fp9(to_dev(torch, body), to_dev(torch, sign), to_dev(torch, x))
    check_close(y.cpu().numpy(), oracle.gemv(codes, x), "gemv 256x512")


def test_gemv_one_hot_columns_exact(torch_dev):
    """With x = e_k the GEMV returns column k exactly: the in-kernel decode and
    the f16-operand FMA reproduce every weight, subnormals included.  (Values,
    not bits: the output is a sum, and -0 * 1 + 0 is +0; the sign of zero is
    pinned by the decode test.)"""
    torch = torch_dev
    say("gemv one-hot columns")
    codes = np.arange(512)
    codes = codes[((codes >> 3) & 31) != 31]          # 496 finite codes
    codes = np.concatenate([codes, codes[:16]]).reshape(8, 64)  # 8 rows x 64 cols
    body, sign = oracle.pack(codes)
    db, ds = to_dev(torch, body), to_dev(torch, sign)
    for k in range(64):
        x = np.zeros(64, dtype=np.float32)
        x[k] = 1.0
        y = dm.gemv_fp9(db, ds, to_dev(torch, x)).cpu().numpy()
        np.testing.assert_array_equal(y, oracle.decode(codes[:, k]).astype(np.float32))


def test_gemv_ragged_shapes(torch_dev):
    torch = torch_dev
    rng = np.random.default_rng(11)
    for rows, cols in [(1, 8), (5, 24), (37, 72), (130, 1032)]:
        say("gemv ragged", rows, cols)
        W = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
        x = rng.standard_normal(cols).astype(np.float32)
        body, sign = dm.quantize_fp9(W)
        y = dm.gemv_fp9(to_dev(torch, body), to_dev(torch, sign), to_dev(torch, x))
        check_close(y.cpu().numpy(), oracle.gemv(oracle.quantize(W), x), "gemv %dx%d" % (rows, cols))


# ------------------------------------------------------------- small layers --

SMALL = [
    # (workload, H, I, n_routed, top_k): ragged last chunk in both GEMVs
    (100, 1040, 336, 24, 8),
    (101, 2064, 1536, 16, 4),
    # power-of-two intermediate sizes below one chunk per shard (shard slices of
    # 64..512 columns), ragged hidden chunk
    (102, 1040, 512, 20, 8),
    (103, 2064, 1024, 12, 6),
]


@pytest.fixture(scope="module")
def small_layers(torch_dev):
    out = {}
    for wl, H, I, E, k in SMALL:
        say("build small layer", wl, H, I, E, k)
        lay = dm.Layer(H, I, E, k).fill_synthetic(SEED, wl, 0)
        out[wl] = (lay, OracleExperts(SEED, wl, 0, H, I))
    return out


def expected_status(ids, n_routed):
    """The status bits a layer call must report for these ids."""
    st = 0
    for row in np.asarray(ids):
        valid = [int(i) for i in row if 0 <= i < n_routed]
        if len(valid) < len(row):
            st |= dm.duckmoe.STATUS_BAD_ID
        if len(set(valid)) < len(valid):
            st |= dm.duckmoe.STATUS_DUP_ID
    return st


def run_layer_case(torch, lay, ox, wl, step, T, n_shards=1, ids=None, w=None):
    H = lay.hidden
    x = synth.activations(SEED, wl, 0, step, T, H)
    if ids is None:
        ids, w = synth.routing(SEED, wl, 0, step, T, lay.n_routed, lay.top_k)
    valid = ids[(ids >= 0) & (ids < lay.n_routed)]
    ox.prefetch(list(valid) + [lay.n_routed])
    ws = lay.workspace(T, n_shards)
    out = dm.moe_layer(lay, to_dev(torch, x), to_dev(torch, ids.astype(np.int32)),
                       to_dev(torch, w.astype(np.float32)), n_shards=n_shards, ws=ws)
    torch.cuda.synchronize()
    assert dm.status(ws) == expected_status(ids, lay.n_routed)
    return x, ids, w, out.cpu().numpy()


@pytest.mark.parametrize("wl", [100, 101, 102, 103])
@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 6, 7, 8])
def test_small_layer_all_batch_sizes(torch_dev, small_layers, wl, T):
    torch = torch_dev
    lay, ox = small_layers[wl]
    if T * lay.top_k > 64:
        pytest.skip("T * top_k above the 64-id limit")
    say("small layer", wl, "T =", T)
    x, ids, w, got = run_layer_case(torch, lay, ox, wl, T, T)
    ref = oracle.moe_layer(ox, x, ids, w, lay.n_routed)
    check_close(got, ref, "layer %d T=%d" % (wl, T))


@pytest.mark.parametrize("n_shards", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("T", [1, 2])
def test_small_layer_pow2_shards(torch_dev, small_layers, n_shards, T):
    """I = 1024: shard slices of 1024 down to 64 columns, each reduced by lane
    groups as wide as the slice."""
    torch = torch_dev
    lay, ox = small_layers[103]
    say("I=1024 layer, T =", T, "n_shards =", n_shards)
    ws = lay.workspace(T, n_shards)
    x = synth.activations(SEED, 103, 0, 300 + n_shards, T, lay.hidden)
    ids, w = synth.routing(SEED, 103, 0, 300 + n_shards, T, lay.n_routed, lay.top_k)
    ox.prefetch(list(ids.ravel()) + [lay.n_routed])
    for rep in range(2):  # the second call reuses the workspace
        got = dm.moe_layer(lay, to_dev(torch, x), to_dev(torch, ids), to_dev(torch, w),
                           n_shards=n_shards, ws=ws).cpu().numpy()
        assert dm.status(ws) == 0
        if n_shards == 1:
            check_close(got, oracle.moe_layer(ox, x, ids, w, lay.n_routed), "I=1024 T=%d" % T)
        else:
            ref = oracle.moe_partials(ox, x, ids, w, lay.n_routed, n_shards)
            for r in range(n_shards):
                check_close(got[r], ref[r], "I=1024 shard %d/%d" % (r, n_shards))


@pytest.mark.parametrize("n_shards", [2, 3, 6, 12, 24])
def test_small_layer_shard_partials(torch_dev, small_layers, n_shards):
    """I = 1536: slices of 768 (n=2) straddle the 1024-chunk boundary are not
    allowed; 512/256/128/64-wide slices are."""
    torch = torch_dev
    lay, ox = small_layers[101]
    if dm.duckmoe.lib().duckmoe_workspace_bytes(
            __import__("ctypes").byref(lay.struct), 2, n_shards) == 0:
        with pytest.raises(dm.DuckMoeError):
            run_layer_case(torch, lay, ox, 101, 50, 2, n_shards=n_shards)
        return
    say("small layer partials n_shards =", n_shards)
    x, ids, w, got = run_layer_case(torch, lay, ox, 101, 50 + n_shards, 2, n_shards=n_shards)
    ref = oracle.moe_partials(ox, x, ids, w, lay.n_routed, n_shards)
    full = oracle.moe_layer(ox, x, ids, w, lay.n_routed)
    for r in range(n_shards):
        check_close(got[r], ref[r], "shard %d/%d" % (r, n_shards))
    check_close(got.sum(axis=0), full, "sum of %d partials" % n_shards)


@pytest.mark.parametrize("wl, T, n_shards", [
    (100, 1, 1), (100, 2, 1), (101, 1, 1), (101, 2, 1), (102, 2, 4), (103, 5, 2), (103, 8, 16)])
def test_small_expert_ffn(torch_dev, small_layers, wl, T, n_shards):
    """One expert per call (its gate/up rows split between wave pairs when the
    rows are fewer than half the waves): the routed expert 3 and the shared
    expert against the oracle, hidden sizes of 2 and 3 chunks with ragged last
    chunks, one to eight tokens, plain and as shard partials; a repeat call is
    bit-identical."""
    torch = torch_dev
    lay, ox = small_layers[wl]
    x = synth.activations(SEED, wl, 0, 700 + T, T, lay.hidden)
    for e in (3, lay.n_routed):
        say("small expert_ffn", wl, "expert", e, "T =", T, "n_shards =", n_shards)
        ox.prefetch([e])
        ws = lay.workspace(T, n_shards)
        got = dm.expert_ffn(lay, e, to_dev(torch, x), n_shards=n_shards, ws=ws).cpu().numpy()
        again = dm.expert_ffn(lay, e, to_dev(torch, x), n_shards=n_shards, ws=ws).cpu().numpy()
        np.testing.assert_array_equal(got, again)
        if n_shards == 1:
            check_close(got, oracle.expert_ffn(ox(e), x), "expert %d T=%d" % (e, T))
        else:
            ref = oracle.moe_partials(lambda _: ox(e), x, np.zeros((T, 0), np.int64),
                                      np.zeros((T, 0)), lay.n_routed, n_shards)
            for r in range(n_shards):
                check_close(got[r], ref[r], "expert %d shard %d/%d" % (e, r, n_shards))


def first_appearance(ids, n_routed):
    """Distinct valid ids in order of first appearance (token-major)."""
    seen = []
    for i in np.asarray(ids).ravel():
        if 0 <= i < n_routed and int(i) not in seen:
            seen.append(int(i))
    return seen


def test_plan_bit_exact(torch_dev):
    """The device plan names the oracle's experts, each once, in the documented
    slot order: the shared expert, then the routed ids by first appearance."""
    torch = torch_dev
    rng = np.random.default_rng(17)
    for T, k, E in [(1, 8, 256), (2, 8, 256), (8, 8, 256), (3, 5, 7), (8, 8, 8192), (1, 1, 1)]:
        say("plan", T, k, E)
        ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
        got = dm.moe_plan(to_dev(torch, ids), E)
        ref = oracle.moe_plan(ids, E)  # ascending routed ids, shared last
        assert got[0] == E
        assert sorted(got[1:]) == ref[:-1]
        assert got[1:] == first_appearance(ids, E)
    # overlapping sets across tokens: the union is streamed once
    ids = np.array([[5, 3, 9, 1], [3, 7, 1, 0]], dtype=np.int32)
    assert dm.moe_plan(to_dev(torch, ids), 10) == [10, 5, 3, 9, 1, 7, 0]
    # 64 distinct ids fill every lane of the plan
    ids = rng.permutation(300)[:64].reshape(8, 8).astype(np.int32)
    got = dm.moe_plan(to_dev(torch, ids), 300)
    assert got == [300] + [int(i) for i in ids.ravel()]
    # invalid ids are skipped, repeats keep their first slot
    ids = np.array([[4, -1, 4, 2], [9, 2, 12, 4]], dtype=np.int32)
    assert dm.moe_plan(to_dev(torch, ids), 10) == [10, 4, 2, 9]


def test_bad_and_duplicate_ids(torch_dev, small_layers):
    torch = torch_dev
    lay, ox = small_layers[100]
    E = lay.n_routed
    ids, w = synth.routing(SEED, 100, 0, 77, 2, E, lay.top_k)
    # an out-of-range id is skipped and flagged
    bad = ids.copy()
    bad[1, 3] = E + 5
    say("bad id")
    ws = lay.workspace(2)
    x = synth.activations(SEED, 100, 0, 77, 2, lay.hidden)
    out = dm.moe_layer(lay, to_dev(torch, x), to_dev(torch, bad), to_dev(torch, w), ws=ws)
    assert dm.status(ws) & dm.duckmoe.STATUS_BAD_ID
    keep = np.ones_like(bad, dtype=bool)
    keep[1, 3] = False
    w_ref = np.where(keep, w, 0.0)
    ids_ref = np.where(keep, bad, bad[1, 0])
    ox.prefetch(list(ids_ref.ravel()) + [E])
    check_close(out.cpu().numpy(), oracle.moe_layer(ox, x, ids_ref, w_ref, E), "bad id skipped")
    # a repeated id within a token: weights add
    dup = ids.copy()
    dup[0, 5] = dup[0, 2]
    say("duplicate id")
    out = dm.moe_layer(lay, to_dev(torch, x), to_dev(torch, dup), to_dev(torch, w), ws=ws)
    assert dm.status(ws) == dm.duckmoe.STATUS_DUP_ID
    ox.prefetch(list(dup.ravel()) + [E])
    check_close(out.cpu().numpy(), oracle.moe_layer(ox, x, dup, w, E), "duplicate id")
    # clean call clears the status
    dm.moe_layer(lay, to_dev(torch, x), to_dev(torch, ids), to_dev(torch, w), ws=ws)
    assert dm.status(ws) == 0


def test_zero_weights_and_stage_split(torch_dev, small_layers):
    torch = torch_dev
    lay, ox = small_layers[100]
    E = lay.n_routed
    x = synth.activations(SEED, 100, 0, 88, 2, lay.hidden)
    ids, w = synth.routing(SEED, 100, 0, 88, 2, E, lay.top_k)
    say("zero weights")
    xd, idd = to_dev(torch, x), to_dev(torch, ids)
    out0 = dm.moe_layer(lay, xd, idd, to_dev(torch, np.zeros_like(w)))
    ox.prefetch([E])
    check_close(out0.cpu().numpy(), oracle.expert_ffn(ox(E), x), "zero routing weights")
    say("stage split")
    wd = to_dev(torch, w)
    ws = lay.workspace(2)
    full = dm.moe_layer(lay, xd, idd, wd, ws=ws).cpu().numpy()
    ws2 = lay.workspace(2)
    dm.moe_gate_up(lay, xd, idd, wd, ws2)
    split = dm.moe_down(lay, xd, idd, wd, ws2).cpu().numpy()
    check_close(split, full, "stage split vs one call")
    ox.prefetch(list(ids.ravel()) + [E])
    check_close(split, oracle.moe_layer(ox, x, ids, w, E), "stage split")


def test_repeat_calls_bit_identical(torch_dev, small_layers):
    torch = torch_dev
    lay, _ = small_layers[101]
    x = to_dev(torch, synth.activations(SEED, 101, 0, 5, 2, lay.hidden))
    ids, w = synth.routing(SEED, 101, 0, 5, 2, lay.n_routed, lay.top_k)
    idd, wd = to_dev(torch, ids), to_dev(torch, w)
    say("repeat calls")
    ws = lay.workspace(2)
    first = dm.moe_layer(lay, x, idd, wd, ws=ws).cpu().numpy()
    for _ in range(20):
        again = dm.moe_layer(lay, x, idd, wd, ws=ws).cpu().numpy()
        np.testing.assert_array_equal(first, again)


# ---------------------------------------------------- full-size V3 workloads --

H3, I3, E3, K3 = 7168, 2048, 256, 8


@pytest.fixture(scope="module")
def v3_layer(torch_dev):
    say("build 256+1 expert layer (12.7 GB fp9)")
    lay = dm.Layer(H3, I3, E3, K3).fill_synthetic(SEED, 3, 0)
    return lay, OracleExperts(SEED, 3, 0, H3, I3)


def test_expert_ffn_full_size(torch_dev, v3_layer):
    """One SwiGLU expert 7168/2048 at bsz 1 (a routed expert), plus
    the shared expert at bsz 2 and its 32 partials."""
    torch = torch_dev
    lay, ox = v3_layer
    x = synth.activations(SEED, 2, 0, 0, 2, H3)
    for e in (17, E3):
        say("expert_ffn", e)
        ox.prefetch([e])
        got = dm.expert_ffn(lay, e, to_dev(torch, x[:1])).cpu().numpy()
        check_close(got, oracle.expert_ffn(ox(e), x[:1]), "expert %d" % e)
    say("expert_ffn partials")
    got = dm.expert_ffn(lay, E3, to_dev(torch, x), n_shards=32).cpu().numpy()
    ref = oracle.moe_partials(lambda _: ox(E3), x, np.zeros((2, 0), np.int64),
                              np.zeros((2, 0)), E3, 32)
    for r in range(32):
        check_close(got[r], ref[r], "shared expert shard %d" % r)


@pytest.mark.parametrize("step", [0, 1, 2])
def test_full_layer_bsz1(torch_dev, v3_layer, step):
    torch = torch_dev
    lay, ox = v3_layer
    say("full layer bsz 1 step", step)
    x, ids, w, got = run_layer_case(torch, lay, ox, 3, step, 1)
    check_close(got, oracle.moe_layer(ox, x, ids, w, E3), "layer bsz1 step %d" % step)


def test_full_layer_bsz2_and_partials(torch_dev, v3_layer):
    """The bsz-2 pair: two tokens with independent top-8 sets; then 32 partials of
    64-wide intermediate slices whose sum is the full output."""
    torch = torch_dev
    lay, ox = v3_layer
    say("full layer bsz 2")
    x, ids, w, got = run_layer_case(torch, lay, ox, 3, 100, 2)
    ref = oracle.moe_layer(ox, x, ids, w, E3)
    check_close(got, ref, "layer bsz2")
    say("full layer bsz 2, 32 partials")
    _, _, _, parts = run_layer_case(torch, lay, ox, 3, 100, 2, n_shards=32)
    pref = oracle.moe_partials(ox, x, ids, w, E3, 32)
    for r in range(32):
        check_close(parts[r], pref[r], "partial %d" % r)
    check_close(parts.sum(axis=0), ref, "sum of 32 partials")


def test_full_layer_matrix_core_batch_sizes(torch_dev, v3_layer):
    """The matrix-core path (3 to 8 tokens) on the full 257-expert layer: one
    draw of 7 tokens, its first T tokens for T = 3 .. 7 (bsz 8 has its own
    test), each against the oracle on the same tokens."""
    torch = torch_dev
    lay, ox = v3_layer
    x = synth.activations(SEED, 3, 0, 300, 7, H3)
    ids, w = synth.routing(SEED, 3, 0, 300, 7, E3, K3)
    ox.prefetch(list(ids.ravel()) + [E3])
    for T in (3, 4, 5, 6, 7):
        say("full layer, first", T, "tokens of a 7-token draw")
        xt, it, wt = x[:T], ids[:T], w[:T]
        ws = lay.workspace(T)
        got = dm.moe_layer(lay, to_dev(torch, xt), to_dev(torch, it.astype(np.int32)),
                           to_dev(torch, wt.astype(np.float32)), ws=ws).cpu().numpy()
        assert dm.status(ws) == 0
        check_close(got, oracle.moe_layer(ox, xt, it, wt, E3), "layer bsz%d" % T)


def test_full_layer_bsz8_max_ids(torch_dev, v3_layer):
    torch = torch_dev
    lay, ox = v3_layer
    say("full layer bsz 8 (64 ids)")
    x, ids, w, got = run_layer_case(torch, lay, ox, 3, 200, 8)
    check_close(got, oracle.moe_layer(ox, x, ids, w, E3), "layer bsz8")


def test_full_layer_prefill_2048(torch_dev, v3_layer):
    """The prefill workload: 2048 tokens through the 257-expert layer (every
    expert selected, the shared one in 32 tiles); sampled tokens against the
    oracle, and the whole output against the decode path on 8-token slices."""
    torch = torch_dev
    lay, ox = v3_layer
    T = 2048
    x = synth.activations(SEED, 7, 0, 0, T, H3)
    ids, w = synth.routing(SEED, 7, 0, 0, T, E3, K3)
    say("full layer prefill T = 2048")
    xd, idd, wd = to_dev(torch, x), to_dev(torch, ids), to_dev(torch, w)
    ws = lay.prefill_workspace(T)
    got = dm.moe_prefill(lay, xd, idd, wd, ws=ws).cpu().numpy()
    assert dm.status(ws) == 0
    toks = [0, 1337]
    ox.prefetch(list(ids[toks].ravel()) + [E3])
    ref = oracle.moe_layer(ox, x[toks], ids[toks], w[toks], E3)
    for i, t in enumerate(toks):
        check_close(got[t], ref[i], "prefill T=2048 token %d" % t)
    say("prefill T = 2048 against the decode path, 8 tokens at a time")
    for t0 in range(0, T, 8):
        dec = dm.moe_layer(lay, xd[t0:t0 + 8], idd[t0:t0 + 8], wd[t0:t0 + 8]).cpu().numpy()
        for t in range(8):
            check_close(got[t0 + t], dec[t], "prefill vs decode token %d" % (t0 + t))


def test_read_probe_runs(torch_dev):
    """The calibration read touches only its buffer and leaves the sink alone."""
    torch = torch_dev
    say("read probe")
    buf = torch.ones(1 << 22, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for nb in (1024, 5 * 1024, 1 << 22):
        dm.read_probe(buf, nb, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0


def test_shard_partials_at_larger_batch(torch_dev, small_layers):
    """Shard partials at T = 4 (the vector kernels; the matrix-core path has no
    partial mode): each shard and their sum against the oracle."""
    torch = torch_dev
    lay, ox = small_layers[103]
    say("shard partials at T = 4")
    x, ids, w, got = run_layer_case(torch, lay, ox, 103, 77, 4, n_shards=8)
    ref = oracle.moe_partials(ox, x, ids, w, lay.n_routed, 8)
    for r in range(8):
        check_close(got[r], ref[r], "T=4 shard %d/8" % r)
    check_close(got.sum(axis=0), oracle.moe_layer(ox, x, ids, w, lay.n_routed), "T=4 sum of partials")
