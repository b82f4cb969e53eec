"""GPU parity of the device quantizer, the RMS glue and the layer stack.

Bars: the device quantizer's planes bit-exact against the oracle's quantizer
and packer; f32 outputs within relative L2 <= 1e-5 and max-abs <= 1e-4 *
max|ref| of the float64 oracle.  The stack is checked per layer with teacher
forcing: the oracle gets the GPU's input to layer l and its output is compared
with the GPU's output of layer l; the native stack call must equal the same
layers and glue called one by one, bit for bit.  The full-size
stack is 16 layers of 7168/2048 with 256 routed + 1 shared experts each (about
204 GB of fp9 weights resident), drawn on the device.
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


# ------------------------------------------------------- device quantizer --

def quantizer_cases():
    """float32 values that exercise every branch of the rounding, plus random bits."""
    rng = np.random.default_rng(5)
    codes = np.arange(512)
    codes = codes[((codes >> 3) & 31) != 31]                       # the 496 finite codes
    vals = oracle.decode(codes)                                    # exact fp9 values
    mids = (vals[:-1] + vals[1:]) / 2                               # ties between neighbours
    pos = np.sort(np.unique(np.abs(vals)))
    ties = (pos[:-1] + pos[1:]) / 2
    exact = np.concatenate([vals, ties, -ties, mids]).astype(np.float32)
    up = np.nextafter(exact, np.float32(np.inf))
    dn = np.nextafter(exact, np.float32(-np.inf))
    special = np.array([0.0, -0.0, np.inf, -np.inf, 61440, 61439.996, 63487.996, 63488, 1e30,
                        2.0 ** -18, -(2.0 ** -18), 2.0 ** -19, 1e-40, -1e-45, 2.0 ** -14,
                        np.nextafter(np.float32(2.0 ** -14), np.float32(0))], dtype=np.float32)
    bits = rng.integers(0, 2 ** 32, size=1 << 21, dtype=np.uint64).astype(np.uint32)
    randbits = bits.view(np.float32)
    randbits = randbits[~np.isnan(randbits)]
    gauss = (rng.standard_normal(1 << 20) * 0.02).astype(np.float32)
    v = np.concatenate([exact, up, dn, special, randbits, gauss])
    return v[: len(v) // 512 * 512].reshape(-1, 512)


def test_device_quantizer_bit_exact(torch_dev):
    torch = torch_dev
    w = quantizer_cases()
    say("device quantizer on", w.size, "values")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    body, sign = dm.quantize_fp9_device(to_dev(torch, w), nonfinite=flag)
    ref_body, ref_sign = oracle.pack(oracle.quantize(w))
    np.testing.assert_array_equal(body.cpu().numpy(), ref_body)
    np.testing.assert_array_equal(sign.cpu().numpy(), ref_sign)
    assert int(flag.item()) == 0
    # the host codec agrees too
    hb, hs = dm.quantize_fp9(w)
    np.testing.assert_array_equal(hb, ref_body)
    np.testing.assert_array_equal(hs, ref_sign)


def test_device_quantizer_nan_flag_and_shapes(torch_dev):
    torch = torch_dev
    say("device quantizer NaN flag, ragged rows")
    w = (np.random.default_rng(6).standard_normal((3, 24)) * 0.02).astype(np.float32)
    w[2, 5] = np.nan
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    body, sign = dm.quantize_fp9_device(to_dev(torch, w), nonfinite=flag)
    assert int(flag.item()) == 1
    ok_b, ok_s = oracle.pack(oracle.quantize(w[:2]))
    np.testing.assert_array_equal(body.cpu().numpy()[:2], ok_b)
    np.testing.assert_array_equal(sign.cpu().numpy()[:2], ok_s)
    # one row of 8 and an empty matrix
    one = np.array([[1.0, -1.0, 0.5, -0.0, 61440, -(2.0 ** -17), 1.5, -3.0]], dtype=np.float32)
    b1, s1 = dm.quantize_fp9_device(to_dev(torch, one))
    np.testing.assert_array_equal(b1.cpu().numpy(), [[0x78, 0x78, 0x70, 0x00, 0xF7, 0x01, 0x7C, 0x84]])
    np.testing.assert_array_equal(s1.cpu().numpy(), [[0xAA]])
    dm.quantize_fp9_device(torch.empty((0, 8), dtype=torch.float32, device="cuda"))


def test_device_and_host_filled_layers_agree(torch_dev):
    """A layer quantized on the device equals one quantized on the host."""
    torch = torch_dev
    H, I, E, K = 1040, 336, 6, 4
    say("device-quantized small layer vs host-quantized")
    a = dm.Layer(H, I, E, K).fill_synthetic(SEED, 120, 0)
    b = dm.Layer(H, I, E, K)
    for e in range(E + 1):
        g, u, d = (to_dev(torch, synth.weights(SEED, 120, 0, e, m, shp))
                   for m, shp in enumerate(synth.expert_shapes(H, I)))
        b.set_expert_device(e, g, u, d)
    torch.cuda.synchronize()
    for name in ("gu_body", "gu_sign", "dn_body", "dn_sign"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name


# ------------------------------------------------------------------ glue --

@pytest.mark.parametrize("T,H", [(1, 7168), (8, 7168), (3, 1000), (2, 17)])
def test_rms_normalize(torch_dev, T, H):
    torch = torch_dev
    say("rms_normalize T =", T, "H =", H)
    x = synth.activations(SEED, 130, 0, H, T, H) * np.float32(37.0)
    for eps in (0.0, 1e-6, 3.0):
        got = dm.rms_normalize(to_dev(torch, x), eps=eps).cpu().numpy()
        ref = oracle.rms_normalize(x, eps=eps)
        for t in range(T):
            check_close(got[t], ref[t], "rms T=%d H=%d eps=%g token %d" % (T, H, eps, t))
    # in place gives the same bits
    xd = to_dev(torch, x)
    out = dm.rms_normalize(xd).clone()
    dm.rms_normalize(xd, out=xd)
    assert torch.equal(out, xd)


def test_rms_normalize_zero_row(torch_dev):
    torch = torch_dev
    say("rms_normalize zero row")
    x = np.zeros((2, 64), dtype=np.float32)
    x[1] = 1.0
    got = dm.rms_normalize(to_dev(torch, x)).cpu().numpy()
    assert np.all(np.isnan(got[0])) and np.all(got[1] == 1.0)
    got = dm.rms_normalize(to_dev(torch, x), eps=1e-6).cpu().numpy()
    assert np.all(got[0] == 0.0)


# ----------------------------------------------------------------- stacks --

def run_chain(torch, stack, x, ids, w, eps):
    """The stack's layers and glue called one by one: (inputs h_l, outputs y_l)."""
    h = to_dev(torch, x)
    hs, ys = [], []
    for l, lay in enumerate(stack.layers):
        hs.append(h.cpu().numpy())
        ws = lay.workspace(x.shape[0])
        y = dm.moe_layer(lay, h, to_dev(torch, ids[l]), to_dev(torch, w[l]), ws=ws)
        assert dm.status(ws) == 0
        ys.append(y.cpu().numpy())
        h = dm.rms_normalize(y, eps=eps)
    return hs, ys


def check_stack(torch, stack, oxs, x, ids, w, eps, samples, what):
    """Stack call == chain, bit for bit; sampled (layer, tokens) against the oracle."""
    n_routed = stack.layers[0].n_routed
    got = dm.moe_stack(stack, to_dev(torch, x), to_dev(torch, ids), to_dev(torch, w),
                       eps=eps).cpu().numpy()
    hs, ys = run_chain(torch, stack, x, ids, w, eps)
    np.testing.assert_array_equal(got, ys[-1])
    for l, toks in samples:
        say(what, "oracle layer", l, "tokens", toks)
        h = hs[l][toks]
        oxs[l].prefetch(list(ids[l][toks].ravel()) + [n_routed])
        ref = oracle.moe_layer(oxs[l], h, ids[l][toks], w[l][toks], n_routed)
        for i, t in enumerate(toks):
            check_close(ys[l][t], ref[i], "%s layer %d token %d" % (what, l, t))
        if l + 1 < len(stack.layers):
            check_close(hs[l + 1][toks], oracle.rms_normalize(ys[l][toks], eps=eps),
                        "%s glue after layer %d" % (what, l))


def stack_inputs(wl, n_layers, T, n_routed, top_k, H, step):
    x = synth.activations(SEED, wl, 0, step, T, H)
    r = [synth.routing(SEED, wl, l, step, T, n_routed, top_k) for l in range(n_layers)]
    ids = np.stack([a for a, _ in r]).astype(np.int32)
    w = np.stack([b for _, b in r]).astype(np.float32)
    return x, ids, w


@pytest.mark.parametrize("T", [1, 3, 8])
def test_small_stack(torch_dev, T):
    torch = torch_dev
    H, I, E, K, NL, wl = 1040, 336, 24, 8, 4, 140
    say("small stack T =", T)
    layers = [dm.Layer(H, I, E, K).fill_synthetic(SEED, wl, l) for l in range(NL)]
    oxs = [OracleExperts(SEED, wl, l, H, I) for l in range(NL)]
    x, ids, w = stack_inputs(wl, NL, T, E, K, H, 10 + T)
    check_stack(torch, dm.Stack(layers), oxs, x, ids, w, 0.0,
                [(l, list(range(T))) for l in range(NL)], "small stack T=%d" % T)


@pytest.mark.parametrize("T,H,eps", [
    (4, 1040, 1e-5),   # matrix-core layers: the next layer's first launch adds the partials
    (6, 1040, 0.0),    # the same with three row tiles per down task
    (3, 8320, 0.0),    # rows past 8192 floats: the partials are added and split in two launches
    (5, 8320, 1e-5),
])
def test_stack_glue_forms(torch_dev, T, H, eps):
    torch = torch_dev
    I, E, K, NL, wl = 208, 12, 4, 3, 141
    say("stack glue forms T =", T, "H =", H, "eps =", eps)
    layers = [dm.Layer(H, I, E, K).fill_synthetic(SEED, wl, l) for l in range(NL)]
    oxs = [OracleExperts(SEED, wl, l, H, I) for l in range(NL)]
    x, ids, w = stack_inputs(wl, NL, T, E, K, H, 20 + T)
    check_stack(torch, dm.Stack(layers), oxs, x, ids, w, eps,
                [(l, list(range(T))) for l in range(NL)], "stack T=%d H=%d" % (T, H))


# The full-size stack: 16 layers x (256 routed + 1 shared) experts of 7168/2048, drawn on
# the device (~204 GB of fp9 planes resident), run at bsz 1, 2, 4 and 8.
FULL = dict(H=7168, I=2048, E=256, K=8, NL=16, wl=5)


@pytest.fixture(scope="module")
def full_stack(torch_dev):
    torch = torch_dev
    torch.cuda.empty_cache()
    free, total = torch.cuda.mem_get_info()
    need = FULL["NL"] * (FULL["E"] + 1) * 3 * FULL["H"] * FULL["I"] * 9 // 8
    if free < need + (8 << 30):
        pytest.skip("the 16-layer stack needs %.0f GB of free device memory (%.0f free)" %
                    (need / 1e9, free / 1e9))
    layers = []
    for l in range(FULL["NL"]):
        say("drawing and quantizing layer", l, "of the full-size stack on the device")
        layers.append(dm.Layer(FULL["H"], FULL["I"], FULL["E"], FULL["K"])
                      .fill_synthetic_device(SEED, FULL["wl"], l))
    torch.cuda.synchronize()
    yield dm.Stack(layers)
    del layers
    torch.cuda.empty_cache()


@pytest.mark.parametrize("T,samples", [
    (1, [(0, [0]), (15, [0])]),
    (2, [(9, [0, 1])]),
    (4, [(6, [3])]),
    (8, [(12, [5])]),
])
def test_full_stack(torch_dev, full_stack, T, samples):
    torch = torch_dev
    say("full-size stack T =", T)
    oxs = {l: OracleExperts(SEED, FULL["wl"], l, FULL["H"], FULL["I"], device_drawn=True)
           for l, _ in samples}
    x, ids, w = stack_inputs(FULL["wl"], FULL["NL"], T, FULL["E"], FULL["K"], FULL["H"], 100 + T)
    check_stack(torch, full_stack, oxs, x, ids, w, 0.0, samples, "full stack T=%d" % T)
