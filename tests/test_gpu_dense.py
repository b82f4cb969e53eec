"""GPU parity of wide intermediate sizes (more 1024-wide chunks than down
waves) and of the dense fp9 MLP (a layer with no routed experts, run through
duckmoe_expert_ffn), against the float64 oracle.

Bar: relative L2 <= 1e-5 and max-abs <= 1e-4 * max|ref|.  The dense MLP at
full size is DeepSeek-V3's dense FFN shape, 7168/18432, drawn on the device.
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


WIDE = {  # workload: (H, I, n_routed, top_k): 3 chunks; 5 full chunks + a 16-wide one
    160: (1040, 3072, 6, 4),
    161: (2064, 5136, 4, 2),
}


@pytest.fixture(scope="module")
def wide_layers(torch_dev):
    out = {}
    for wl, (H, I, E, K) in WIDE.items():
        say("building wide layer", wl, (H, I, E, K))
        out[wl] = (dm.Layer(H, I, E, K).fill_synthetic(SEED, wl, 0), OracleExperts(SEED, wl, 0, H, I))
    return out


@pytest.mark.parametrize("wl", sorted(WIDE))
@pytest.mark.parametrize("T", [1, 2, 3, 8])
def test_wide_layer(torch_dev, wide_layers, wl, T):
    torch = torch_dev
    lay, ox = wide_layers[wl]
    say("wide layer", wl, "T =", T)
    x = synth.activations(SEED, wl, 0, T, T, lay.hidden)
    ids, w = synth.routing(SEED, wl, 0, T, T, lay.n_routed, lay.top_k)
    ox.prefetch(list(ids.ravel()) + [lay.n_routed])
    got = dm.moe_layer(lay, to_dev(torch, x), to_dev(torch, ids), to_dev(torch, w)).cpu().numpy()
    check_close(got, oracle.moe_layer(ox, x, ids, w, lay.n_routed), "wide %d T=%d" % (wl, T))


def test_wide_layer_rejects_shards(torch_dev, wide_layers):
    torch = torch_dev
    lay, _ = wide_layers[160]
    x = to_dev(torch, synth.activations(SEED, 160, 0, 1, 1, lay.hidden))
    ids, w = synth.routing(SEED, 160, 0, 1, 1, lay.n_routed, lay.top_k)
    with pytest.raises(dm.DuckMoeError):
        dm.moe_layer(lay, x, to_dev(torch, ids), to_dev(torch, w), n_shards=3)


@pytest.mark.parametrize("T", [1, 2, 5, 8])
def test_small_dense_mlp(torch_dev, T):
    torch = torch_dev
    H, I, wl = 1040, 4112, 162                     # 5 chunks, the last 16 wide
    say("small dense MLP T =", T)
    mlp = dm.Layer(H, I, 0, 1).fill_synthetic(SEED, wl, 0)
    ox = OracleExperts(SEED, wl, 0, H, I)
    x = synth.activations(SEED, wl, 0, T, T, H)
    got = dm.expert_ffn(mlp, 0, to_dev(torch, x)).cpu().numpy()
    check_close(got, oracle.expert_ffn(ox(0), x), "dense 1040/4112 T=%d" % T)


def test_full_size_dense_mlp(torch_dev):
    """7168/18432: gate/up 2 x 132 M weights, down 132 M, drawn on the device."""
    torch = torch_dev
    H, I, wl = 7168, 18432, 163
    say("full-size dense MLP: drawing and quantizing on the device")
    mlp = dm.Layer(H, I, 0, 1).fill_synthetic_device(SEED, wl, 0)
    ox = OracleExperts(SEED, wl, 0, H, I, device_drawn=True)
    say("oracle quantizes the same draws")
    codes = ox(0)
    for T in (1, 4):
        say("full-size dense MLP T =", T)
        x = synth.activations(SEED, wl, 0, T, T, H)
        got = dm.expert_ffn(mlp, 0, to_dev(torch, x)).cpu().numpy()
        check_close(got, oracle.expert_ffn(codes, x), "dense 7168/18432 T=%d" % T)
