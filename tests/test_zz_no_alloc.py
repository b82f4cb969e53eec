"""GPU test of duckmoe_moe_layer_noalloc, the layer call that allocates nothing
and runs on the library's static device workspace: called through the C ABI,
its outputs must equal duckmoe_moe_layer's on a caller workspace bit for bit
(the same kernels on the same inputs), on two calls in a row with the second
smaller than the first (the array keeps the first call's contents), on the
vector path (T <= 2), the matrix-core path (T >= 3) and shard partials; a
call whose workspace would exceed the array is refused on the host.  The
outputs are also within the f32 bar of the float64 oracle.
"""

import ctypes

import numpy as np
import pytest

import oracle
from gpu_util import OracleExperts, check_close, say
from lib_util import ensure_built

import bit_moe_expert_fp9_amd as dm
from bit_moe_expert_fp9_amd import synth

pytestmark = pytest.mark.gpu

SEED = 0
WL, H, I, E, K = 108, 2064, 1536, 16, 4


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a GPU (deselect with -m 'not gpu')")
    ensure_built()
    return torch


@pytest.fixture(scope="module")
def layer(torch_dev):
    say("build no-alloc test layer", WL, H, I, E, K)
    return dm.Layer(H, I, E, K).fill_synthetic(SEED, WL, 0), OracleExperts(SEED, WL, 0, H, I)


def inputs(torch, T, draw):
    x = synth.activations(SEED, WL, 0, draw, T, H)
    ids, w = synth.routing(SEED, WL, 0, draw, T, E, K)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return x, ids, w, dev(x), dev(ids.astype(np.int32)), dev(w.astype(np.float32))


@pytest.mark.parametrize("sizes", [(8, 2), (5, 1), (2, 1)])
def test_noalloc_matches_layer_call(torch_dev, layer, sizes):
    torch = torch_dev
    lay, ox = layer
    for k, T in enumerate(sizes):
        x, ids, w, xd, idd, wd = inputs(torch, T, 200 + 10 * T + k)
        out = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
        say("noalloc call", k, "T =", T)
        dm.moe_layer_noalloc(lay, xd, idd, wd, out)
        ref = dm.moe_layer(lay, xd, idd, wd, ws=lay.workspace(T))
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.array_equal(got, ref.cpu().numpy()), "T=%d differs from duckmoe_moe_layer" % T
        ox.prefetch([int(i) for i in np.unique(ids)] + [E])
        check_close(got, oracle.moe_layer(ox, x, ids, w, E), "noalloc T=%d" % T)


def test_noalloc_shard_partials(torch_dev, layer):
    torch = torch_dev
    lay, ox = layer
    for k, (T, ns) in enumerate(((2, 6), (1, 3))):
        x, ids, w, xd, idd, wd = inputs(torch, T, 300 + k)
        out = torch.empty((ns, T, H), dtype=torch.float32, device="cuda")
        say("noalloc shard partials T =", T, "n_shards =", ns)
        dm.moe_layer_noalloc(lay, xd, idd, wd, out, n_shards=ns)
        ref = dm.moe_layer(lay, xd, idd, wd, n_shards=ns, ws=lay.workspace(T, ns))
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        ox.prefetch([int(i) for i in np.unique(ids)] + [E])
        want = oracle.moe_partials(ox, x, ids, w, E, ns)
        for r in range(ns):
            check_close(out[r].cpu().numpy(), want[r], "noalloc shard %d/%d" % (r, ns))


def test_noalloc_refuses_oversize(torch_dev):
    # 65 slots x 8 tokens x 8192 rows of f32 h' is 17 MB, past the 16 MiB array
    big = dm.LayerStruct(64, 8192, 64, 8, 256, 256, 256, 256)
    L = dm.lib()
    assert L.duckmoe_workspace_bytes(ctypes.byref(big), 8, 1) > (16 << 20)
    rc = L.duckmoe_moe_layer_noalloc(ctypes.byref(big), ctypes.c_void_p(256),
                                     ctypes.c_void_p(256), ctypes.c_void_p(256), 8,
                                     ctypes.c_void_p(256), 1, None)
    assert rc == dm.duckmoe.EWORKSPACE
    # the same layer at 2 tokens fits, but a null pointer is still refused first
    rc = L.duckmoe_moe_layer_noalloc(ctypes.byref(big), None, ctypes.c_void_p(256),
                                     ctypes.c_void_p(256), 2, ctypes.c_void_p(256), 1, None)
    assert rc == dm.duckmoe.EINVAL
