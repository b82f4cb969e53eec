"""GPU tests: the layer calls captured in a HIP graph (torch.cuda.CUDAGraph).

The calls launch kernels only (no memset or copy nodes), so a captured call
replays as the same kernels on the same buffers.  Each graph is replayed
several times with eager calls on other inputs and host synchronizations in
between, and every replay must equal the eager result bit for bit.
"""

import numpy as np
import pytest

from gpu_util import say
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


@pytest.fixture(scope="module")
def small(torch_dev):
    H, I, E, K, wl = 1040, 336, 24, 8, 180
    return dm.Layer(H, I, E, K).fill_synthetic(SEED, wl, 0), wl


def dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def replay_matches_eager(torch, call, other, out):
    """call(stream) writes `out`; other(stream) is eager work on other buffers.
    Captures call, replays it 4 times with `other` and synchronizations in
    between, and checks each replay against the eager result."""
    torch.cuda.synchronize()
    call(torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref = out.clone()
    out.fill_(float("nan"))
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(side)  # the first call of each launch site outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    out.fill_(float("nan"))
    with torch.cuda.graph(g):
        call(torch.cuda.current_stream())
    for rep in range(4):
        other(torch.cuda.current_stream())
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), "replay %d differs from the eager call" % rep
    del g


@pytest.mark.parametrize("T", [1, 2, 4])
def test_layer_call_in_graph(torch_dev, small, T):
    torch = torch_dev
    lay, wl = small
    say("graph: layer T =", T)
    x = dev(torch, synth.activations(SEED, wl, 0, T, T, lay.hidden))
    ids, w = synth.routing(SEED, wl, 0, T, T, lay.n_routed, lay.top_k)
    ids, w = dev(torch, ids), dev(torch, w)
    x2 = dev(torch, synth.activations(SEED, wl, 0, 50 + T, T, lay.hidden))
    out = torch.empty((T, lay.hidden), dtype=torch.float32, device="cuda")
    out2 = torch.empty_like(out)
    ws, ws2 = lay.workspace(T), lay.workspace(T)

    def call(st):
        dm.moe_layer(lay, x, ids, w, out=out, ws=ws, stream=st)

    def other(st):
        dm.moe_layer(lay, x2, ids, w, out=out2, ws=ws2, stream=st)

    replay_matches_eager(torch, call, other, out)


@pytest.mark.parametrize("T", [1, 2])
def test_expert_call_in_graph(torch_dev, small, T):
    torch = torch_dev
    lay, wl = small
    say("graph: expert_ffn T =", T)
    x = dev(torch, synth.activations(SEED, wl, 0, 90 + T, T, lay.hidden))
    x2 = dev(torch, synth.activations(SEED, wl, 0, 95 + T, T, lay.hidden))
    out = torch.empty((T, lay.hidden), dtype=torch.float32, device="cuda")
    out2 = torch.empty_like(out)
    ws, ws2 = lay.workspace(T), lay.workspace(T)

    def call(st):
        dm.expert_ffn(lay, 5, x, out=out, ws=ws, stream=st)

    def other(st):
        dm.expert_ffn(lay, lay.n_routed, x2, out=out2, ws=ws2, stream=st)

    replay_matches_eager(torch, call, other, out)
