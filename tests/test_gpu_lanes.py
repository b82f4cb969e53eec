"""GPU tests of the asynchronous lanes (duckmoe_lane_*).

A lane's layer must equal the plain duckmoe_moe_layer call bit for bit (same
kernels, its own stream and workspace), must not start before the producer
stream has written its input, and its output must be visible to a consumer
stream after finish.  The full-size case runs the bsz-2 pair (two
tokens with independent top-8 sets on the 257-expert layer) as two lanes.
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


@pytest.fixture(scope="module")
def small(torch_dev):
    H, I, E, K, wl = 1040, 336, 24, 8, 170
    return dm.Layer(H, I, E, K).fill_synthetic(SEED, wl, 0), OracleExperts(SEED, wl, 0, H, I), wl


def inputs(torch, lay, wl, step):
    x = synth.activations(SEED, wl, 0, step, 1, lay.hidden)
    ids, w = synth.routing(SEED, wl, 0, step, 1, lay.n_routed, lay.top_k)
    return x, ids, w, to_dev(torch, x), to_dev(torch, ids), to_dev(torch, w)


def test_two_lanes_equal_plain_calls(torch_dev, small):
    torch = torch_dev
    lay, ox, wl = small
    say("two lanes vs plain calls")
    cases = [inputs(torch, lay, wl, s) for s in (1, 2)]
    ref = [dm.moe_layer(lay, xd, idd, wd).cpu().numpy() for _, _, _, xd, idd, wd in cases]
    lanes = [dm.Lane(lay), dm.Lane(lay)]
    outs = [torch.full((1, lay.hidden), float("nan"), device="cuda") for _ in lanes]
    for rep in range(3):
        for lane, (_, _, _, xd, idd, wd), o in zip(lanes, cases, outs):
            lane.begin(lay, xd, idd, wd, o)
        for lane in lanes:
            lane.finish()
        for o, r in zip(outs, ref):
            np.testing.assert_array_equal(o.cpu().numpy(), r)
    for (x, ids, w, *_), o in zip(cases, outs):
        ox.prefetch(list(ids.ravel()) + [lay.n_routed])
        check_close(o.cpu().numpy(), oracle.moe_layer(ox, x, ids, w, lay.n_routed), "lane")
    for lane in lanes:
        lane.close()


def test_lane_waits_for_its_producer(torch_dev, small):
    """x is written on another stream behind a long spin; the lane must read the
    new x, not the zeros it held when begin was called."""
    torch = torch_dev
    lay, _, wl = small
    say("lane waits for its producer stream")
    x, ids, w, xd, idd, wd = inputs(torch, lay, wl, 3)
    ref = dm.moe_layer(lay, xd, idd, wd).cpu().numpy()
    producer = torch.cuda.Stream()
    xin = torch.zeros_like(xd)
    torch.cuda.synchronize()
    with torch.cuda.stream(producer):
        torch.cuda._sleep(50_000_000)
        xin.copy_(xd)
    lane = dm.Lane(lay)
    out = torch.empty_like(xd)
    lane.begin(lay, xin, idd, wd, out, producer=producer)
    lane.finish(block=True)
    np.testing.assert_array_equal(out.cpu().numpy(), ref)
    lane.close()


def test_lane_output_ordered_for_consumer(torch_dev, small):
    torch = torch_dev
    lay, _, wl = small
    say("consumer stream waits for the lane")
    x, ids, w, xd, idd, wd = inputs(torch, lay, wl, 4)
    ref = dm.moe_layer(lay, xd, idd, wd).cpu().numpy()
    consumer = torch.cuda.Stream()
    lane = dm.Lane(lay)
    out = torch.zeros_like(xd)
    torch.cuda.synchronize()
    lane.begin(lay, xd, idd, wd, out)
    lane.finish(consumer=consumer)
    with torch.cuda.stream(consumer):
        copy = out.clone()
    consumer.synchronize()
    np.testing.assert_array_equal(copy.cpu().numpy(), ref)
    lane.close()


def test_full_size_pair_as_two_lanes(torch_dev):
    torch = torch_dev
    H, I, E, K, wl = 7168, 2048, 256, 8, 4
    say("full-size layer for the lane pair")
    lay = dm.Layer(H, I, E, K).fill_synthetic_device(SEED, 171, 0)
    ox = OracleExperts(SEED, 171, 0, H, I, device_drawn=True)
    x = synth.activations(SEED, wl, 0, 7, 2, H)
    ids, w = synth.routing(SEED, wl, 0, 7, 2, E, K)
    lanes = [dm.Lane(lay), dm.Lane(lay)]
    outs = [torch.empty((1, H), device="cuda") for _ in lanes]
    # the device inputs stay referenced until the lanes finish
    xs = [to_dev(torch, x[t:t + 1]) for t in range(2)]
    idss = [to_dev(torch, ids[t:t + 1]) for t in range(2)]
    wss = [to_dev(torch, w[t:t + 1]) for t in range(2)]
    for t in range(2):
        lanes[t].begin(lay, xs[t], idss[t], wss[t], outs[t])
    for lane in lanes:
        lane.finish()
    got = torch.cat(outs).cpu().numpy()
    pair = dm.moe_layer(lay, to_dev(torch, x), to_dev(torch, ids), to_dev(torch, w)).cpu().numpy()
    check_close(got, pair, "two lanes vs one bsz-2 call")
    ox.prefetch(list(ids.ravel()) + [E])
    check_close(got, oracle.moe_layer(ox, x, ids, w, E), "two lanes vs oracle")
    for lane in lanes:
        lane.close()


@pytest.mark.parametrize("T", [1, 2, 5])
def test_lanes_on_cu_halves(torch_dev, small, T):
    """Two lanes with a CU budget of half the device each: each lane sizes its
    grids to half the CUs and still gives the plain call's outputs bit for bit
    (vector path at T <= 2, matrix cores at 5)."""
    torch = torch_dev
    lay, _, wl = small
    n_cus = torch.cuda.get_device_properties(0).multi_processor_count
    say("lanes on half the CUs each, T =", T, "of", n_cus, "CUs")
    lanes = [dm.Lane(lay, max_tokens=T, cus=n_cus // 2) for _ in range(2)]
    for lane in lanes:
        assert lane.cus == n_cus // 2, lane.cus
    cases = []
    for s in (3, 4):
        x = synth.activations(SEED, wl, 0, 40 + 10 * T + s, T, lay.hidden)
        ids, w = synth.routing(SEED, wl, 0, 40 + 10 * T + s, T, lay.n_routed, lay.top_k)
        cases.append((to_dev(torch, x), to_dev(torch, ids), to_dev(torch, w)))
    ref = [dm.moe_layer(lay, *c).cpu().numpy() for c in cases]
    outs = [torch.full((T, lay.hidden), float("nan"), device="cuda") for _ in lanes]
    for rep in range(3):
        for lane, c, o in zip(lanes, cases, outs):
            lane.begin(lay, *c, o)
        for lane in lanes:
            lane.finish(block=True)
        for o, r in zip(outs, ref):
            np.testing.assert_array_equal(o.cpu().numpy(), r)
    for lane in lanes:
        lane.close()
