"""GPU parity of the fp8 (E4M3, block-scaled) -> fp9 converter.

Bar: the device planes bit-exact against the oracle's conversion (one rounding
from the exact product) packed by the oracle's packer; an expert filled from
fp8 on the device matches the oracle's expert on its own conversion within the
f32 tolerance.
"""

import numpy as np
import pytest

import oracle
from oracle import fp8 as ofp8
from gpu_util import check_close, say
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


def convert(torch, codes, scale, block=128, flag=None):
    body, sign = dm.fp8_to_fp9_device(to_dev(torch, codes), to_dev(torch, scale), block,
                                      nonfinite=flag)
    return body.cpu().numpy(), sign.cpu().numpy()


def test_every_code_under_many_scales(torch_dev):
    """All 254 non-NaN codes in every block; each block a different scale: powers
    of two from 2^-24 to 2^12, and float32 values over 16 decades."""
    torch = torch_dev
    rng = np.random.default_rng(11)
    rows, cols, block = 300, 520, 128             # 3 x 5 blocks, the last ones partial
    base = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    for trial in range(4):
        codes = rng.choice(base, size=(rows, cols)).astype(np.uint8)
        codes[:2, :254] = base                     # every code at least once
        if trial == 0:
            scale = (2.0 ** rng.integers(-24, 13, size=(3, 5))).astype(np.float32)
        else:
            scale = (10.0 ** rng.uniform(-12, 4, size=(3, 5))).astype(np.float32)
            scale *= np.where(rng.random((3, 5)) < 0.2, -1, 1).astype(np.float32)
        say("fp8 -> fp9 all codes, trial", trial)
        body, sign = convert(torch, codes, scale, block)
        rb, rs = oracle.pack(oracle.fp8_to_fp9(codes, scale, block))
        np.testing.assert_array_equal(body, rb)
        np.testing.assert_array_equal(sign, rs)


def test_double_rounding_case_on_device(torch_dev):
    """1.125 times a scale that puts the product just above the fp9 tie 1.0625:
    one rounding gives 1.125 (a float32 product would have given 1.0)."""
    torch = torch_dev
    v = 1.125
    s = np.float32(1.0625 / v)
    while v * float(s) <= 1.0625:
        s = np.nextafter(s, np.float32(2))
    assert float(np.float32(v * float(s))) == 1.0625
    codes = np.full((1, 8), 0x39, dtype=np.uint8)
    body, sign = convert(torch, codes, np.array([[s]], dtype=np.float32))
    assert oracle.unpack(body, sign)[0, 0] == 0x079
    np.testing.assert_array_equal(oracle.unpack(body, sign),
                                  oracle.fp8_to_fp9(codes, np.array([[s]], np.float32)))


def test_nan_code_flag_and_block_sizes(torch_dev):
    torch = torch_dev
    say("fp8 NaN flag, block 8 and 64")
    codes, scale = synth.fp8_weights(SEED, 150, 0, 0, 0, (40, 48), block=8)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    body, sign = convert(torch, codes, scale, 8, flag)
    assert int(flag.item()) == 0
    np.testing.assert_array_equal(oracle.unpack(body, sign), oracle.fp8_to_fp9(codes, scale, 8))
    codes2, scale2 = synth.fp8_weights(SEED, 150, 0, 0, 1, (70, 200), block=64)
    body, sign = convert(torch, codes2, scale2, 64)
    np.testing.assert_array_equal(oracle.unpack(body, sign), oracle.fp8_to_fp9(codes2, scale2, 64))
    bad = codes.copy()
    bad[3, 5] = 0xFF
    convert(torch, bad, scale, 8, flag)
    assert int(flag.item()) == 1


def test_full_size_expert_from_fp8(torch_dev):
    """One 7168/2048 expert (and the shared one) converted on the device: planes
    bit-exact, then the expert FFN against the oracle's expert on its own codes."""
    torch = torch_dev
    H, I, wl = 7168, 2048, 151
    lay = dm.Layer(H, I, 1, 1)
    oc = {}
    for e in range(2):
        mats = [synth.fp8_weights(SEED, wl, 0, e, m, shp) for m, shp in
                enumerate(synth.expert_shapes(H, I))]
        say("fp8 expert", e, "to fp9 on the device")
        lay.set_expert_fp8(e, *[(to_dev(torch, c), to_dev(torch, s)) for c, s in mats])
        oc[e] = tuple(ofp8.fp8_to_fp9(c, s) for c, s in mats)
    torch.cuda.synchronize()
    mat = I * H
    gb, gs = oracle.pack(np.concatenate([oc[0][0], oc[0][1]], axis=0))
    np.testing.assert_array_equal(lay.gu_body[:2 * mat].cpu().numpy(), gb.reshape(-1))
    np.testing.assert_array_equal(lay.gu_sign[:2 * mat // 8].cpu().numpy(), gs.reshape(-1))
    db, ds = oracle.pack(oc[1][2])
    np.testing.assert_array_equal(lay.dn_body[mat:].cpu().numpy(), db.reshape(-1))
    np.testing.assert_array_equal(lay.dn_sign[mat // 8:].cpu().numpy(), ds.reshape(-1))
    x = synth.activations(SEED, wl, 0, 1, 2, H)
    for e in range(2):
        got = dm.expert_ffn(lay, e, to_dev(torch, x)).cpu().numpy()
        check_close(got, oracle.expert_ffn(oc[e], x), "fp8 expert %d" % e)
