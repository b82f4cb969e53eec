"""Pins for the oracle's fp9 codec (CPU only).

Each check ties the oracle to something other than its own formula: the fp16
decode route the memoir page's fp9 section describes (code << 7 read as an IEEE
fp16 by numpy), hand-worked fixtures under tests/golden/, brute-force nearest
search for rounding, and format invariants.
"""

import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_kv(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, *v = line.split()
            out[k] = v
    return out


ALL = np.arange(512)
VALS = oracle.decode(ALL)
FINITE = np.isfinite(VALS)
# the 248 non-negative finite codes, by magnitude
POS_CODES = np.arange(0, 0xF8)
POS_VALS = oracle.decode(POS_CODES)


def _fp16_route(codes):
    """The pages' decode route, done by numpy: (code << 7) read as fp16."""
    c = np.asarray(codes).astype(np.uint16)
    return (c << np.uint16(7)).view(np.float16).astype(np.float64)


# ---------------------------------------------------------------- decode ----

def test_decode_matches_fp16_route_all_finite_codes():
    ref = _fp16_route(ALL)
    assert FINITE.sum() == 496
    np.testing.assert_array_equal(VALS[FINITE], ref[FINITE])
    # sign of zero too
    np.testing.assert_array_equal(np.signbit(VALS[FINITE]), np.signbit(ref[FINITE]))


def test_decode_exponent31_class_matches_fp16():
    ref = _fp16_route(ALL)
    e31 = ((ALL >> 3) & 31) == 31
    assert e31.sum() == 16
    np.testing.assert_array_equal(np.isinf(VALS[e31]), np.isinf(ref[e31]))
    np.testing.assert_array_equal(np.isnan(VALS[e31]), np.isnan(ref[e31]))
    np.testing.assert_array_equal(np.signbit(VALS[e31 & np.isinf(ref)]),
                                  np.signbit(ref[e31 & np.isinf(ref)]))


def test_layout_fixture():
    kv = _read_kv("fp9_layout.txt")
    assert int(kv["exponent_bias"][0]) == 15
    # bias: exponent field 15, mantissa 0 is exactly 1.0
    assert oracle.decode([15 << 3])[0] == 1.0
    # sign lives in bit 8
    assert oracle.decode([1 << int(kv["sign_bit"][0]) | (15 << 3)])[0] == -1.0
    # mantissa bits 2..0: each step is 1/8 of the binade
    assert oracle.decode([(15 << 3) | 1])[0] == 1.125
    # exponent bits 7..3: one exponent step doubles
    assert oracle.decode([16 << 3])[0] == 2.0
    # signed zero
    z = oracle.decode([int(kv["negative_zero_code"][0], 16)])[0]
    assert z == 0.0 and np.signbit(z)
    assert int(kv["fp16_shift"][0]) == 7


def test_decode_special_values():
    d = oracle.decode
    assert d([0x000])[0] == 0.0 and not np.signbit(d([0x000])[0])
    assert d([0x0F7])[0] == 61440.0 == oracle.FP9_MAX
    assert d([0x008])[0] == 2.0 ** -14          # smallest normal
    assert d([0x001])[0] == 2.0 ** -17          # smallest subnormal
    assert d([0x007])[0] == 7 * 2.0 ** -17      # largest subnormal
    assert d([0x1F7])[0] == -61440.0
    assert d([0x0F8])[0] == np.inf and d([0x1F8])[0] == -np.inf


def test_decode_monotone_and_distinct():
    # non-negative finite codes are ordered by magnitude and all distinct
    assert np.all(np.diff(POS_VALS) > 0)
    vals = VALS[FINITE]
    assert len(np.unique(vals)) == 495   # +0 and -0 compare equal


# -------------------------------------------------------------- quantize ----

def _brute_force(x):
    """Nearest finite fp9 magnitude, ties to the even code; sign kept."""
    xf = np.asarray(x, dtype=np.float32)
    a = np.abs(xf.astype(np.float64))
    # above the largest fp9 value every input has that value as its nearest
    # candidate; clamping to twice it keeps every distance exact in float64
    # (for 1e38 or inf all distances would otherwise round to the same number)
    a = np.minimum(a, 2.0 * POS_VALS[-1])
    dist = np.abs(a[:, None] - POS_VALS[None, :])
    best = dist.min(axis=1, keepdims=True)
    cand = dist == best
    # among tied candidates take the even code (at most two are tied)
    even = cand & (POS_CODES[None, :] % 2 == 0)
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    mag = POS_CODES[pick]
    return ((np.signbit(xf).astype(np.int64) << 8) | mag).astype(np.uint16)


def _probe_points():
    pts = [0.0, -0.0, np.inf, -np.inf, 61440.0, 61441.0, 63488.0, 65504.0, 1e30,
           np.finfo(np.float32).max, np.finfo(np.float32).tiny,
           float(np.float32(1.4e-45)), 2.0 ** -18, 3 * 2.0 ** -19]
    mids = (POS_VALS[:-1] + POS_VALS[1:]) / 2
    p32 = np.concatenate([POS_VALS, mids]).astype(np.float32)
    assert np.all(p32.astype(np.float64) == np.concatenate([POS_VALS, mids])), \
        "fp9 values and midpoints are exact in float32"
    up = np.nextafter(p32, np.float32(np.inf))
    dn = np.nextafter(p32, np.float32(0))
    rng = np.random.default_rng(1234)
    bits = rng.integers(0, 1 << 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    rnd = bits.view(np.float32)
    rnd = rnd[~np.isnan(rnd)]
    gauss = (rng.standard_normal(50_000) * 0.02).astype(np.float32)
    allp = np.concatenate([np.array(pts, dtype=np.float32), p32, up, dn, rnd, gauss])
    return np.concatenate([allp, -allp])


def test_quantize_matches_brute_force_nearest_even():
    x = _probe_points()
    got = oracle.quantize(x)
    for chunk in range(0, len(x), 20_000):
        sl = slice(chunk, chunk + 20_000)
        np.testing.assert_array_equal(got[sl], _brute_force(x[sl]))


def test_quantize_ties_go_to_even():
    # midway between 1.0 (m=0) and 1.125 (m=1): even wins -> 1.0
    assert oracle.quantize([1.0625])[0] == 0x078
    # midway between 1.125 (m=1) and 1.25 (m=2): even wins -> 1.25
    assert oracle.quantize([1.1875])[0] == 0x07A
    # midway between largest subnormal and smallest normal -> normal (code 8)
    assert oracle.quantize([7.5 * 2.0 ** -17])[0] == 0x008
    # half the smallest subnormal -> +0 ; negative side keeps the sign
    assert oracle.quantize([2.0 ** -18])[0] == 0x000
    assert oracle.quantize([-(2.0 ** -18)])[0] == 0x100


def test_quantize_rounds_once_not_via_fp16():
    # 1.0625 + 2^-20 is just above the 1.0 / 1.125 midpoint; an fp16 detour
    # would first round it onto the midpoint and then tie down to 1.0.
    x = np.float32(1.0625 + 2.0 ** -20)
    assert float(x) == 1.0625 + 2.0 ** -20
    assert oracle.quantize([x])[0] == 0x079
    via16 = oracle.quantize([np.float32(np.float16(x))])[0]
    assert via16 == 0x078


def test_quantize_saturates_and_never_exponent31():
    x = np.array([61440, 61441, 63487, 63488, 65504, 1e38, np.inf], dtype=np.float32)
    np.testing.assert_array_equal(oracle.quantize(x), 0x0F7)
    np.testing.assert_array_equal(oracle.quantize(-x), 0x1F7)
    q = oracle.quantize(_probe_points())
    assert np.all(((q.astype(np.int64) >> 3) & 31) != 31)


def test_quantize_rejects_nan():
    with pytest.raises(ValueError):
        oracle.quantize(np.array([1.0, np.nan], dtype=np.float32))


def test_quantize_roundtrip_all_finite_codes():
    codes = ALL[FINITE]
    np.testing.assert_array_equal(oracle.quantize(VALS[FINITE].astype(np.float32)), codes)


def test_quantize_monotone():
    x = np.sort(_probe_points()[np.isfinite(_probe_points())])
    v = oracle.decode(oracle.quantize(x))
    assert np.all(np.diff(v) >= 0)


# ------------------------------------------------------------------ pack ----

def test_pack_worked_example():
    kv = _read_kv("pack_example.txt")
    vals = np.array([float(v) for v in kv["values"]], dtype=np.float32)
    codes = np.array([int(c, 16) for c in kv["codes"]])
    np.testing.assert_array_equal(oracle.quantize(vals), codes)
    body, sign = oracle.pack(codes[None, :])
    np.testing.assert_array_equal(body[0], [int(b, 16) for b in kv["body"]])
    assert sign.shape == (1, 1) and sign[0, 0] == int(kv["sign"][0], 16)
    np.testing.assert_array_equal(oracle.decode(codes), vals.astype(np.float64))


def test_pack_roundtrip_and_size():
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 512, size=(13, 96))
    body, sign = oracle.pack(codes)
    kv = _read_kv("fp9_layout.txt")
    per8 = int(kv["bytes_per_8_weights"][0])
    assert body.nbytes + sign.nbytes == codes.size * per8 // 8
    assert (body.nbytes + sign.nbytes) / body.nbytes - 1 == float(kv["overhead_vs_fp8_percent"][0]) / 100
    np.testing.assert_array_equal(oracle.unpack(body, sign), codes)
    np.testing.assert_array_equal(oracle.decode_planes(body, sign), oracle.decode(codes))


def test_pack_rejects_ragged_rows():
    with pytest.raises(ValueError):
        oracle.pack(np.zeros((2, 12), dtype=np.int64))
