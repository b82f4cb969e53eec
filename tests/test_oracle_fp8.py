"""Pins of the oracle's fp8 (E4M3, 128 x 128 block scale) -> fp9 conversion.

What fixes it, independently of its own formulas:
* a hand-worked value table of the E4M3 format (tests/golden/e4m3_values.txt);
* every finite E4M3 value is an fp9 value, with the fp9 code (s, e + 8, m) for
  normal codes: an identity between two formats pinned on their own;
* one rounding from the exact product, checked against a brute-force nearest
  search in exact rational arithmetic, including a product where rounding to
  float32 first would round twice;
* power-of-two scales shift the fp9 exponent and nothing else; block indexing
  on ragged shapes.
"""

import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import fp8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_values.txt")


def golden():
    out = []
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if line:
            c, v = line.split()
            out.append((int(c, 16), float(v)))
    return out


def test_e4m3_golden_values():
    for code, val in golden():
        got = oracle.decode_e4m3([code])[0]
        if np.isnan(val):
            assert np.isnan(got), hex(code)
        else:
            assert got == val and np.signbit(got) == np.signbit(val), (hex(code), got, val)


def test_e4m3_order_and_count():
    pos = oracle.decode_e4m3(np.arange(0x7F))
    assert np.all(np.diff(pos) > 0)                 # 0x00..0x7E strictly increasing
    np.testing.assert_array_equal(oracle.decode_e4m3(np.arange(0x80, 0xFF)), -pos)
    assert np.isnan(oracle.decode_e4m3(np.arange(256))).sum() == 2
    assert pos[-1] == oracle.E4M3_MAX


def test_every_e4m3_value_is_an_fp9_value():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F])
    v = oracle.decode_e4m3(codes)
    f9 = oracle.quantize_f64(v)
    np.testing.assert_array_equal(oracle.decode(f9), v)
    # normal codes map field by field: exponent + 8, same mantissa, same sign
    s, e, m = codes >> 7, (codes >> 3) & 15, codes & 7
    nz = e > 0
    np.testing.assert_array_equal(f9[nz], (s[nz] << 8) | ((e[nz] + 8) << 3) | m[nz])


def nearest_fp9(x):
    """Brute force: the finite fp9 value nearest to the exact rational x, ties to
    the even mantissa; magnitudes above the largest value saturate."""
    codes = [c for c in range(256) if (c >> 3) != 31]
    vals = [(Fraction(float(oracle.decode([c])[0])), c) for c in codes]
    ax = abs(x)
    best = min(vals, key=lambda vc: (abs(vc[0] - ax), vc[1] & 1))
    if ax >= Fraction(61440):
        best = (Fraction(61440), 0xF7)
    return best[1] | (0x100 if x < 0 else 0)


def test_one_rounding_from_the_exact_product():
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 256, size=400)
    codes = codes[(codes & 0x7F) != 0x7F]
    scales = np.concatenate([(rng.standard_normal(200) * 1e-3).astype(np.float32),
                             rng.uniform(1e-6, 300, 200).astype(np.float32)])[: len(codes)]
    got = oracle.quantize_f64(oracle.decode_e4m3(codes) * scales.astype(np.float64))
    for c, sc, g in zip(codes, scales, got):
        exact = Fraction(float(oracle.decode_e4m3([c])[0])) * Fraction(float(sc))
        if exact == 0:
            continue  # the sign of an exact zero is the product's sign bit; checked below
        assert int(g) == nearest_fp9(exact), (hex(int(c)), float(sc))


def test_double_rounding_case():
    """A product just above an fp9 tie that float32 rounds onto the tie: rounding
    the float32 value would go to the even neighbour (down), the exact one goes up."""
    v = oracle.decode_e4m3([0x39])[0]                 # 1.125
    tie = 1.0625                                      # between fp9 1.0 and 1.125
    s = np.float32(tie / v)
    while float(v) * float(s) <= tie:
        s = np.nextafter(s, np.float32(2))
    prod = float(v) * float(s)                        # exact in float64
    assert prod > tie and float(np.float32(prod)) == tie
    assert oracle.quantize_f64([prod])[0] == nearest_fp9(Fraction(prod)) == 0x079  # 1.125
    assert oracle.quantize(np.float32(prod)) == 0x078                              # 1.0


def test_power_of_two_scales_shift_the_exponent():
    codes = np.array([[0x38, 0x39, 0xBF, 0x01, 0x00, 0x80, 0x7E, 0x08]])
    for k in (-8, -3, 0, 5, 7):
        got = oracle.fp8_to_fp9(codes, np.array([[2.0 ** k]], dtype=np.float32))
        np.testing.assert_array_equal(oracle.decode(got), oracle.decode_e4m3(codes) * 2.0 ** k)
    # 448 * 2^8 saturates; 2^-9 * 2^-10 is below half the smallest fp9 step
    assert oracle.fp8_to_fp9(np.array([[0x7E] * 8]), np.array([[256.0]], np.float32))[0, 0] == 0xF7
    assert oracle.fp8_to_fp9(np.array([[0x81] * 8]), np.array([[2.0 ** -10]], np.float32))[0, 0] == 0x100


def test_block_indexing_on_ragged_shapes():
    rows, cols = 130, 264                             # 2 x 3 blocks, last ones partial
    codes = np.full((rows, cols), 0x38)               # 1.0 everywhere
    scale = np.array([[1, 2, 4], [8, 16, 32]], dtype=np.float32)
    got = oracle.decode(oracle.fp8_to_fp9(codes, scale))
    assert got[0, 0] == 1 and got[127, 127] == 1 and got[127, 128] == 2 and got[0, 263] == 4
    assert got[128, 0] == 8 and got[129, 255] == 16 and got[129, 256] == 32
    assert np.unique(got).size == 6
    with pytest.raises(ValueError):
        oracle.fp8_to_fp9(codes, scale[:, :2])


def test_nan_is_rejected():
    with pytest.raises(ValueError):
        oracle.fp8_to_fp9(np.array([[0x7F] + [0] * 7]), np.ones((1, 1), np.float32))
    with pytest.raises(ValueError):
        oracle.fp8_to_fp9(np.zeros((1, 8), np.int64), np.full((1, 1), np.nan, np.float32))


def test_quantize_f64_equals_quantize_on_float32():
    x = np.random.default_rng(9).standard_normal(10000).astype(np.float32) * np.float32(0.02)
    np.testing.assert_array_equal(oracle.quantize_f64(x.astype(np.float64)), oracle.quantize(x))
    assert fp8.BLOCK == 128
