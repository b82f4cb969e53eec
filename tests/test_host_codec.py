"""Host quantizer/packer of the library against the oracle (CPU).

The oracle's own rounding is pinned in test_oracle_fp9.py; here the C++ codec
must reproduce it bit for bit: codes (body byte + sign bit) and sign-plane
layout.  A sample of float32 bit patterns that covers every exponent is
checked first; then all 2^32 patterns, in 256 chunks over up to 8 worker
processes (about a minute on 8 cores; DUCKMOE_QUICK=1 skips that sweep).
"""

import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np
import pytest

from lib_util import ensure_built

import oracle


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()


def _compare(bits):
    """bits: uint32 patterns (no NaNs) -> number of mismatching codes."""
    import bit_moe_expert_fp9_amd as dm
    x = bits.view(np.float32)
    n = (len(x) // 8) * 8
    x = x[:n]
    body, sign = dm.quantize_fp9(x.reshape(-1, 8))
    got = oracle.unpack(body, sign).reshape(-1)
    ref = oracle.quantize(x)
    return int(np.count_nonzero(got != ref))


def _no_nan(bits):
    return bits[(bits & 0x7fffffff) <= 0x7f800000]


def test_sampled_bit_patterns():
    rng = np.random.default_rng(99)
    parts = [
        np.arange(0, 1 << 32, 1021, dtype=np.uint64).astype(np.uint32),
        rng.integers(0, 1 << 32, size=1 << 21, dtype=np.uint64).astype(np.uint32),
    ]
    # every mantissa step of 7 around the subnormal/normal and saturation edges
    for e in (110, 111, 112, 113, 141, 142, 143):
        m = np.arange(0, 1 << 23, 7, dtype=np.uint32)
        parts.append((np.uint32(e) << np.uint32(23)) | m)
        parts.append(np.uint32(0x80000000) | (np.uint32(e) << np.uint32(23)) | m)
    bits = _no_nan(np.concatenate(parts))
    assert _compare(bits) == 0


def test_special_values():
    vals = np.array([0.0, -0.0, np.inf, -np.inf, 61440, 61441, 65504, 1e38, 2 ** -17,
                     -2 ** -18, 3 * 2 ** -19, 1.0625, 1.0625 + 2 ** -20, 7.5 * 2 ** -17],
                    dtype=np.float32)
    bits = np.concatenate([vals, np.zeros(2, np.float32)]).view(np.uint32)
    assert _compare(bits) == 0


def test_plane_layout_matches_oracle_pack():
    import bit_moe_expert_fp9_amd as dm
    rng = np.random.default_rng(5)
    for shape in [(3, 8), (5, 24), (16, 1024), (7, 7168)]:
        w = (rng.standard_normal(shape) * 0.02).astype(np.float32)
        w[0, :3] = [-0.0, 1e-9, -1e-9]
        body, sign = dm.quantize_fp9(w)
        ob, os_ = oracle.pack(oracle.quantize(w))
        np.testing.assert_array_equal(body, ob)
        np.testing.assert_array_equal(sign, os_)
        assert body.nbytes + sign.nbytes == w.size * 9 // 8


def test_nan_is_rejected():
    import bit_moe_expert_fp9_amd as dm
    w = np.ones((1, 16), dtype=np.float32)
    w[0, 9] = np.nan
    with pytest.raises(dm.DuckMoeError):
        dm.quantize_fp9(w)


def _chunk(start):
    ensure_built()
    bits = np.arange(start, start + (1 << 24), dtype=np.uint64).astype(np.uint32)
    return _compare(_no_nan(bits))


@pytest.mark.exhaustive
def test_all_float32_bit_patterns():
    starts = list(range(0, 1 << 32, 1 << 24))
    workers = min(8, len(os.sched_getaffinity(0)))
    with ProcessPoolExecutor(workers) as ex:
        bad = sum(ex.map(_chunk, starts))
    assert bad == 0
