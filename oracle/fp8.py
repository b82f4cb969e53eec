"""fp8 block-scaled weights -> fp9, oracle side (float64 numpy).  TEST INFRASTRUCTURE ONLY.

The pages say the models' official checkpoints are fp8 (duck-llm memoir page
"一鸭三吃：我把评测鸭变成了满血 DeepSeek-V3.2 推理系统", section
"真正埋下伏笔的是内存；R1 之后，问题第一次被改写": the release format is fp8,
about 688 GB) with a 128 x 128 block-scale layout (same page, section
"先用 Qwen3 练级，再让 Qwen3.5 充当高压试炼场": Qwen3's fp8 checkpoints use
the same 128 x 128 block-scale format as DeepSeek-V3).  They do not spell the
format out.  Readings taken here:

* the 8-bit code is E4M3 with exponent bias 7, subnormals, no infinities,
  and NaN only for exponent 15 with mantissa 7 (codes 0x7F and 0xFF): the
  finite-only E4M3 variant of the OCP 8-bit floating-point format, largest
  magnitude 448;
* a weight matrix [rows, cols] comes with one float32 scale per 128 x 128
  block (block (i, j) covers rows 128i..128i+127 and cols 128j..128j+127; the
  last blocks may be partial), and the weight is value(code) * scale;
* the conversion to fp9 rounds once, from the exact product (a 4-bit
  significand times a 24-bit one fits float64 exactly), with the fp9
  quantizer's rounding (nearest, ties to even, saturate at 61440); a NaN code
  or a NaN product is an error.  Every finite E4M3 value is itself an fp9 value
  (3 mantissa bits, a wider exponent range), so with a power-of-two scale the
  conversion is exact unless it saturates or underflows.
"""

import numpy as np

from .fp9 import quantize_f64

#: largest finite E4M3 magnitude: exponent 15, mantissa 6.
E4M3_MAX = 448.0
BLOCK = 128


def decode_e4m3(codes):
    """8-bit E4M3 codes -> float64 values by the closed form.

    value = (-1)^s * 2^(e-7) * (1 + m/8)   for 1 <= e <= 15 (not e = 15, m = 7)
          = (-1)^s * 2^(-6)  * (m/8)       for e = 0 (subnormal)
          = NaN                            for e = 15, m = 7
    """
    c = np.asarray(codes).astype(np.int64)
    if np.any((c < 0) | (c > 0xFF)):
        raise ValueError("E4M3 codes are bytes")
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    mf = m.astype(np.float64)
    mag = np.where(e == 0, np.ldexp(mf / 8.0, -6), np.ldexp(1.0 + mf / 8.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def block_scales(scale, rows, cols, block=BLOCK):
    """The per-element scale [rows, cols] of a [ceil(rows/b), ceil(cols/b)] grid."""
    sc = np.asarray(scale, dtype=np.float32).astype(np.float64)
    nb_r, nb_c = -(-rows // block), -(-cols // block)
    if sc.shape != (nb_r, nb_c):
        raise ValueError("scale grid must be [%d, %d]" % (nb_r, nb_c))
    out = np.empty((rows, cols), dtype=np.float64)
    for i in range(nb_r):
        for j in range(nb_c):
            out[i * block:(i + 1) * block, j * block:(j + 1) * block] = sc[i, j]
    return out


def dequantize(codes, scale, block=BLOCK):
    """Exact float64 weights value(code) * scale of the code's block."""
    c = np.asarray(codes)
    if c.ndim != 2:
        raise ValueError("codes must be [rows, cols]")
    return decode_e4m3(c) * block_scales(scale, c.shape[0], c.shape[1], block)


def fp8_to_fp9(codes, scale, block=BLOCK):
    """E4M3 codes [rows, cols] with block scales -> fp9 codes [rows, cols] (uint16)."""
    w = dequantize(codes, scale, block)
    if np.any(np.isnan(w)):
        raise ValueError("fp8 -> fp9: NaN code or scale")
    return quantize_f64(w)
