"""fp9 codec, oracle side (float64 numpy).  TEST INFRASTRUCTURE ONLY.

Follows the fp9 section of the duck-llm memoir page
("一鸭三吃：我把评测鸭变成了满血 DeepSeek-V3.2 推理系统", section
"在只有 AVX2 的 N100 上，我先做出了单核 MLP fp9"):

* bit-layout figure: a 9-bit code holds the sign in bit 8, a 5-bit exponent in
  bits 7..3 whose bias is 15 (the same bias as IEEE fp16), and a 3-bit mantissa
  in bits 2..0;
* storage paragraph: the code is stored as a body byte (the 8 bits below the
  sign) plus a separate sign bitplane in which the signs of 8 consecutive
  weights share one byte, so 8 weights cost 9 bytes;
* decode paragraph: because the bias matches fp16, the code shifted left by 7
  is a valid fp16 bit pattern; +0 and -0 come out right with no special case.

The pages do not describe the quantizer.  The reading taken here: round to
nearest with ties to even, saturate at the largest finite magnitude 61440
(exponent 30, mantissa 7) and never produce exponent 31; NaN input is an error.
Readings for details the pages leave open:

* sign bit order inside a sign byte: least significant bit first (bit i of
  sign byte j belongs to element 8*j + i along the row);
* exponent-31 codes are never produced; when decoded they follow fp16
  (mantissa 0 -> infinity, otherwise NaN);
* the sign of zero is kept (a tiny negative input gives code 0x100, -0.0).
"""

import numpy as np

#: largest finite fp9 magnitude: exponent field 30, mantissa 7.
FP9_MAX = 61440.0

_BIAS = 15
_EXP_MASK = 0x1F
_MAN_BITS = 3


def _fields(codes):
    c = np.asarray(codes).astype(np.int64)
    if np.any((c < 0) | (c > 0x1FF)):
        raise ValueError("fp9 codes are 9-bit values in [0, 511]")
    s = (c >> 8) & 1
    e = (c >> _MAN_BITS) & _EXP_MASK
    m = c & 0x7
    return s, e, m


def decode(codes):
    """9-bit codes -> float64 values, by the closed form of the layout figure.

    value = (-1)^s * 2^(e-15) * (1 + m/8)   for 1 <= e <= 30
          = (-1)^s * 2^(-14)  * (m/8)       for e = 0 (subnormal)
          = (-1)^s * inf if m == 0 else NaN for e = 31 (never produced)
    """
    s, e, m = _fields(codes)
    mf = m.astype(np.float64)
    normal = np.ldexp(1.0 + mf / 8.0, (e - _BIAS).astype(np.int64))
    subnormal = np.ldexp(mf / 8.0, 1 - _BIAS)
    mag = np.where(e == 0, subnormal, normal)
    mag = np.where(e == 31, np.where(m == 0, np.inf, np.nan), mag)
    return np.where(s == 1, -mag, mag)


def quantize(x):
    """float32 values -> 9-bit codes (uint16), round to nearest, ties to even.

    Computed directly from the float32 value in float64 (exact), never through
    fp16: rounding to fp16 first and then to fp9 would round twice.
      1. NaN is rejected.
      2. |x| >= 61440 (including infinity) saturates to exponent 30, mantissa 7.
      3. |x| <  2^-14 (fp9 subnormal range): n = round_half_even(|x| / 2^-17),
         0 <= n <= 8; the magnitude code is n (n = 8 is exponent 1, mantissa 0).
      4. otherwise E = floor(log2 |x|), n = round_half_even(|x| / 2^(E-3)),
         8 <= n <= 16; n = 16 carries into the exponent (E+1, n = 8).  The
         magnitude code is (E+15) << 3 | (n - 8).
      5. the sign bit of x (also of -0.0) becomes bit 8.
    """
    xf = np.asarray(x, dtype=np.float32)
    if np.any(np.isnan(xf)):
        raise ValueError("fp9 quantize: NaN input")
    return _quantize_f64(xf.astype(np.float64), np.signbit(xf))


def quantize_f64(x):
    """float64 values -> 9-bit codes with the same rounding as `quantize`.

    For values that are not float32 numbers (such as an fp8 value times a
    block scale, computed exactly): one rounding from the exact value, where
    rounding to float32 first could round twice.  For float32 inputs it equals
    `quantize`.
    """
    xd = np.asarray(x, dtype=np.float64)
    if np.any(np.isnan(xd)):
        raise ValueError("fp9 quantize: NaN input")
    return _quantize_f64(xd, np.signbit(xd))


def _quantize_f64(xd, neg):
    """Steps 2..5 of `quantize` on exact float64 values xd with sign bits neg."""
    a = np.abs(xd)

    mag = np.zeros(a.shape, dtype=np.int64)

    sat = a >= FP9_MAX
    sub = a < 2.0 ** (1 - _BIAS)
    nor = ~sat & ~sub

    mag[sat] = (30 << _MAN_BITS) | 7

    # subnormal range: multiples of 2^-17
    n_sub = np.rint(a[sub] * 2.0 ** 17).astype(np.int64)
    mag[sub] = n_sub

    # normal range: 8 significand steps per binade
    an = a[nor]
    _, k = np.frexp(an)          # an = f * 2^k, f in [0.5, 1)
    E = k.astype(np.int64) - 1   # floor(log2 an)
    n = np.rint(np.ldexp(an, (3 - E))).astype(np.int64)
    carry = n == 16
    E = E + carry
    n = np.where(carry, 8, n)
    mag[nor] = ((E + _BIAS) << _MAN_BITS) | (n - 8)

    code = (neg.astype(np.int64) << 8) | mag
    return code.astype(np.uint16)


def pack(codes):
    """codes [rows, cols] -> (body uint8 [rows, cols], sign uint8 [rows, cols/8]).

    body = the low 8 bits (exponent and mantissa); sign byte j of a row holds the
    sign bits of elements 8j..8j+7, element 8j+i in bit i.  Rows never share a
    sign byte, so cols must be a multiple of 8.
    """
    c = np.asarray(codes).astype(np.int64)
    if c.ndim != 2 or c.shape[1] % 8 != 0:
        raise ValueError("pack: codes must be [rows, cols] with cols % 8 == 0")
    rows, cols = c.shape
    body = (c & 0xFF).astype(np.uint8)
    sbits = ((c >> 8) & 1).reshape(rows, cols // 8, 8)
    weights = (1 << np.arange(8, dtype=np.int64))
    sign = (sbits * weights).sum(axis=2).astype(np.uint8)
    return body, sign


def unpack(body, sign):
    """(body [rows, cols], sign [rows, cols/8]) -> codes [rows, cols] (uint16)."""
    b = np.asarray(body).astype(np.int64)
    s = np.asarray(sign).astype(np.int64)
    rows, cols = b.shape
    if s.shape != (rows, cols // 8) or cols % 8 != 0:
        raise ValueError("unpack: plane shapes do not match")
    bits = (s[:, :, None] >> np.arange(8)[None, None, :]) & 1
    return (b | (bits.reshape(rows, cols) << 8)).astype(np.uint16)


def decode_planes(body, sign):
    """Decode stored planes straight to float64 values [rows, cols]."""
    return decode(unpack(body, sign))
