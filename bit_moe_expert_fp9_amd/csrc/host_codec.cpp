// host_codec.cpp - host side of libduckmoe: fp32 -> fp9 quantizer/packer and
// error strings.
//
// The fp9 format is the one of the duck-llm memoir page ("一鸭三吃：我把评测鸭
// 变成了满血 DeepSeek-V3.2 推理系统", section "在只有 AVX2 的 N100 上，我先做出
// 了单核 MLP fp9"): code = s<<8 | e<<3 | m, exponent bias 15, stored as a body
// byte (e, m) plus one sign bit per weight packed 8 to a byte.  The pages do
// not describe how weights get into fp9; this quantizer rounds to nearest with
// ties to even, saturates at +-61440 (e = 30, m = 7), never emits e = 31, keeps
// the sign of zero and rejects NaN.
//
// It works on the float32 bit pattern with integer arithmetic only, rounding
// once from the full 24-bit significand (a detour through fp16 would round
// twice).
#include <stdint.h>
#include <string.h>

#include "../../include/duckmoe.h"

namespace {

constexpr uint32_t kAbsMask = 0x7fffffffu;
constexpr uint32_t kInfBits = 0x7f800000u;
constexpr uint32_t kSatBits = 0x47700000u;  // 61440.0f = 2^15 * 1.875
constexpr uint32_t kSatCode = (30u << 3) | 7u;

// Shift right by `sh` (>= 1) rounding to nearest, ties to even.
inline uint32_t shr_rne(uint32_t v, int sh) {
  if (sh >= 32) return 0u;  // v < 2^24 <= half of 2^sh for sh >= 25
  const uint32_t q = v >> sh;
  const uint32_t rem = v & ((1u << sh) - 1u);
  const uint32_t half = 1u << (sh - 1);
  return q + ((rem > half || (rem == half && (q & 1u))) ? 1u : 0u);
}

// Magnitude code (9th bit excluded) of a finite non-NaN |x| given by its bits.
inline uint32_t fp9_mag(uint32_t a) {
  if (a >= kSatBits) return kSatCode;          // includes +inf
  const int e32 = (int)(a >> 23);
  const uint32_t man = a & 0x7fffffu;
  if (e32 >= 113) {                            // |x| >= 2^-14: fp9 normal range
    // value = (8 + m') * 2^(E-3) with E = e32 - 127; keep 3 mantissa bits.
    // (e << 3) + mantissa, with the rounding carry running into the exponent.
    const uint32_t top = ((uint32_t)(e32 - 112) << 3) | (man >> 20);
    const uint32_t rem = man & 0xfffffu;
    const uint32_t half = 0x80000u;
    return top + ((rem > half || (rem == half && (top & 1u))) ? 1u : 0u);
  }
  // |x| < 2^-14: count steps of 2^-17.  |x| = sig * 2^(max(e32,1) - 150).
  const uint32_t sig = e32 ? (man | 0x800000u) : man;
  const int ebits = e32 ? e32 : 1;
  return shr_rne(sig, 133 - ebits);            // 0..8; 8 is e = 1, m = 0
}

}  // namespace

extern "C" {

const char *duckmoe_strerror(int code) {
  switch (code) {
    case DUCKMOE_OK: return "ok";
    case DUCKMOE_EINVAL: return "invalid argument (null or misaligned pointer, or index out of range)";
    case DUCKMOE_ESHAPE: return "unsupported shape";
    case DUCKMOE_ENONFINITE: return "NaN in quantizer input";
    case DUCKMOE_EWORKSPACE: return "workspace too small";
    case DUCKMOE_EHIP: return "HIP runtime error";
    default: return "unknown error code";
  }
}

int duckmoe_quantize_fp9(const float *w, int64_t rows, int64_t cols, uint8_t *body,
                         uint8_t *sign) {
  if (rows < 0 || cols < 0) return DUCKMOE_EINVAL;
  if (cols % 8) return DUCKMOE_ESHAPE;
  if (rows == 0 || cols == 0) return DUCKMOE_OK;
  if (!w || !body || !sign) return DUCKMOE_EINVAL;
  const int64_t n = rows * cols;
  int bad = 0;
  for (int64_t g = 0; g < n / 8; ++g) {
    uint32_t sbyte = 0;
    for (int i = 0; i < 8; ++i) {
      uint32_t bits;
      memcpy(&bits, w + 8 * g + i, 4);
      const uint32_t a = bits & kAbsMask;
      bad |= a > kInfBits;
      body[8 * g + i] = (uint8_t)fp9_mag(a > kInfBits ? 0u : a);
      sbyte |= (bits >> 31) << i;
    }
    sign[g] = (uint8_t)sbyte;
  }
  return bad ? DUCKMOE_ENONFINITE : DUCKMOE_OK;
}

}  // extern "C"
