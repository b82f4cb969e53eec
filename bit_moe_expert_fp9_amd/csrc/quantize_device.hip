// quantize_device.hip - fp32 -> fp9 quantizer and packer on the GPU.
//
// The same function as the host quantizer (duck-llm memoir page
// "一鸭三吃：我把评测鸭变成了满血 DeepSeek-V3.2 推理系统", section
// "在只有 AVX2 的 N100 上，我先做出了单核 MLP fp9": 9-bit code s|eeeee|mmm,
// exponent bias 15, body byte + sign bitplane), computed from the float32 bit
// pattern with integer operations only:
//   - round to nearest, ties to even, directly from float32 (never via fp16);
//   - |x| >= 61440 and +-inf saturate to exponent 30, mantissa 7; exponent 31
//     is never produced;
//   - below 2^-14 the code is the subnormal count n = RNE(|x| / 2^-17) in
//     0..8, where n = 8 is, bit for bit, the smallest normal code;
//   - the sign of zero is kept; NaN raises a flag (its code is unspecified).
// One thread packs one group of 8 consecutive weights: 8 body bytes and the
// sign byte they share (weight 8j+i of a row in bit i of sign byte j).
//
// The same file converts fp8 checkpoints (same page, sections
// "真正埋下伏笔的是内存；R1 之后，问题第一次被改写" and "先用 Qwen3 练级，再让
// Qwen3.5 充当高压试炼场": the released weights are fp8 with a 128 x 128
// block-scale format).  The code is read as finite-only E4M3 (bias 7,
// subnormals, NaN = exponent 15 with mantissa 7), the weight as value * the
// float32 scale of its block, and the fp9 code is rounded once from the exact
// product: a 4-bit significand times a 24-bit one is exact in float64, so the
// product is formed in double and rounded from its bit pattern.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/duckmoe.h"

namespace duckmoe {
namespace {

constexpr uint32_t kSatBits = 0x47700000u;  // 61440.0f
constexpr uint32_t kMinNormalBits = 0x38800000u;  // 2^-14

// add 1 to q when the discarded low bits rem (half = the weight of their top
// bit) round it up under ties-to-even
__device__ __forceinline__ uint32_t rne(uint32_t q, uint32_t rem, uint32_t half) {
  return q + ((rem > half || (rem == half && (q & 1u))) ? 1u : 0u);
}

__device__ __forceinline__ uint32_t fp9_code(uint32_t bits, bool &nan) {
  const uint32_t s = bits >> 31, a = bits & 0x7fffffffu;
  uint32_t c;
  if (a > 0x7f800000u) {
    nan = true;
    c = 0u;
  } else if (a >= kSatBits) {
    c = 0xF7u;
  } else if (a >= kMinNormalBits) {
    // exponent (E - 127) + 15 in bits 7..3 and the top 3 mantissa bits; a
    // round-up carry out of the mantissa moves to the next exponent, which is
    // the right result (and never reaches exponent 31 below 61440)
    const uint32_t m = a & 0x7fffffu;
    c = rne((((a >> 23) - 112u) << 3) | (m >> 20), m & 0xfffffu, 0x80000u);
  } else {
    const uint32_t eb = a >> 23;  // biased float32 exponent, <= 112 here
    if (eb <= 108u) {             // |x| < 2^-18 (float32 subnormals included)
      c = 0u;
    } else {                      // |x| in [2^-18, 2^-14): n = sig * 2^(eb - 133)
      const uint32_t sig = 0x800000u | (a & 0x7fffffu);
      const uint32_t sh = 133u - eb;  // 21 .. 24
      c = rne(sig >> sh, sig & ((1u << sh) - 1u), 1u << (sh - 1u));
    }
  }
  return c | (s << 8);
}

// The same rounding from a float64 value (exponent bias 1023, 52 mantissa bits).
__device__ __forceinline__ uint32_t fp9_code_f64(double v, bool &nan) {
  const uint64_t bits = (uint64_t)__double_as_longlong(v);
  const uint32_t s = (uint32_t)(bits >> 63);
  const uint64_t a = bits & 0x7fffffffffffffffull;
  const uint64_t man = a & 0xfffffffffffffull;
  const uint32_t eb = (uint32_t)(a >> 52);
  uint32_t c;
  if (a > 0x7ff0000000000000ull) {
    nan = true;
    c = 0u;
  } else if (a >= 0x40EE000000000000ull) {  // 61440 and above, infinity included
    c = 0xF7u;
  } else if (a >= 0x3F10000000000000ull) {  // 2^-14 and above: exponent eb - 1008
    const uint64_t rem = man & ((1ull << 49) - 1ull), half = 1ull << 48;
    const uint32_t q = ((eb - 1008u) << 3) | (uint32_t)(man >> 49);
    c = q + ((rem > half || (rem == half && (q & 1u))) ? 1u : 0u);
  } else if (eb <= 1004u) {                 // below 2^-18
    c = 0u;
  } else {                                  // [2^-18, 2^-14): n = sig * 2^(eb - 1058)
    const uint64_t sig = (1ull << 52) | man;
    const uint32_t sh = 1058u - eb;         // 50 .. 53
    const uint64_t rem = sig & ((1ull << sh) - 1ull), half = 1ull << (sh - 1u);
    const uint32_t q = (uint32_t)(sig >> sh);
    c = q + ((rem > half || (rem == half && (q & 1u))) ? 1u : 0u);
  }
  return c | (s << 8);
}

// finite-only E4M3 -> float (exact); NaN for exponent 15 with mantissa 7
__device__ __forceinline__ float e4m3_value(uint32_t b) {
  const uint32_t s = (b >> 7) & 1u, e = (b >> 3) & 15u, m = b & 7u;
  float v;
  if (e == 0u)
    v = (float)m * 0x1p-9f;
  else if (e == 15u && m == 7u)
    v = __builtin_nanf("");
  else
    v = __uint_as_float(((e + 120u) << 23) | (m << 20));
  return s ? -v : v;
}

__global__ __launch_bounds__(256) void k_fp8_to_fp9(const uint2 *__restrict__ fp8,
                                                    const float *__restrict__ scale,
                                                    int64_t groups, int64_t cols, int32_t block,
                                                    int64_t nbc, uint2 *__restrict__ body,
                                                    uint8_t *__restrict__ sign,
                                                    int32_t *__restrict__ nonfinite) {
  bool nan = false;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t gpr = cols / 8;  // groups per row
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < groups; g += stride) {
    const int64_t row = g / gpr, col = (g - row * gpr) * 8;
    const double sc = (double)scale[(row / block) * nbc + col / block];
    const uint2 in = fp8[g];
    uint32_t b[2] = {0u, 0u}, sg = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t byte = ((i < 4 ? in.x : in.y) >> (8 * (i & 3))) & 0xFFu;
      const uint32_t c = fp9_code_f64((double)e4m3_value(byte) * sc, nan);
      b[i >> 2] |= (c & 0xFFu) << (8 * (i & 3));
      sg |= (c >> 8) << i;
    }
    body[g] = make_uint2(b[0], b[1]);
    sign[g] = (uint8_t)sg;
  }
  if (nan && nonfinite) *nonfinite = 1;
}

__global__ __launch_bounds__(256) void k_quantize(const float4 *__restrict__ w, int64_t groups,
                                                  uint2 *__restrict__ body,
                                                  uint8_t *__restrict__ sign,
                                                  int32_t *__restrict__ nonfinite) {
  bool nan = false;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < groups; g += stride) {
    const float4 lo = w[2 * g], hi = w[2 * g + 1];
    const float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    uint32_t b[2] = {0u, 0u}, sg = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t c = fp9_code(__float_as_uint(v[i]), nan);
      b[i >> 2] |= (c & 0xFFu) << (8 * (i & 3));
      sg |= (c >> 8) << i;
    }
    body[g] = make_uint2(b[0], b[1]);
    sign[g] = (uint8_t)sg;
  }
  if (nan && nonfinite) *nonfinite = 1;  // every writer stores the same value
}

}  // namespace
}  // namespace duckmoe

extern "C" int duckmoe_quantize_fp9_device(const float *w, int64_t rows, int64_t cols,
                                           uint8_t *body, uint8_t *sign, int32_t *nonfinite,
                                           hipStream_t stream) {
  if (rows < 0 || cols < 0) return DUCKMOE_EINVAL;
  if (cols % 8) return DUCKMOE_ESHAPE;
  if (rows == 0 || cols == 0) return DUCKMOE_OK;  // nothing to write: pointers unused
  if (!w || !body || !sign) return DUCKMOE_EINVAL;
  if ((uintptr_t)w % 16 || (uintptr_t)body % 8) return DUCKMOE_EINVAL;
  if (rows > INT64_MAX / cols) return DUCKMOE_ESHAPE;
  const int64_t groups = rows * cols / 8;
  const int64_t want = (groups + 255) / 256;
  const unsigned blocks = (unsigned)(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(duckmoe::k_quantize, dim3(blocks), dim3(256), 0, stream,
                     reinterpret_cast<const float4 *>(w), groups,
                     reinterpret_cast<uint2 *>(body), sign, nonfinite);
  return hipGetLastError() == hipSuccess ? DUCKMOE_OK : DUCKMOE_EHIP;
}

extern "C" int duckmoe_fp8_to_fp9(const uint8_t *fp8, const float *scale, int64_t rows,
                                  int64_t cols, int32_t block, uint8_t *body, uint8_t *sign,
                                  int32_t *nonfinite, hipStream_t stream) {
  if (rows < 0 || cols < 0 || block < 8) return DUCKMOE_EINVAL;
  if (cols % 8 || block % 8) return DUCKMOE_ESHAPE;
  if (rows == 0 || cols == 0) return DUCKMOE_OK;
  if (!fp8 || !scale || !body || !sign) return DUCKMOE_EINVAL;
  if ((uintptr_t)fp8 % 8 || (uintptr_t)body % 8 || (uintptr_t)scale % 4) return DUCKMOE_EINVAL;
  if (rows > INT64_MAX / cols) return DUCKMOE_ESHAPE;
  const int64_t groups = rows * cols / 8;
  const int64_t nbc = (cols + block - 1) / block;
  const int64_t want = (groups + 255) / 256;
  const unsigned blocks = (unsigned)(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(duckmoe::k_fp8_to_fp9, dim3(blocks), dim3(256), 0, stream,
                     reinterpret_cast<const uint2 *>(fp8), scale, groups, cols, block, nbc,
                     reinterpret_cast<uint2 *>(body), sign, nonfinite);
  return hipGetLastError() == hipSuccess ? DUCKMOE_OK : DUCKMOE_EHIP;
}
