// fp9_device.h - inline fp9 decode and wavefront reductions for gfx950.
//
// The fp9 format (duck-llm memoir page "一鸭三吃：我把评测鸭变成了满血
// DeepSeek-V3.2 推理系统", section "在只有 AVX2 的 N100 上，我先做出了单核 MLP
// fp9"): a 9-bit code s|eeeee|mmm with exponent bias 15, stored as a body byte
// eeeeemmm plus one sign bit per weight in a separate bitplane (8 signs per
// byte).  Because the bias equals fp16's, (sign << 8 | body) << 7 is exactly
// the fp16 encoding of the value, subnormals and signed zero included; the
// hardware converts it from there.
//
// On CDNA the fp16 patterns of two weights are built in one 32-bit register:
//   v_perm_b32 picks, for each 16-bit half, the weight's body byte as the low
//   byte and, as the high byte, some byte whose bit 0 is that weight's sign;
//   v_pk_lshlrev_b16 by 7 then shifts both halves at once.  The garbage in bits
//   1..7 of the high byte leaves the 16-bit lane, only its bit 0 lands on the
//   fp16 sign bit.
// The packed halves are consumed by v_fma_mix_f32, which converts an fp16 half
// to f32 inside the fused multiply-add, so each weight costs one perm/shift
// half-pair (1 VALU op per weight) plus one FMA per token.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace duckmoe {

typedef unsigned short us2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

// Two fp16 weights from a body word and a sign-source word (see above).
// perm(src0=sgn, src1=body): selector bytes 0..3 address body, 4..7 address sgn.
__device__ __forceinline__ h2_t fp9_pair(uint32_t sgn, uint32_t body, uint32_t sel) {
  const uint32_t p = __builtin_amdgcn_perm(sgn, body, sel);
  const us2_t v = __builtin_bit_cast(us2_t, p) << (us2_t)(7);
  return __builtin_bit_cast(h2_t, v);
}

// Sign sources.  For up to 16 sign bits s (bit k = sign of weight k) let
//   r  = (s >> 1) << 16 | s,   y_j = r >> 2j   (j = 0..3).
// Then bit 0 of the bytes of y_j is:
//   byte 0 -> s_{2j}, byte 2 -> s_{2j+1}, byte 1 -> s_{8+2j}, byte 3 -> s_{9+2j}.
// The selectors below place [sign byte | body byte] in each 16-bit half:
//   kSelLo01: (w0, w1) of a body word with signs from bytes 0 / 2
//   kSelLo23: (w2, w3)                      "            bytes 0 / 2
//   kSelHi01: (w0, w1) with signs from bytes 1 / 3   (weights 8..15)
//   kSelHi23: (w2, w3)                 "
constexpr uint32_t kSelLo01 = 0x06010400u;
constexpr uint32_t kSelLo23 = 0x06030402u;
constexpr uint32_t kSelHi01 = 0x07010500u;
constexpr uint32_t kSelHi23 = 0x07030502u;

// 16 consecutive weights: body bytes in d (weight k in byte k%4 of word k/4),
// sign bits in s16 (bit k).  h[p] holds weights (2p, 2p+1) as (lo, hi).
__device__ __forceinline__ void fp9_decode16(const uint4 d, const uint32_t s16, h2_t h[8]) {
  const uint32_t r = ((s16 >> 1) << 16) | s16;
  const uint32_t y0 = r, y1 = r >> 2, y2 = r >> 4, y3 = r >> 6;
  h[0] = fp9_pair(y0, d.x, kSelLo01);
  h[1] = fp9_pair(y1, d.x, kSelLo23);
  h[2] = fp9_pair(y2, d.y, kSelLo01);
  h[3] = fp9_pair(y3, d.y, kSelLo23);
  h[4] = fp9_pair(y0, d.z, kSelHi01);
  h[5] = fp9_pair(y1, d.z, kSelHi23);
  h[6] = fp9_pair(y2, d.w, kSelHi01);
  h[7] = fp9_pair(y3, d.w, kSelHi23);
}

// 8 consecutive weights: body words d0 (weights 0..3) and d1 (4..7), sign byte s8.
__device__ __forceinline__ void fp9_decode8(const uint32_t d0, const uint32_t d1,
                                            const uint32_t s8, h2_t h[4]) {
  const uint32_t r = ((s8 >> 1) << 16) | s8;
  h[0] = fp9_pair(r, d0, kSelLo01);
  h[1] = fp9_pair(r >> 2, d0, kSelLo23);
  h[2] = fp9_pair(r >> 4, d1, kSelLo01);
  h[3] = fp9_pair(r >> 6, d1, kSelLo23);
}

// acc += w * x for the 16 decoded weights of one row and a 16-float x slice.
// The compiler turns (float)half * x + acc into v_fma_mix_f32.  Even and odd
// weights go to two accumulators: two dependent v_fma_mix_f32 back to back
// cost a wait state on gfx950, alternating chains do not.
__device__ __forceinline__ void fma16(const h2_t h[8], const float x[16], float &a0, float &a1) {
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    a0 = __builtin_fmaf((float)h[p].x, x[2 * p], a0);
    a1 = __builtin_fmaf((float)h[p].y, x[2 * p + 1], a1);
  }
}

// ---------------------------------------------------------------------------
// Buffer resources.  Weights are read with raw buffer loads: one descriptor
// (base address, byte size) per expert matrix in SGPRs and a 32-bit per-lane
// offset in a VGPR.  An offset at or beyond the size reads as zero, which is
// how rows and lanes past the end of a matrix are masked.
constexpr uint32_t kBufCfg = 0x00020000u;  // dword 3 of a gfx9 raw buffer descriptor
constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           (int)kBufCfg);
}

// Cache policy of a buffer load (the instruction's aux bits).  kStream sets
// the non-temporal bit: plain streaming reads of a fresh 446 MB window with it
// run at 6.8 TB/s on an MI355X against 6.06 TB/s without it (one launch, 32
// waves per CU, 8 dwordx4 loads in flight per lane), and the bsz 1-2 decode
// kernels, whose every weight load instruction covers whole 128-byte lines,
// take it for their weight planes.  The matrix-core kernels read a line's
// halves (and a row's sign bytes) with separate instructions; there the bit
// made them 15-20% slower, so they keep the default policy, as do the
// activations and plans, which are read again.
constexpr int kCached = 0;
constexpr int kStream = 2;

// The 128-bit results are reinterpreted as a whole vector: extracting and
// bit-casting single elements (bit_cast<float>(v[i])) miscompiles with this
// toolchain (one dword gets loaded and the offset register is read as data).
template <int CP = kCached>
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, CP));
}

template <int CP = kCached>
__device__ __forceinline__ uint32_t buf_load2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, CP);
}

// The 16-bit result kept as 16 bits: widening it where it is used (not right
// after the load) keeps the compiler from waiting for the load early.
template <int CP = kCached>
__device__ __forceinline__ uint16_t buf_load2h(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, CP);
}

template <int CP = kCached>
__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, CP);
}

template <int CP = kCached>
__device__ __forceinline__ uint2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, CP));
}

__device__ __forceinline__ float4 buf_loadf4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// ---------------------------------------------------------------------------
// Wavefront (64-lane) sums with DPP.  After the steps up to group size G the
// last lane of every aligned group of G lanes holds that group's sum (for
// G <= 16 every lane of the group does).
template <int CTRL, int ROW_MASK = 0xF, int BANK_MASK = 0xF>
__device__ __forceinline__ float dpp_src(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK,
                                         BANK_MASK, false));
}

template <int G>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(G == 4 || G == 8 || G == 16 || G == 32 || G == 64, "group size");
  v += dpp_src<0xB1>(v);              // quad_perm [1,0,3,2]: lane ^ 1
  v += dpp_src<0x4E>(v);              // quad_perm [2,3,0,1]: lane ^ 2
  if (G >= 8) v += dpp_src<0x141>(v);  // row_half_mirror: other quad of the 8
  if (G >= 16) v += dpp_src<0x140>(v); // row_mirror: other half of the row of 16
  if (G >= 32) v += dpp_src<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  if (G >= 64) v += dpp_src<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

// Full 64-lane maximum of non-negative values, returned in every lane.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_src<0xB1>(v));
  v = fmaxf(v, dpp_src<0x4E>(v));
  v = fmaxf(v, dpp_src<0x141>(v));
  v = fmaxf(v, dpp_src<0x140>(v));
  v = fmaxf(v, dpp_src<0x142, 0xA>(v));
  v = fmaxf(v, dpp_src<0x143, 0xC>(v));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Full 64-lane sum, returned in every lane.
__device__ __forceinline__ float wave_sum(float v) {
  v = group_sum<64>(v);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

}  // namespace duckmoe
