// mfma_device.h - fp9 weight tiles for v_mfma_f32_16x16x32_f16 on gfx950.
//
// The fp9 weights decode exactly to fp16 (fp9_device.h), so a 16-row slab of a
// weight matrix is an fp16 A operand of the matrix cores.  Lane layout of
// v_mfma_f32_16x16x32_f16 (checked on gfx950): A[i][k] sits in lane
// i + 16 * (k / 8), element k % 8; B[k][j] in lane j + 16 * (k / 8), element
// k % 8; the accumulator element D[i][j] in lane j + 16 * (i / 4), element i % 4.
// The k index only has to agree between A and B.
//
// A unit is 128 columns of one 16-row tile.  Its body is loaded in whole
// 128-byte lines (mx_load_body_ln: lane 8r + q reads 16-byte chunk q of rows
// r and r + 8), the form the non-temporal cache policy needs, and
// ds_bpermute then gives lane i + 16g its row i's chunks g and 4 + g, the
// MFMA's place for row i and lane group g.  Lane group g then holds columns
// 16g .. 16g + 15 (MFMA steps 0 and 1: 8 columns each) and 64 + 16g ..
// 64 + 16g + 15 (steps 2 and 3), so in step s the group's 8 columns are
// 16g + 8 (s & 1) + 64 (s >> 1) .. + 7, and B must follow them.
//
// The unit's 16 sign bytes of row i are loaded as one dword per lane (lane
// 4i + q: bytes 4q .. 4q + 3), 16 bytes per row in one request, instead of two
// 2-byte loads per lane (8 bytes per row and request): the address unit
// handles each request of a wave's load separately, and the matrix-core
// kernels are bound by it.  Lane i + 16g then takes its two 16-bit words,
// bytes 2g, 2g + 1 and 8 + 2g, 9 + 2g, from lanes 4i + g / 2 and
// 4i + 2 + g / 2 with two ds_bpermute.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp9_device.h"

namespace duckmoe {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f4v_t __attribute__((ext_vector_type(4)));

constexpr int kMxUnit = 128;  // columns per unit: 4 lane groups x 32

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// power-of-two scale 2^k with max * 2^k in [2^13, 2^14) (k clamped to +-126)
__device__ __forceinline__ int mx_scale_exp(float m) {
  if (!(m > 0.0f)) return 0;
  int e;
  frexpf(m, &e);  // m = f * 2^e, f in [0.5, 1)
  return max(-126, min(126, 14 - e));
}

struct MxTile {     // one unit of one 16-row tile for one lane, as loaded
  uint4 b0, b1;     // 2 x 16 body bytes (see the layout note)
  uint32_t s;       // sign bytes 4q .. 4q + 3 of the unit's 16 in this row
};

struct MxFrag {     // the same unit moved to MFMA lane order
  uint4 b0, b1;     // columns 16g .. 16g + 15 and 64 + 16g .. 64 + 16g + 15 of row i
  uint16_t s0, s1;  // their sign bits (16 + 16)
};

// Lane 4i + q's sign word of a unit: bytes c0 / 8 + 4q .. + 3 of row `row`
// (= the tile's row i) of a [rows][K] matrix, the signs of columns
// c0 + 32q .. c0 + 32q + 31.  Rows with rv false and columns at or past K
// read as zero (a sign word that starts below K may end past it; its extra
// bits belong to columns whose body reads as zero, so they only choose the
// sign of a zero).  SA: the sign rows are whole dwords (K % 32 == 0), so the
// four bytes are one dword load; otherwise they are two 2-byte loads (dword
// loads must be dword-aligned; see mx_sign_mode for the choice).
template <bool SA>
__device__ __forceinline__ uint32_t mx_load_sign_word(__amdgpu_buffer_rsrc_t rs, uint32_t row,
                                                      uint32_t K, uint32_t c0, bool rv) {
  const uint32_t q = threadIdx.x & 3;
  const bool vs = rv && c0 + 32 * q < K;
  const uint32_t so = row * (K / 8) + c0 / 8 + 4 * q;
  if (SA) return buf_load4(rs, vs ? so : kOutOfRange);
  const bool vs1 = rv && c0 + 32 * q + 16 < K;
  return (uint32_t)buf_load2h(rs, vs ? so : kOutOfRange) |
         ((uint32_t)buf_load2h(rs, vs1 ? so + 2 : kOutOfRange) << 16);
}

// Whole-line body loads: lane 8r + q takes row r0 + r into b0 and row
// r0 + 8 + r into b1, 16 bytes each at column c0 + 16q, so each load
// instruction reads 8 rows x 128 contiguous bytes of the unit: whole 128-byte
// lines.  The non-temporal policy needs that: with a line's two halves read by
// two instructions it reads slower than without it.
// moff is added to every row index (the up half of a gate/up matrix); rows
// r0 + r at or past `rows`, and all rows when live is false, read as zero.
// W is MxTile or MxBody (only b0 and b1 are written).
template <int CP, class W>
__device__ __forceinline__ void mx_load_body_ln(W &w, __amdgpu_buffer_rsrc_t rb, uint32_t moff,
                                                int r0, int rows, uint32_t K, uint32_t c0,
                                                bool live) {
  const int l = threadIdx.x & 63;
  const int ra = r0 + (l >> 3), rc = ra + 8;
  const uint32_t c = c0 + 16 * (l & 7);
  const bool cv = live && c < K;
  w.b0 = buf_load16<CP>(rb, cv && ra < rows ? (moff + (uint32_t)ra) * K + c : kOutOfRange);
  w.b1 = buf_load16<CP>(rb, cv && rc < rows ? (moff + (uint32_t)rc) * K + c : kOutOfRange);
}

// Body words (mx_load_body_ln) to MFMA lane order.  Lane i + 16g needs row i's
// 16-byte chunks g (b0) and 4 + g (b1), held by lanes 8 (i % 8) + g and
// 8 (i % 8) + 4 + g in their b0 (i < 8) or b1 (i >= 8).  Two moves per dword
// carry them: in the first each lane sends b0 if its chunk is below 4, else
// b1, and lane i + 16g reads lane 8 (i % 8) + g + 4 (i / 8); in the second the
// other word, read from lane 8 (i % 8) + g + 4 (1 - i / 8).  Rows 0-7 receive
// chunk g first, rows 8-15 chunk 4 + g.
__device__ __forceinline__ void mx_move_body(const uint4 &b0, const uint4 &b1, MxFrag &o) {
  const int l = threadIdx.x & 63;
  const int i = l & 15, g = l >> 4;
  const bool up = (l & 4) != 0, hi = i >= 8;
  const int sA = 4 * (8 * (i & 7) + g + (hi ? 4 : 0));
  const int sB = 4 * (8 * (i & 7) + g + (hi ? 0 : 4));
  auto two = [&](uint32_t v0, uint32_t v1, uint32_t &d0, uint32_t &d1) {
    const uint32_t a = (uint32_t)__builtin_amdgcn_ds_bpermute(sA, (int)(up ? v1 : v0));
    const uint32_t b = (uint32_t)__builtin_amdgcn_ds_bpermute(sB, (int)(up ? v0 : v1));
    d0 = hi ? b : a;
    d1 = hi ? a : b;
  };
  two(b0.x, b1.x, o.b0.x, o.b1.x);
  two(b0.y, b1.y, o.b0.y, o.b1.y);
  two(b0.z, b1.z, o.b0.z, o.b1.z);
  two(b0.w, b1.w, o.b0.w, o.b1.w);
}

// Move the body words to MFMA lane order and gather lane i + 16g's sign words
// (see the layout note).  The empty volatile asm consumes the loaded sign word
// here: without it the compiler may move work on it above an earlier barrier,
// which makes that barrier wait for loads meant to stay in flight across it.
__device__ __forceinline__ MxFrag mx_to_mfma(const MxTile &w) {
  const int l = threadIdx.x & 63;
  const int i = l & 15, g = l >> 4;
  uint32_t s = w.s;
  asm volatile("" : "+v"(s));
  MxFrag o;
  mx_move_body(w.b0, w.b1, o);
  // bytes 2g, 2g + 1 sit in dword g / 2 of the row, bytes 8 + 2g, 9 + 2g in
  // dword 2 + g / 2; half g % 2 of each
  const uint32_t x = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * (4 * i + (g >> 1)), (int)s);
  const uint32_t y = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * (4 * i + 2 + (g >> 1)), (int)s);
  const uint32_t sg = __builtin_amdgcn_perm(y, x, (g & 1) ? 0x07060302u : 0x05040100u);
  o.s0 = (uint16_t)(sg & 0xFFFFu);
  o.s1 = (uint16_t)(sg >> 16);
  return o;
}

// ---------------------------------------------------------------------------
// Unit pairs (the decode kernels).  A wave that takes units 2p and 2p + 1 of
// the same rows one after the other loads the sign bytes of both with one
// request per row where the rows allow it: the address unit's cost is per
// load instruction, so a second dword in the same instruction is nearly free.
// Sign modes, by the column count K of the matrix:
//   2: K % 64 == 0: one 8-byte load per lane, lane 4i + q taking bytes
//      8q .. 8q + 7 of the pair's 32 (units 2p: q = 0, 1; 2p + 1: q = 2, 3);
//      8-byte aligned, and a lane's 64 columns lie all below K or all past it;
//   1: K % 32 == 0: one dword per lane and unit (mx_load_sign_word);
//   0: two 2-byte loads per lane and unit.
// The mode also needs the sign plane's base aligned to the load width (the
// expert and row offsets then are: K % 16 == 0 for every matrix).
__host__ inline int mx_sign_mode(int K, const void *sign) {
  const uintptr_t p = reinterpret_cast<uintptr_t>(sign);
  return (K % 64 == 0 && p % 8 == 0) ? 2 : ((K % 32 == 0 && p % 4 == 0) ? 1 : 0);
}

struct MxBody {     // one unit of one 16-row tile for one lane, as loaded
  uint4 b0, b1;
};

struct MxSigns {    // the lane's sign words of a unit pair (layout by sign mode)
  uint32_t a, b;
};

// The sign words of row `row` for the units starting at columns c0 and
// c0 + 128; columns at or past K (and rows with rv false) read as zero.
template <int SM>
__device__ __forceinline__ void mx_load_signs(MxSigns &s, __amdgpu_buffer_rsrc_t rs, uint32_t row,
                                              uint32_t K, uint32_t c0, bool rv) {
  const uint32_t q = threadIdx.x & 3;
  const uint32_t so = row * (K / 8) + c0 / 8;
  if (SM == 2) {
    const uint2 v = buf_load8(rs, rv && c0 + 64 * q < K ? so + 8 * q : kOutOfRange);
    s.a = v.x;
    s.b = v.y;
  } else if (SM == 1) {
    s.a = buf_load4(rs, rv && c0 + 32 * q < K ? so + 4 * q : kOutOfRange);
    s.b = buf_load4(rs, rv && c0 + 128 + 32 * q < K ? so + 16 + 4 * q : kOutOfRange);
  } else {
    auto half = [&](uint32_t col, uint32_t off) {
      return (uint32_t)buf_load2h(rs, rv && col < K ? off : kOutOfRange);
    };
    s.a = half(c0 + 32 * q, so + 4 * q) | (half(c0 + 32 * q + 16, so + 4 * q + 2) << 16);
    s.b = half(c0 + 128 + 32 * q, so + 16 + 4 * q) |
          (half(c0 + 128 + 32 * q + 16, so + 18 + 4 * q) << 16);
  }
}

// mx_to_mfma for unit HALF (0: 2p, 1: 2p + 1) of a pair.  Lane i + 16g needs
// dwords g / 2 and 2 + g / 2 of its unit's 16 sign bytes of row i.  In sign
// mode 2 those sit in the .a (g < 2) or .b (g >= 2) word of lane 4i + 2 HALF
// (dwords 0, 1) and 4i + 2 HALF + 1 (dwords 2, 3); one quad-local DPP move
// per word first gathers, in v1, dword 0 / 1 of each unit on its even / odd
// lane and, in v2, dword 2 / 3, so that each needed dword is one ds_bpermute
// away.  In the other modes the unit's word is laid out as in mx_load_sign_word.
template <int SM, int HALF>
__device__ __forceinline__ MxFrag mx_to_mfma_pair(const MxBody &w, const MxSigns &sp) {
  const int l = threadIdx.x & 63;
  const int i = l & 15, g = l >> 4;
  uint32_t sa = sp.a, sb = sp.b;
  asm volatile("" : "+v"(sa), "+v"(sb));
  MxFrag o;
  mx_move_body(w.b0, w.b1, o);
  uint32_t x, y;
  if (SM == 2) {
    const bool odd = (l & 1) != 0;
    // quad_perm [0, 0, 2, 2] of .b and [1, 1, 3, 3] of .a
    const uint32_t bl = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)sb, 0xA0, 0xF, 0xF, false);
    const uint32_t ar = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)sa, 0xF5, 0xF, 0xF, false);
    const uint32_t v1 = odd ? bl : sa;
    const uint32_t v2 = odd ? sb : ar;
    const int from = 4 * (4 * i + 2 * HALF + (g >> 1));
    x = (uint32_t)__builtin_amdgcn_ds_bpermute(from, (int)v1);
    y = (uint32_t)__builtin_amdgcn_ds_bpermute(from, (int)v2);
  } else {
    const uint32_t s = HALF ? sb : sa;
    x = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * (4 * i + (g >> 1)), (int)s);
    y = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * (4 * i + 2 + (g >> 1)), (int)s);
  }
  const uint32_t sg = __builtin_amdgcn_perm(y, x, (g & 1) ? 0x07060302u : 0x05040100u);
  o.s0 = (uint16_t)(sg & 0xFFFFu);
  o.s1 = (uint16_t)(sg >> 16);
  return o;
}

}  // namespace duckmoe
