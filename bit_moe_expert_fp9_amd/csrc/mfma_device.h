// mfma_device.h - fp9 weight tiles for v_mfma_f32_16x16x32_f16 on gfx950.
//
// The fp9 weights decode exactly to fp16 (fp9_device.h), so a 16-row slab of a
// weight matrix is an fp16 A operand of the matrix cores.  Lane layout of
// v_mfma_f32_16x16x32_f16 (checked on gfx950): A[i][k] sits in lane
// i + 16 * (k / 8), element k % 8; B[k][j] in lane j + 16 * (k / 8), element
// k % 8; the accumulator element D[i][j] in lane j + 16 * (i / 4), element i % 4.
// The k index only has to agree between A and B.
//
// A unit is 128 columns of one 16-row tile.  It is loaded so that 4
// consecutive lanes read 64 contiguous bytes of one row (lane 4i + q: row i,
// columns 16q .. 16q + 15 and 64 + 16q .. 64 + 16q + 15), which the memory
// pipeline merges; ds_bpermute then moves lane 4i + g's words to lane i + 16g,
// the MFMA's place for row i and lane group g.  After the move lane group g
// holds columns 16g .. 16g + 15 (MFMA steps 0 and 1: 8 columns each) and
// 64 + 16g .. 64 + 16g + 15 (steps 2 and 3), so in step s the group's 8
// columns are 16g + 8 (s & 1) + 64 (s >> 1) .. + 7, and B must follow them.
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

struct MxTile {     // one unit of one 16-row tile for one lane
  uint4 b0, b1;     // 2 x 16 body bytes (see the layout note)
  uint16_t s0, s1;  // their sign bits (16 + 16)
};

// Load lane 4i + q's share: row `row` (= the tile's row i), columns
// c0 + 16q .. and c0 + 64 + 16q .. (16 each) of a [rows][K] matrix.  Rows with
// rv false and columns at or past K read as zero.
__device__ __forceinline__ void mx_load_w(MxTile &w, __amdgpu_buffer_rsrc_t rb,
                                          __amdgpu_buffer_rsrc_t rs, uint32_t row, uint32_t K,
                                          uint32_t c0, bool rv) {
  const uint32_t c = c0 + 16 * (threadIdx.x & 3);
  const bool v0 = rv && c < K, v1 = rv && c + 64 < K;
  w.b0 = buf_load16(rb, v0 ? row * K + c : kOutOfRange);
  w.b1 = buf_load16(rb, v1 ? row * K + c + 64 : kOutOfRange);
  w.s0 = buf_load2h(rs, v0 ? row * (K / 8) + c / 8 : kOutOfRange);
  w.s1 = buf_load2h(rs, v1 ? row * (K / 8) + c / 8 + 8 : kOutOfRange);
}

// Move lane 4i + g's tile words to lane i + 16g.  The empty volatile asm
// consumes the loaded sign words here: without it the compiler may hoist the
// arithmetic that merges them above an earlier barrier, which makes that
// barrier wait for loads meant to stay in flight across it.
__device__ __forceinline__ MxTile mx_to_mfma(const MxTile &w) {
  const int l = threadIdx.x & 63;
  const int src = 4 * ((4 * (l & 15) + (l >> 4)) & 63);  // byte address of lane 4(l % 16) + l / 16
  auto mv = [&](uint32_t v) { return (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)v); };
  uint16_t s0 = w.s0, s1 = w.s1;
  asm volatile("" : "+v"(s0), "+v"(s1));
  MxTile o;
  o.b0 = make_uint4(mv(w.b0.x), mv(w.b0.y), mv(w.b0.z), mv(w.b0.w));
  o.b1 = make_uint4(mv(w.b1.x), mv(w.b1.y), mv(w.b1.z), mv(w.b1.w));
  const uint32_t sg = mv((uint32_t)s0 | ((uint32_t)s1 << 16));
  o.s0 = (uint16_t)(sg & 0xFFFFu);
  o.s1 = (uint16_t)(sg >> 16);
  return o;
}

}  // namespace duckmoe
