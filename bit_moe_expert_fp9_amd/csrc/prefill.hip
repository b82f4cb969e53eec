// prefill.hip - the larger-T (prefill) routed layer: per-expert token lists and
// a grouped GEMM on the matrix cores.
//
// What is computed is the routed layer of duckmoe.hip, for many tokens at once:
// out_t = shared(x_t) + sum_i w_ti expert_{ids_ti}(x_t) with the SwiGLU experts
// in fp9 (duck-llm memoir page "一鸭三吃：我把评测鸭变成了满血 DeepSeek-V3.2 推理
// 系统", fp9 section "在只有 AVX2 的 N100 上，我先做出了单核 MLP fp9"; chapter
// page "第 9 章 MTP1 dual-lane overlap", section 9.2 "两条路线的判断" for top-8
// routing plus the shared expert).  The pages name the fp9 prefill kernel as
// the part still far from peak (memoir page, section "限制条件", which also
// tests contexts up to 2048 tokens); this file is that path on gfx950.
//
// Decode streams every selected expert once per step; at prefill sizes an
// expert serves many tokens, so its weights should be read once for all of
// them.  The tokens are grouped by expert:
//   k_pf_count / k_pf_scan / k_pf_fill: list p = 0 is the shared expert (every
//     token, weight 1), list p >= 1 routed expert p - 1 with the tokens that
//     name it in ascending order (a repeated id adds its weights; an id out of
//     range is skipped; both are flagged in the status word).  Entries are
//     numbered list by list; tok_entry[t] names token t's entries (shared
//     first, then by id position, -1 for a repeat or a bad id).  Lists are cut
//     into tiles of 64 entries, or 96 (pf_tile).  Only per-list scans, a block
//     scan and a ballot: no atomics, the same lists every call.
//   k_pf_xprep: x rows -> fp16 hi/lo pairs (below).
//   k_pf_gemm (gate/up): a workgroup of 8 waves takes tasks (tile, block of
//     8 * 16 * RT intermediate rows): each wave owns 16 * RT gate rows and the
//     matching up rows, the tile's activations of each 128-column unit are
//     staged once in LDS for all 8 waves, and the epilogue writes
//     h' = w * silu(gate) * up as scaled fp16 hi/lo pairs per (entry, 128-row
//     unit).
//   k_pf_gemm (down): the same grouped GEMM over (tile, block of output rows)
//     with the down weights, writing y[entry][H] in f32.
//   k_pf_combine: out_t = the entries of tok_entry[t] added in slot order.
// Every output element is a fixed-order sum: bit-identical run to run.
//
// Precision.  fp9 -> fp16 is exact (A operand).  An f32 activation v (B) is
// carried as hi = fp16(v s) and lo = fp16(v s - hi), s a power of two per
// token row (x) or per (entry, 128-row unit) (h') that puts the row's largest
// magnitude in [2^13, 2^14): both parts stay finite, v s - hi is exact in f32
// and lo keeps 11 more bits.  A * hi and A * lo go into the same f32
// accumulator (fp16 x fp16 products are exact in f32), and the scale is
// undone in f32.  The error is that of a ~22-bit activation plus f32
// accumulation.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "../../include/duckmoe.h"
#include "fp9_device.h"
#include "host_util.h"
#include "mfma_device.h"

namespace duckmoe {
namespace {

// Tiles hold 64 entries (tokens), or 96 when the routed lists average 49 to 72
// entries (see pf_tile); the workspace is sized for 64.
constexpr int kPfTileMin = 64;
constexpr int kPfTileMax = 96;
constexpr int kPfWaves = 8;                     // waves per GEMM workgroup
template <int TILE>
constexpr int pf_cols() { return TILE / 16; }   // MFMA column tiles per tile
template <int TILE>
constexpr int pf_q() { return TILE / 32; }      // token rows a thread stages per unit
// Launch shapes per tile size: 16-row tiles per wave (RT) and resident
// workgroups per CU the registers must allow.  At 96 entries the double-buffered
// activation tile (105 KB of LDS) leaves room for one workgroup per CU, and
// gate/up takes 32 rows per wave.
#ifndef DUCKMOE_PF_GU_RT
#define DUCKMOE_PF_GU_RT 1          // gate/up, 64-entry tiles
#endif
#ifndef DUCKMOE_PF_GU_WG_PER_CU
#define DUCKMOE_PF_GU_WG_PER_CU 2
#endif
#ifndef DUCKMOE_PF_GU_RT96
#define DUCKMOE_PF_GU_RT96 2        // gate/up, 96-entry tiles (one workgroup per CU)
#endif
#ifndef DUCKMOE_PF_DN_RT
#define DUCKMOE_PF_DN_RT 2          // down, both tile sizes (one workgroup per CU)
#endif
#ifndef DUCKMOE_PF_DN_WG_PER_CU
#define DUCKMOE_PF_DN_WG_PER_CU 1
#endif
#ifndef DUCKMOE_PF_WCP
#define DUCKMOE_PF_WCP 2
#endif
constexpr int kPfWeightPolicy = DUCKMOE_PF_WCP;  // cache policy of the weight loads
constexpr int kPfPitch = 2 * kMxUnit + 16;      // LDS bytes per token row of a unit (padded)
constexpr int kPfMaxTopK = 32;
constexpr int kPfMaxRouted = 1024;
constexpr int kPfMaxTokens = 32768;
// rows of one GEMM task, and (gate/up) waves per 128-row unit of h'
template <int RT>
constexpr int pf_rows() { return kPfWaves * RT * 16; }
template <int RT>
constexpr int pf_wpu() { return kMxUnit / (RT * 16); }
static_assert(kPfWaves * 64 == 512 && kMxUnit == 128,
              "staging: 16 threads per token row of 256 bytes, 32 rows per pass");

struct PfArgs {
  int H, I, E, K, T, Hp, Ip, A;  // A = entry capacity, T * (K + 1)
  int tile;              // entries per tile (kPfTileMin or kPfTileMax)
  const uint8_t *gu_body, *gu_sign, *dn_body, *dn_sign;
  const float *x;        // [T][H]
  const int32_t *ids;    // [T][K] (K = 0: no routed ids)
  const float *w;        // [T][K]
  float *out;            // [T][H]
  int32_t *status;       // status word
  int32_t *n_tiles;      // tile count (null: no tile table)
  int32_t *off;          // [E + 2] first entry of each list
  int4 *tiles;           // {list, first entry, entries, 0}
  int32_t *tok;          // [A] token of each entry
  float *wt;             // [A] routing weight of each entry
  int32_t *tok_entry;    // [T][K + 1]
  _Float16 *xh, *xl;     // [T][Hp] scaled x, hi and lo (zero padded)
  float *xinv;           // [T] 1 / scale
  _Float16 *hh, *hl;     // [A][Ip] scaled h'
  float *hs;             // [A][Ip / 128] 1 / scale per 128-row unit
  float *y;              // [A][H] down outputs per entry
};

__device__ __forceinline__ int block_sum256(int v, int *red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const int s = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return s;
}

// ------------------------------------------------------------------ plan ----
// The K ids of token t, loaded together (every load issued before any is
// used; -1 past K).  KM >= K bounds the unrolled loops, so that the ids stay
// in registers: 8, 16 or kPfMaxTopK (chosen by launch_plan).
template <int KM>
__device__ __forceinline__ void pf_row_ids(const PfArgs &a, int t, int (&v)[KM]) {
  const int32_t *row = a.ids + (size_t)t * a.K;
#pragma unroll
  for (int i = 0; i < KM; ++i) v[i] = i < a.K ? row[i] : -1;
}

// One workgroup per list.  List 0 (shared) counts every token and checks every
// token's ids (status word; -1 in tok_entry for repeats and bad ids); list
// p >= 1 counts the tokens naming expert p - 1.  Counts go to off[p + 1].
template <int KM>
__global__ __launch_bounds__(256) void k_pf_count(const PfArgs a) {
  __shared__ int red[4];
  const int p = blockIdx.x, K = a.K, T = a.T;
  if (p == 0) {
    int st = 0;
    for (int t = threadIdx.x; t < T; t += 256) {
      int v[KM];
      pf_row_ids(a, t, v);
#pragma unroll
      for (int i = 0; i < KM; ++i) {
        if (i < K) {
          const int id = v[i];
          bool keep = id >= 0 && id < a.E;
          if (!keep) {
            st |= DUCKMOE_STATUS_BAD_ID;
          } else {
            bool dup = false;
#pragma unroll
            for (int q = 0; q < i; ++q) dup |= v[q] == id;
            if (dup) {
              keep = false;
              st |= DUCKMOE_STATUS_DUP_ID;
            }
          }
          if (!keep) a.tok_entry[(size_t)t * (K + 1) + 1 + i] = -1;
        }
      }
    }
    const int bad = block_sum256((st & DUCKMOE_STATUS_BAD_ID) ? 1 : 0, red);
    const int dup = block_sum256((st & DUCKMOE_STATUS_DUP_ID) ? 1 : 0, red);
    if (threadIdx.x == 0) {
      a.status[0] = (bad ? DUCKMOE_STATUS_BAD_ID : 0) | (dup ? DUCKMOE_STATUS_DUP_ID : 0);
      a.off[1] = T;
    }
    return;
  }
  const int e = p - 1;
  int c = 0;
  for (int t = threadIdx.x; t < T; t += 256) {
    int v[KM];
    pf_row_ids(a, t, v);
    bool hit = false;
#pragma unroll
    for (int i = 0; i < KM; ++i) hit |= v[i] == e;
    c += hit ? 1 : 0;
  }
  c = block_sum256(c, red);
  if (threadIdx.x == 0) a.off[p + 1] = c;
}

// One workgroup of 1024: counts -> first entries (exclusive scan over lists),
// the tile table (lists cut into tiles of a.tile entries) and its size.
__global__ __launch_bounds__(1024) void k_pf_scan(const PfArgs a) {
  __shared__ int cnt[kPfMaxRouted + 1];
  __shared__ int se[1024], st[1024];
  const int n = a.E + 1, tid = threadIdx.x, tile = a.tile;
  for (int p = tid; p < n; p += 1024) cnt[p] = a.off[p + 1];
  __syncthreads();
  const int per = (n + 1023) / 1024, p0 = min(n, tid * per), p1 = min(n, p0 + per);
  int ce = 0, ct = 0;
  for (int p = p0; p < p1; ++p) {
    ce += cnt[p];
    ct += (cnt[p] + tile - 1) / tile;
  }
  se[tid] = ce;
  st[tid] = ct;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {  // inclusive Hillis-Steele scan
    const int ve = tid >= d ? se[tid - d] : 0, vt = tid >= d ? st[tid - d] : 0;
    __syncthreads();
    se[tid] += ve;
    st[tid] += vt;
    __syncthreads();
  }
  int eb = se[tid] - ce, tb = st[tid] - ct;
  for (int p = p0; p < p1; ++p) {
    a.off[p] = eb;
    if (a.tiles) {
      for (int k = 0; k * tile < cnt[p]; ++k)
        a.tiles[tb + k] = make_int4(p, eb + k * tile, min(tile, cnt[p] - k * tile), 0);
    }
    tb += (cnt[p] + tile - 1) / tile;
    eb += cnt[p];
  }
  if (tid == 1023) {
    a.off[n] = se[1023];
    if (a.n_tiles) *a.n_tiles = st[1023];
  }
}

// One workgroup per list: the list's tokens in ascending order, 256 at a time;
// a token's rank is the hits before it (ballot within the wave, wave counts
// across the workgroup).
template <int KM>
__global__ __launch_bounds__(256) void k_pf_fill(const PfArgs a) {
  __shared__ int wc[4];
  const int p = blockIdx.x, K = a.K, T = a.T;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int base = a.off[p];
  if (p == 0) {
    for (int t = threadIdx.x; t < T; t += 256) {
      a.tok[base + t] = t;
      a.wt[base + t] = 1.0f;
      a.tok_entry[(size_t)t * (K + 1)] = base + t;
    }
    return;
  }
  const int e = p - 1;
  int run = 0;
  for (int t0 = 0; t0 < T; t0 += 256) {
    const int t = t0 + threadIdx.x;
    bool hit = false;
    int first = 0;
    float s = 0.0f;
    if (t < T) {
      int v[KM];
      pf_row_ids(a, t, v);
      const float *wr = a.w + (size_t)t * K;
#pragma unroll
      for (int i = 0; i < KM; ++i) {
        if (v[i] == e) {
          if (!hit) first = i;
          hit = true;
          s += wr[i];
        }
      }
    }
    const uint64_t m = __ballot(hit);
    const int rank = __popcll(m & ((1ull << lane) - 1ull));
    if (lane == 0) wc[wave] = __popcll(m);
    __syncthreads();
    int before = run;
    for (int q = 0; q < wave; ++q) before += wc[q];
    if (hit) {
      const int ent = base + before + rank;
      a.tok[ent] = t;
      a.wt[ent] = s;
      a.tok_entry[(size_t)t * (K + 1) + 1 + first] = ent;
    }
    run += wc[0] + wc[1] + wc[2] + wc[3];
    __syncthreads();
  }
}

// --------------------------------------------------------------- x prep ----
// One workgroup per token: x row -> scaled hi/lo fp16 rows of width Hp.
__global__ __launch_bounds__(256) void k_pf_xprep(const PfArgs a) {
  __shared__ float red[4];
  const int t = blockIdx.x;
  const float4 *s4 = reinterpret_cast<const float4 *>(a.x + (size_t)t * a.H);
  const int n4 = a.H / 4, np4 = a.Hp / 4;
  float m = 0.0f;
  for (int i = threadIdx.x; i < n4; i += 256) {
    const float4 v = s4[i];
    m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  }
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  const int k = mx_scale_exp(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])));
  const float sc = ldexpf(1.0f, k);
  typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
  for (int i = threadIdx.x; i < np4; i += 256) {
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i < n4) v = s4[i];
    const float e[4] = {v.x * sc, v.y * sc, v.z * sc, v.w * sc};
    h4_t hi, lo;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      hi[q] = (_Float16)e[q];
      lo[q] = (_Float16)(e[q] - (float)hi[q]);
    }
    const size_t o = (size_t)t * a.Hp + 4 * i;
    *reinterpret_cast<h4_t *>(a.xh + o) = hi;
    *reinterpret_cast<h4_t *>(a.xl + o) = lo;
  }
  if (threadIdx.x == 0) a.xinv[t] = ldexpf(1.0f, -k);
}

// ------------------------------------------------------- grouped GEMMs ----
// Workgroups are dispatched to the 8 XCDs round robin; virtual ids that are
// consecutive within a round stay on one XCD, so the tasks of one tile (which
// read the same activations) share that XCD's L2.
__device__ __forceinline__ int pf_vid() {
  const int G = gridDim.x, b = blockIdx.x;
  if (G % 8) return b;
  return (b % 8) * (G / 8) + b / 8;
}

// B staging: a unit's tile is [2 parts][TILE tokens][256 bytes]; thread tid
// moves the 16-byte pieces (part h, token tid / 16 + 32 q, bytes 16 (tid % 16) ..)
// for h in {0, 1}, q < Q = TILE / 32: global -> registers, then registers -> LDS.
template <int Q>
struct PfStage {
  uint4 v[2][Q];
};

template <int Q>
__device__ __forceinline__ void pf_stage_load(PfStage<Q> &s, __amdgpu_buffer_rsrc_t rh,
                                              __amdgpu_buffer_rsrc_t rl, const uint32_t src[Q],
                                              uint32_t ubytes) {
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const uint32_t o = src[q] == kOutOfRange ? kOutOfRange : src[q] + ubytes;
    s.v[0][q] = buf_load16(rh, o);
    s.v[1][q] = buf_load16(rl, o);
  }
}

template <int TILE>
__device__ __forceinline__ void pf_stage_store(const PfStage<pf_q<TILE>()> &s, uint8_t *buf) {
  const int tok = threadIdx.x >> 4, seg = threadIdx.x & 15;
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int q = 0; q < pf_q<TILE>(); ++q)
      *reinterpret_cast<uint4 *>(buf + h * (TILE * kPfPitch) + (tok + 32 * q) * kPfPitch +
                                 seg * 16) = s.v[h][q];
}

// MFMA B operand of lane (token j, group g) for column tile ct and step s.
template <int TILE>
__device__ __forceinline__ half8_t pf_b(const uint8_t *buf, int part, int ct, int s) {
  const int lane = threadIdx.x & 63, j = lane & 15, g = lane >> 4;
  const int seg = 2 * g + (s & 1) + 8 * (s >> 1);
  return *reinterpret_cast<const half8_t *>(buf + part * (TILE * kPfPitch) +
                                            (16 * ct + j) * kPfPitch + seg * 16);
}

__device__ __forceinline__ half8_t pf_a(const h2_t d[8], int ss) {
  return __builtin_bit_cast(half8_t, make_uint4(__builtin_bit_cast(uint32_t, d[4 * ss]),
                                                __builtin_bit_cast(uint32_t, d[4 * ss + 1]),
                                                __builtin_bit_cast(uint32_t, d[4 * ss + 2]),
                                                __builtin_bit_cast(uint32_t, d[4 * ss + 3])));
}

// acc[r][m][ct] += A(r, m) * B(ct) over one 128-column unit.  M matrices of
// RT row tiles each; wm holds the unit's weight tiles in MFMA order; only the
// first nct column tiles are live.
template <int RT, int M, int TILE>
__device__ __forceinline__ void pf_unit(const MxFrag (&wm)[RT][M], const uint8_t *buf, int nct,
                                        f4v_t (&acc)[RT][M][pf_cols<TILE>()]) {
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    h2_t d[RT][M][8];
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int m = 0; m < M; ++m)
        fp9_decode16(hf ? wm[r][m].b1 : wm[r][m].b0, hf ? wm[r][m].s1 : wm[r][m].s0, d[r][m]);
#pragma unroll
    for (int ss = 0; ss < 2; ++ss) {
      const int s = 2 * hf + ss;
#pragma unroll
      for (int ct = 0; ct < pf_cols<TILE>(); ++ct) {
        if (ct < nct) {
          const half8_t bh = pf_b<TILE>(buf, 0, ct, s), bl = pf_b<TILE>(buf, 1, ct, s);
#pragma unroll
          for (int r = 0; r < RT; ++r)
#pragma unroll
            for (int m = 0; m < M; ++m) {
              const half8_t A = pf_a(d[r][m], ss);
              acc[r][m][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, bh, acc[r][m][ct], 0, 0, 0);
              acc[r][m][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, bl, acc[r][m][ct], 0, 0, 0);
            }
        }
      }
    }
  }
}

// One task of a grouped GEMM: a tile (list, first entry, entries) times a
// block of kPfRows output rows.  task >= ntask is "no task": no entries, every
// load out of range.  Scalar fields are wave-uniform.
template <int Q>
struct PfTask {
  int task, blk;
  int e0, n, nct;
  const uint8_t *body, *sign;  // the expert's planes of this matrix
  uint32_t src[Q];             // staging sources of this thread, unit 0 (bytes)
  uint32_t hsrc;               // down: this thread's h' scale source, unit 0 (bytes)
};

template <bool GU, int TILE>
__device__ __forceinline__ PfTask<pf_q<TILE>()> pf_task(const PfArgs &a, int task, int NB,
                                                        int ntask, __amdgpu_buffer_rsrc_t rtok) {
  PfTask<pf_q<TILE>()> t;
  t.task = task;
  const bool ok = task < ntask;
  const int tile = ok ? task / NB : 0;
  const int4 tl = a.tiles[tile];
  t.blk = ok ? task - tile * NB : 0;
  t.e0 = __builtin_amdgcn_readfirstlane(tl.y);
  t.n = ok ? __builtin_amdgcn_readfirstlane(tl.z) : 0;
  t.nct = (t.n + 15) / 16;
  const int p = __builtin_amdgcn_readfirstlane(tl.x);
  const size_t ex = p == 0 ? (size_t)a.E : (size_t)(p - 1);
  const size_t mat = (size_t)a.I * a.H;
  t.body = GU ? a.gu_body + ex * 2 * mat : a.dn_body + ex * mat;
  t.sign = GU ? a.gu_sign + ex * 2 * (mat / 8) : a.dn_sign + ex * (mat / 8);
  const uint32_t seg = threadIdx.x & 15;
#pragma unroll
  for (int q = 0; q < pf_q<TILE>(); ++q) {
    const int tt = (threadIdx.x >> 4) + 32 * q;
    uint32_t row;
    if (GU)  // the token's x row (gathered)
      row = buf_load4(rtok, tt < t.n ? (uint32_t)(t.e0 + tt) * 4u : kOutOfRange) * (uint32_t)a.Hp;
    else     // the entry's h' row
      row = (uint32_t)(t.e0 + tt) * (uint32_t)a.Ip;
    t.src[q] = tt < t.n ? (row + 8u * seg) * 2u : kOutOfRange;
  }
  const int nv = a.Ip / kMxUnit;
  t.hsrc = (!GU && (int)threadIdx.x < t.n) ? (uint32_t)(t.e0 + threadIdx.x) * (uint32_t)nv * 4u
                                           : kOutOfRange;
  return t;
}

// Grouped GEMM over tasks (tile, block of kPfRows rows), the contraction in
// 128-wide units.  GU: gate and up rows of the block against x (gathered by
// token), epilogue h' = w * silu(gate) * up as scaled hi/lo rows.  !GU: down
// rows against h' (the tile's entries are contiguous), each unit's h' scale
// applied after its MFMAs, epilogue y[entry][row].
//
// Software pipeline over a flat stream of (task, unit) items: while item i is
// computed, the weight tiles and the activation tile of item i + 1 (in the
// next task after a task's last unit) are in flight; every load in the loop is
// issued unconditionally (out-of-range offsets read zero) so the compiler's
// wait counts stay exact and never drain the queue.  One barrier per unit.
// SM is the sign-load form (mx_sign_mode); in form 2 the units of a task come
// in pairs (the host picks it only for an even unit count): the odd unit's
// loads also fetch the sign bytes of the next pair, which the next two units
// decode.
template <bool GU, int RT, int WGCU, int TILE, int SM>
__global__ __launch_bounds__(kPfWaves * 64) __attribute__((amdgpu_waves_per_eu(
    WGCU * kPfWaves / 4, WGCU * kPfWaves / 4))) void k_pf_gemm(const PfArgs a) {
  constexpr int NT = pf_cols<TILE>(), M = GU ? 2 : 1, Q = pf_q<TILE>();
  constexpr int kPfRows = pf_rows<RT>(), kPfWPU = pf_wpu<RT>();
  static_assert(!GU || (kPfWPU * RT * 16 == kMxUnit && kPfWaves % kPfWPU == 0),
                "gate/up waves tile the 128-row units of h'");
  __shared__ __attribute__((aligned(16))) uint8_t lb[2][2 * TILE * kPfPitch];
  __shared__ float red[GU ? kPfWaves : 1][TILE];
  __shared__ float lsc[2][GU ? 1 : TILE];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane & 15, g = lane >> 4;
  const int H = a.H, I = a.I;
  const int rows = GU ? I : H, Kd = GU ? H : I;
  const int nu = (GU ? a.Hp : a.Ip) / kMxUnit, nv = a.Ip / kMxUnit;
  const int NB = (rows + kPfRows - 1) / kPfRows;
  const int ntask = __builtin_amdgcn_readfirstlane(*a.n_tiles) * NB;
  const uint32_t mbytes = (GU ? 2u : 1u) * (uint32_t)I * (uint32_t)H;
  const uint32_t act_bytes = GU ? (uint32_t)a.T * (uint32_t)a.Hp * 2u
                                : (uint32_t)a.A * (uint32_t)a.Ip * 2u;
  const __amdgpu_buffer_rsrc_t rh = make_rsrc(GU ? (const void *)a.xh : (const void *)a.hh, act_bytes);
  const __amdgpu_buffer_rsrc_t rl = make_rsrc(GU ? (const void *)a.xl : (const void *)a.hl, act_bytes);
  const __amdgpu_buffer_rsrc_t rtok = make_rsrc(a.tok, (uint32_t)a.A * 4u);
  const __amdgpu_buffer_rsrc_t rhs = make_rsrc(a.hs, (uint32_t)a.A * (uint32_t)nv * 4u);

  int task = pf_vid();
  if (task >= ntask) return;
  PfTask<Q> cur = pf_task<GU, TILE>(a, task, NB, ntask, rtok);
  PfTask<Q> nxt = pf_task<GU, TILE>(a, task + (int)gridDim.x, NB, ntask, rtok);

  auto stage_src = [&](const PfTask<Q> &t, int u, uint32_t (&src)[Q]) {
#pragma unroll
    for (int q = 0; q < Q; ++q)
      src[q] = t.src[q] == kOutOfRange ? kOutOfRange : t.src[q] + (uint32_t)u * (2u * kMxUnit);
  };
  auto scale_src = [&](const PfTask<Q> &t, int u) {
    return t.hsrc == kOutOfRange ? kOutOfRange : t.hsrc + (uint32_t)u * 4u;
  };
  auto load_w = [&](MxTile (&w)[RT][M], const PfTask<Q> &t, int u) {
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(t.body, mbytes);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(t.sign, mbytes / 8u);
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const int row = t.blk * kPfRows + wave * RT * 16 + 16 * r + (lane >> 2);
      const bool rv = row < rows && t.n > 0;
      const int r0 = t.blk * kPfRows + wave * RT * 16 + 16 * r;
#pragma unroll
      for (int m = 0; m < M; ++m) {
        mx_load_body_ln<kPfWeightPolicy>(w[r][m], rb, (uint32_t)(m * I), r0, rows, (uint32_t)Kd,
                                         (uint32_t)(u * kMxUnit), t.n > 0);
        w[r][m].s = mx_load_sign_word<SM == 1>(rs, (uint32_t)(m * I + row), (uint32_t)Kd,
                                               (uint32_t)(u * kMxUnit), rv);
      }
    }
  };
  // form 2: the body of unit u, and (signs) the sign words of units u, u + 1
  auto load_body = [&](MxBody (&w)[RT][M], const PfTask<Q> &t, int u) {
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(t.body, mbytes);
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const int r0 = t.blk * kPfRows + wave * RT * 16 + 16 * r;
#pragma unroll
      for (int m = 0; m < M; ++m)
        mx_load_body_ln<kPfWeightPolicy>(w[r][m], rb, (uint32_t)(m * I), r0, rows, (uint32_t)Kd,
                                         (uint32_t)(u * kMxUnit), t.n > 0);
    }
  };
  auto load_signs = [&](MxSigns (&w)[RT][M], const PfTask<Q> &t, int u) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(t.sign, mbytes / 8u);
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const int row = t.blk * kPfRows + wave * RT * 16 + 16 * r + (lane >> 2);
      const bool rv = row < rows && t.n > 0;
#pragma unroll
      for (int m = 0; m < M; ++m)
        mx_load_signs<2>(w[r][m], rs, (uint32_t)(m * I + row), (uint32_t)Kd, (uint32_t)(u * kMxUnit), rv);
    }
  };

  f4v_t acc[RT][M][NT];
  auto zero = [&]() {
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int m = 0; m < M; ++m)
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) acc[r][m][ct] = f4v_t{0, 0, 0, 0};
  };
  zero();

  PfStage<Q> stg;
  MxTile raw[RT][M];     // forms 0 and 1
  MxBody rawb[RT][M];    // form 2: the unit's body ...
  MxSigns sgn[RT][M];    // ... and its pair's sign words
  float scv = 0.0f;
  {
    uint32_t src[Q];
    stage_src(cur, 0, src);
    pf_stage_load(stg, rh, rl, src, 0);
    scv = __builtin_bit_cast(float, buf_load4(rhs, scale_src(cur, 0)));
    if constexpr (SM == 2) {
      load_body(rawb, cur, 0);
      load_signs(sgn, cur, 0);
    } else {
      load_w(raw, cur, 0);
    }
    pf_stage_store<TILE>(stg, lb[0]);
    if (!GU && threadIdx.x < TILE) lsc[0][threadIdx.x] = scv;
    __syncthreads();
  }
  int par = 0;
  // One unit: decode its weights (loaded one unit ahead), issue the next
  // unit's loads, compute against the staged activations, stage the next ones.
  // HALF is the unit's place in its pair (form 2 only).
  auto step = [&](int u, auto half) {
    constexpr int HALF = decltype(half)::value;
    const bool last = u + 1 == nu;
    const PfTask<Q> &nt = last ? nxt : cur;
    const int un = last ? 0 : u + 1;
    uint32_t src[Q];
    stage_src(nt, un, src);
    pf_stage_load(stg, rh, rl, src, 0);
    if (!GU) scv = __builtin_bit_cast(float, buf_load4(rhs, scale_src(nt, un)));
    MxFrag wm[RT][M];
    if constexpr (SM == 2) {
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) wm[r][m] = mx_to_mfma_pair<2, HALF>(rawb[r][m], sgn[r][m]);
      load_body(rawb, nt, un);
      if (HALF == 1) load_signs(sgn, nt, un);  // un starts the next pair
    } else {
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) wm[r][m] = mx_to_mfma(raw[r][m]);
      load_w(raw, nt, un);
    }
    if (GU) {
      pf_unit<RT, M, TILE>(wm, lb[par], cur.nct, acc);
    } else {
      f4v_t tmp[RT][M][NT];
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) tmp[r][0][ct] = f4v_t{0, 0, 0, 0};
      pf_unit<RT, M, TILE>(wm, lb[par], cur.nct, tmp);
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) {
        if (ct < cur.nct) {
          const float sc = lsc[par][16 * ct + j];
#pragma unroll
          for (int r = 0; r < RT; ++r) acc[r][0][ct] += tmp[r][0][ct] * sc;
        }
      }
    }
    pf_stage_store<TILE>(stg, lb[par ^ 1]);
    if (!GU && threadIdx.x < TILE) lsc[par ^ 1][threadIdx.x] = scv;
    __syncthreads();
    par ^= 1;
  };
  for (;;) {
    if constexpr (SM == 2) {
      for (int u = 0; u < nu; u += 2) {
        step(u, std::integral_constant<int, 0>());
        step(u + 1, std::integral_constant<int, 1>());
      }
    } else {
      for (int u = 0; u < nu; ++u) step(u, std::integral_constant<int, 0>());
    }

    const int r0 = cur.blk * kPfRows + wave * RT * 16;  // the wave's first row
    if (GU) {
      // h' = w * silu(gate) * up; per (entry, 128-row unit) scaled hi/lo rows,
      // the unit being the 4 waves q0 .. q0 + 3
      const __amdgpu_buffer_rsrc_t rxi = make_rsrc(a.xinv, (uint32_t)a.T * 4u);
      const __amdgpu_buffer_rsrc_t rwt = make_rsrc(a.wt, (uint32_t)a.A * 4u);
      bool tv[NT];
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) {
        const int tt = 16 * ct + j;
        tv[ct] = tt < cur.n;
        const uint32_t tk = buf_load4(rtok, tv[ct] ? (uint32_t)(cur.e0 + tt) * 4u : kOutOfRange);
        const float xs = __builtin_bit_cast(float, buf_load4(rxi, tv[ct] ? tk * 4u : kOutOfRange));
        const float wv = __builtin_bit_cast(
            float, buf_load4(rwt, tv[ct] ? (uint32_t)(cur.e0 + tt) * 4u : kOutOfRange));
        float m = 0.0f;
#pragma unroll
        for (int r = 0; r < RT; ++r)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float gs = acc[r][0][ct][i] * xs, us = acc[r][M - 1][ct][i] * xs;
            const float hv = (wv == 0.0f) ? 0.0f : wv * (silu(gs) * us);
            acc[r][0][ct][i] = hv;
            m = fmaxf(m, fabsf(hv));
          }
        m = fmaxf(m, __shfl_xor(m, 16));
        m = fmaxf(m, __shfl_xor(m, 32));
        if (g == 0) red[wave][tt] = m;
      }
      __syncthreads();
      const int q0 = wave - wave % kPfWPU;
      const int unit = (cur.blk * kPfRows) / kMxUnit + wave / kPfWPU;
      typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) {
        const int tt = 16 * ct + j;
        float mx = red[q0][tt];
#pragma unroll
        for (int q = 1; q < kPfWPU; ++q) mx = fmaxf(mx, red[q0 + q][tt]);
        const int k = mx_scale_exp(mx);
        const float sc = ldexpf(1.0f, k);
        if (tv[ct] && unit < nv) {
          const size_t rowbase = (size_t)(cur.e0 + tt) * a.Ip;
#pragma unroll
          for (int r = 0; r < RT; ++r) {
            const int row = r0 + 16 * r + 4 * g;
            h4_t hi, lo;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float v = acc[r][0][ct][i] * sc;
              hi[i] = (_Float16)v;
              lo[i] = (_Float16)(v - (float)hi[i]);
            }
            *reinterpret_cast<h4_t *>(a.hh + rowbase + row) = hi;
            *reinterpret_cast<h4_t *>(a.hl + rowbase + row) = lo;
          }
          if (wave == q0 && g == 0) a.hs[(size_t)(cur.e0 + tt) * nv + unit] = ldexpf(1.0f, -k);
        }
      }
      __syncthreads();
    } else {
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) {
        const int tt = 16 * ct + j;
        if (tt < cur.n) {
#pragma unroll
          for (int r = 0; r < RT; ++r) {
            const int row = r0 + 16 * r + 4 * g;
            if (row < H)
              *reinterpret_cast<float4 *>(a.y + (size_t)(cur.e0 + tt) * H + row) =
                  make_float4(acc[r][0][ct][0], acc[r][0][ct][1], acc[r][0][ct][2],
                              acc[r][0][ct][3]);
          }
        }
      }
    }
    zero();
    if (nxt.task >= ntask) break;
    cur = nxt;
    nxt = pf_task<GU, TILE>(a, cur.task + (int)gridDim.x, NB, ntask, rtok);
  }
}

// out[t] = y of token t's entries, shared first, then by id position.
__global__ __launch_bounds__(256) void k_pf_combine(const PfArgs a) {
  const int H4 = a.H / 4, K1 = a.K + 1;
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (size_t)a.T * H4) return;
  const int t = (int)(i / H4), c = (int)(i - (size_t)t * H4);
  const int32_t *te = a.tok_entry + (size_t)t * K1;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int q = 0; q < K1; ++q) {
    const int ent = te[q];
    if (ent >= 0) {
      const float4 v = reinterpret_cast<const float4 *>(a.y + (size_t)ent * a.H)[c];
      s.x += v.x;
      s.y += v.y;
      s.z += v.z;
      s.w += v.w;
    }
  }
  reinterpret_cast<float4 *>(a.out)[i] = s;
}

// ------------------------------------------------------------ host side ----
size_t align256(size_t n) { return (n + 255) / 256 * 256; }

// Entries per tile.  A list longer than a tile streams its expert's weights
// once per tile.  When the routed lists average 49 to 72 entries, many would
// spill just past a 64-entry tile into a second one while nearly all fit in
// 96, so the tiles take 96 entries.  Otherwise the 64-entry tiles keep two
// workgroups per CU on gate/up (measured faster at T = 256, 1024 and 4096 over
// 256 experts, top-8; 96 is faster at 2048).  Without routed ids the one list
// holds every token.
int pf_tile(int T, int K, int E) {
  const long mean = (K > 0 && E > 0) ? (long)T * K / E : T;
  return (mean > 48 && mean <= 72) ? kPfTileMax : kPfTileMin;
}

// One grouped GEMM (gate/up or down) for one tile size and sign-row alignment.
template <bool GU, int RT, int WGCU, int TILE, int SM>
hipError_t launch_pf_gemm(const PfArgs &a, int max_tiles, hipStream_t stream) {
  const int threads = kPfWaves * 64;
  const auto kern = k_pf_gemm<GU, RT, WGCU, TILE, SM>;
  int grid = 0;
  const int NB = ((GU ? a.I : a.H) + pf_rows<RT>() - 1) / pf_rows<RT>();
  static OccCache occ;
  const hipError_t err = persistent_grid(occ, kern, threads, WGCU * kPfWaves, max_tiles * NB, 0,
                                         grid);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(threads), 0, stream, a);
  return hipSuccess;
}

// The sign-load form of one GEMM: that of its weight matrix (K columns, K_p
// padded to whole units), pairs only for an even unit count.
int pf_sign_mode(int K, int Kp, const void *sign) {
  const int sm = mx_sign_mode(K, sign);
  return (sm == 2 && (Kp / kMxUnit) % 2 != 0) ? 1 : sm;
}

// Pairs for a kernel configuration (measured): the gate/up kernel with 96-entry
// tiles has no registers to spare for the second unit's sign words (it spills
// and runs slower), so it keeps one sign load per unit.
#ifndef DUCKMOE_PF_PAIR_GU96
#define DUCKMOE_PF_PAIR_GU96 0
#endif
#ifndef DUCKMOE_PF_PAIR_DN96
#define DUCKMOE_PF_PAIR_DN96 1
#endif
template <bool GU, int TILE>
constexpr bool pf_pairs() {
  return TILE != kPfTileMax || (GU ? DUCKMOE_PF_PAIR_GU96 : DUCKMOE_PF_PAIR_DN96);
}

template <bool GU, int RT, int WGCU, int TILE>
hipError_t launch_pf_gemm_sm(const PfArgs &a, int max_tiles, hipStream_t stream) {
  int sm = GU ? pf_sign_mode(a.H, a.Hp, a.gu_sign) : pf_sign_mode(a.I, a.Ip, a.dn_sign);
  if (!pf_pairs<GU, TILE>() && sm == 2) sm = 1;
  return sm == 2   ? launch_pf_gemm<GU, RT, WGCU, TILE, pf_pairs<GU, TILE>() ? 2 : 1>(a, max_tiles, stream)
         : sm == 1 ? launch_pf_gemm<GU, RT, WGCU, TILE, 1>(a, max_tiles, stream)
                   : launch_pf_gemm<GU, RT, WGCU, TILE, 0>(a, max_tiles, stream);
}

// The two grouped GEMMs for one tile size (gate/up contracts over H, down
// over I; each picks its sign-load form by its own matrix).
template <int TILE, int RG, int CG, int RD, int CD>
hipError_t launch_pf_gemms(const PfArgs &a, int max_tiles, hipStream_t stream) {
  const hipError_t err = launch_pf_gemm_sm<true, RG, CG, TILE>(a, max_tiles, stream);
  if (err != hipSuccess) return err;
  return launch_pf_gemm_sm<false, RD, CD, TILE>(a, max_tiles, stream);
}

struct PfLayout {
  size_t off, tiles, tok, wt, tok_entry, xh, xl, xinv, hh, hl, hs, y, end;
  int Hp, Ip, A, K, max_tiles;
};

PfLayout pf_layout(const duckmoe_layer *L, int T, bool routed) {
  PfLayout l;
  l.K = routed ? L->top_k : 0;
  l.Hp = (L->hidden + kMxUnit - 1) / kMxUnit * kMxUnit;
  l.Ip = (L->inter + kMxUnit - 1) / kMxUnit * kMxUnit;
  l.A = T * (l.K + 1);
  l.max_tiles = (l.A + kPfTileMin - 1) / kPfTileMin + L->n_routed + 1;
  size_t o = 256;  // status word, tile count
  l.off = o;       o = align256(o + (size_t)(L->n_routed + 2) * 4);
  l.tiles = o;     o = align256(o + (size_t)l.max_tiles * 16);
  l.tok = o;       o = align256(o + (size_t)l.A * 4);
  l.wt = o;        o = align256(o + (size_t)l.A * 4);
  l.tok_entry = o; o = align256(o + (size_t)T * (l.K + 1) * 4);
  l.xh = o;        o = align256(o + (size_t)T * l.Hp * 2);
  l.xl = o;        o = align256(o + (size_t)T * l.Hp * 2);
  l.xinv = o;      o = align256(o + (size_t)T * 4);
  l.hh = o;        o = align256(o + (size_t)l.A * l.Ip * 2);
  l.hl = o;        o = align256(o + (size_t)l.A * l.Ip * 2);
  l.hs = o;        o = align256(o + (size_t)l.A * (l.Ip / kMxUnit) * 4);
  l.y = o;         o = align256(o + (size_t)l.A * L->hidden * 4);
  l.end = o;
  return l;
}

int pf_check(const duckmoe_layer *L, int T, bool routed) {
  if (!L || !L->gu_body || !L->gu_sign || !L->dn_body || !L->dn_sign) return DUCKMOE_EINVAL;
  if (T < 1 || T > kPfMaxTokens) return DUCKMOE_EINVAL;
  if (L->hidden < 16 || L->hidden % 16 || L->inter < 16 || L->inter % 16 || L->top_k < 1 ||
      L->n_routed < 0 || L->n_routed > kPfMaxRouted || (routed && L->top_k > kPfMaxTopK))
    return DUCKMOE_ESHAPE;
  if (2ll * L->hidden * L->inter > 0x7fffffffll) return DUCKMOE_ESHAPE;
  const PfLayout l = pf_layout(L, T, routed);
  // 32-bit buffer offsets: the staged operands stay below 2 GiB
  if ((int64_t)T * l.Hp * 2 > 0x7fffffffll || (int64_t)l.A * l.Ip * 2 > 0x7fffffffll)
    return DUCKMOE_ESHAPE;
  if (!aligned(L->gu_body, 16) || !aligned(L->dn_body, 16) || !aligned(L->gu_sign, 2) ||
      !aligned(L->dn_sign, 2))
    return DUCKMOE_EINVAL;
  return DUCKMOE_OK;
}


template <int KM>
void launch_plan_km(const PfArgs &a, hipStream_t st) {
  hipLaunchKernelGGL(k_pf_count<KM>, dim3(a.E + 1), dim3(256), 0, st, a);
  hipLaunchKernelGGL(k_pf_scan, dim3(1), dim3(1024), 0, st, a);
  hipLaunchKernelGGL(k_pf_fill<KM>, dim3(a.E + 1), dim3(256), 0, st, a);
}

// The plan kernels unroll their loops over a token's ids to the smallest
// bound of 8, 16 and kPfMaxTopK that holds K.
hipError_t launch_plan(const PfArgs &a, hipStream_t st) {
  if (a.K <= 8)
    launch_plan_km<8>(a, st);
  else if (a.K <= 16)
    launch_plan_km<16>(a, st);
  else
    launch_plan_km<kPfMaxTopK>(a, st);
  return hipGetLastError();
}

}  // namespace
}  // namespace duckmoe

using namespace duckmoe;

extern "C" {

size_t duckmoe_prefill_workspace_bytes(const duckmoe_layer *L, int32_t T, int32_t routed) {
  if (pf_check(L, T, routed != 0)) return 0;
  return pf_layout(L, T, routed != 0).end;
}

int duckmoe_moe_prefill(const duckmoe_layer *L, const float *x, const int32_t *ids,
                        const float *w, int32_t T, float *out, void *ws, size_t ws_bytes,
                        hipStream_t stream) {
  const bool routed = ids != nullptr;
  int rc = pf_check(L, T, routed);
  if (rc) return rc;
  if (routed && !w) return DUCKMOE_EINVAL;
  if (!x || !out || !ws) return DUCKMOE_EINVAL;
  if (!aligned(x, 16) || !aligned(out, 16) || !aligned(ws, 256)) return DUCKMOE_EINVAL;
  const PfLayout l = pf_layout(L, T, routed);
  if (ws_bytes < l.end) return DUCKMOE_EWORKSPACE;
  uint8_t *b = reinterpret_cast<uint8_t *>(ws);
  PfArgs a;
  a.H = L->hidden;
  a.I = L->inter;
  a.E = L->n_routed;
  a.K = l.K;
  a.T = T;
  a.Hp = l.Hp;
  a.Ip = l.Ip;
  a.A = l.A;
  a.tile = pf_tile(T, l.K, L->n_routed);
  a.gu_body = L->gu_body;
  a.gu_sign = L->gu_sign;
  a.dn_body = L->dn_body;
  a.dn_sign = L->dn_sign;
  a.x = x;
  a.ids = ids;
  a.w = w;
  a.out = out;
  a.status = reinterpret_cast<int32_t *>(b);
  a.n_tiles = reinterpret_cast<int32_t *>(b) + 1;
  a.off = reinterpret_cast<int32_t *>(b + l.off);
  a.tiles = reinterpret_cast<int4 *>(b + l.tiles);
  a.tok = reinterpret_cast<int32_t *>(b + l.tok);
  a.wt = reinterpret_cast<float *>(b + l.wt);
  a.tok_entry = reinterpret_cast<int32_t *>(b + l.tok_entry);
  a.xh = reinterpret_cast<_Float16 *>(b + l.xh);
  a.xl = reinterpret_cast<_Float16 *>(b + l.xl);
  a.xinv = reinterpret_cast<float *>(b + l.xinv);
  a.hh = reinterpret_cast<_Float16 *>(b + l.hh);
  a.hl = reinterpret_cast<_Float16 *>(b + l.hl);
  a.hs = reinterpret_cast<float *>(b + l.hs);
  a.y = reinterpret_cast<float *>(b + l.y);

  if (launch_plan(a, stream) != hipSuccess) return DUCKMOE_EHIP;
  hipLaunchKernelGGL(k_pf_xprep, dim3(T), dim3(256), 0, stream, a);
  const hipError_t err =
      a.tile == kPfTileMax
          ? launch_pf_gemms<kPfTileMax, DUCKMOE_PF_GU_RT96, 1, DUCKMOE_PF_DN_RT,
                            DUCKMOE_PF_DN_WG_PER_CU>(a, l.max_tiles, stream)
          : launch_pf_gemms<kPfTileMin, DUCKMOE_PF_GU_RT, DUCKMOE_PF_GU_WG_PER_CU,
                            DUCKMOE_PF_DN_RT, DUCKMOE_PF_DN_WG_PER_CU>(a, l.max_tiles, stream);
  if (err != hipSuccess) return DUCKMOE_EHIP;
  const size_t n4 = (size_t)T * (a.H / 4);
  hipLaunchKernelGGL(k_pf_combine, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, stream, a);
  return hipGetLastError() == hipSuccess ? DUCKMOE_OK : DUCKMOE_EHIP;
}

int duckmoe_prefill_plan(const int32_t *ids, const float *w, int32_t T, int32_t top_k,
                         int32_t n_routed, int32_t *offsets, int32_t *tokens, float *weights,
                         int32_t *tok_entry, int32_t *status, hipStream_t stream) {
  if (T < 1 || T > kPfMaxTokens || top_k < 0 || top_k > kPfMaxTopK || n_routed < 0 ||
      n_routed > kPfMaxRouted)
    return DUCKMOE_EINVAL;
  if ((top_k > 0 && (!ids || !w)) || !offsets || !tokens || !weights || !tok_entry || !status)
    return DUCKMOE_EINVAL;
  PfArgs a = {};
  a.E = n_routed;
  a.K = top_k;
  a.T = T;
  a.ids = ids;
  a.w = w;
  a.status = status;
  a.n_tiles = nullptr;
  a.tiles = nullptr;
  a.tile = kPfTileMin;  // no tile table is written; the scan still counts tiles
  a.off = offsets;
  a.tok = tokens;
  a.wt = weights;
  a.tok_entry = tok_entry;
  return launch_plan(a, stream) == hipSuccess ? DUCKMOE_OK : DUCKMOE_EHIP;
}

}  // extern "C"
