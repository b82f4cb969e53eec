// duckmoe.hip - device side of libduckmoe: fp9 routed-expert MoE FFN on gfx950.
//
// What is computed (sources cited by page title and section):
//  * fp9 decode and split storage: duck-llm memoir page "一鸭三吃：我把评测鸭
//    变成了满血 DeepSeek-V3.2 推理系统", section "在只有 AVX2 的 N100 上，我先做
//    出了单核 MLP fp9" (see fp9_device.h).
//  * expert FFN of the routed layer, out_t = shared(x_t) + sum_i w_ti expert_i(x_t),
//    top_k = 8 routed experts per token, bsz 1-2: chapter page "第 9 章 MTP1
//    dual-lane overlap", section 9.2 "两条路线的判断"; the expert weights are the
//    part the memoir page's section "真正埋下伏笔的是内存；R1 之后，问题第一次被
//    改写" moves off the GPU.
//  * shard partials: the memoir page's sections "真正难的不是把参数塞下，而是
//    通信" (tensor parallel) and "16 tok/s 之后：一段没有跑通的路" (per-box
//    partials, host reduce); ds4 glossary page "张量并行（Tensor Parallelism,
//    TP）", section "形态一：Mac-to-Mac 张量并行（RDMA）" (f32 partials).
//
// How it maps to CDNA (gfx950): the layer is a weight-streaming GEMV (about 2
// flops per weight byte at bsz 1), so it is HBM-bound and uses the vector ALUs,
// not MFMA.  Two launches per layer:
//   k_gate_up: one workgroup per (expert slot, block of intermediate rows).
//     Each wave owns P (gate row, up row) pairs and walks the hidden dimension
//     in 1024-weight chunks: every lane loads 16 body bytes (one 128-bit load)
//     and 2 sign bytes per row, decodes them in registers and FMAs them against
//     the activation slice it reads from LDS (x is staged there once per
//     workgroup).  At the end the wave sums its lanes with DPP, applies SwiGLU
//     and the routing weight, and stores h' = w * silu(g) * v (f32) in the
//     workspace.
//   k_down: one workgroup per block of R output rows.  Its waves split the
//     (expert slot, 1024-wide chunk of the intermediate dimension) items, each
//     wave streaming the R down rows of its items and FMAing them against h'.
//     Because the routing weight is already folded into h', the weighted
//     combine is part of the same dot product.  Lanes are reduced in groups
//     whose width matches the shard slice, and the waves' partial sums are
//     added in LDS in a fixed order: every output element is written once, no
//     atomics, bit-reproducible run to run.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>

#include "../../include/duckmoe.h"
#include "fp9_device.h"

namespace duckmoe {
namespace {

constexpr int kMaxT = DUCKMOE_MAX_TOKENS;
constexpr int kMaxIds = DUCKMOE_MAX_IDS;
constexpr int kMaxSlots = kMaxIds + 1;
constexpr int kMaxWords = DUCKMOE_MAX_ROUTED / 32;
constexpr int kChunk = 1024;          // weights per wave-row step: 64 lanes x 16
constexpr size_t kHdrBytes = 16384;   // workspace header (status, plan size, fused-path counters)

// Launch shape of the gate/up kernel (compile-time; defaults measured on MI355X).
#ifndef DUCKMOE_GU_WAVES
#define DUCKMOE_GU_WAVES 8     // waves per workgroup
#endif
#ifndef DUCKMOE_GU_PAIRS
#define DUCKMOE_GU_PAIRS 1     // (gate, up) row pairs per wave task
#endif
#ifndef DUCKMOE_GU_PREFETCH
#define DUCKMOE_GU_PREFETCH 1  // 1: next chunk's loads in flight while computing
#endif
#ifndef DUCKMOE_GU_WAVES_PER_CU
#define DUCKMOE_GU_WAVES_PER_CU 16  // target resident waves per CU (capped by occupancy)
#endif
constexpr int kGuTokens = 4;   // tokens per gate/up pass (x of all of them sits in LDS)

// Workspace header, written by block 0 of the gate/up launch: the status word
// and, at kPlanOff, the plan (slot count and expert of each slot) that the down
// launch reads instead of rebuilding it.
struct WsHeader {
  int32_t status;
  int32_t n_slots;
};
constexpr size_t kPlanOff = 4096;

struct LayerArgs {
  int H, I, n_routed, top_k, T, n_shards;
  const uint8_t *gu_body, *gu_sign, *dn_body, *dn_sign;
  const float *x;
  const int32_t *ids;  // nullptr: single-expert mode
  const float *w;
  int single_expert;
  float *out;
  WsHeader *hdr;
  float *hbuf;         // h' [slot][t][I]
};

// ----------------------------------------------------------------- plan ----
// Expert-selection plan, built by every workgroup from the <= 64 routed ids:
// slots 0..n-1 are the ascending distinct valid ids, slot n is the shared
// expert (index n_routed, weight 1).  w[slot][t] is token t's routing weight
// for the slot (summed over repeats, 0 if the token does not use it).
struct PlanLds {
  int n_slots;
  int status;
  int expert[kMaxSlots];
  float w[kMaxSlots][kMaxT];
  int id[kMaxIds];      // the routed ids and weights, staged for the loops below
  float wi[kMaxIds];
};

// Thread tid < T * top_k loads its id and weight before anything else, so that
// the plan's first global round trip is not queued behind other loads.
struct PlanIn {
  int id;
  float w;
};

__device__ __forceinline__ PlanIn plan_load(const LayerArgs &a) {
  PlanIn in{-1, 0.0f};
  const int tid = threadIdx.x;
  if (a.ids != nullptr && tid < a.T * a.top_k) {
    in.id = a.ids[tid];
    if (a.w != nullptr) in.w = a.w[tid];
  }
  return in;
}

// bitmap/prefix: 2 * kMaxWords words of scratch LDS, free again on return.
__device__ void build_plan(PlanLds &P, const LayerArgs &a, const PlanIn in, uint32_t *bitmap,
                           int *prefix) {
  const int tid = threadIdx.x, nt = blockDim.x;
  if (a.ids == nullptr) {
    if (tid == 0) {
      P.n_slots = 1;
      P.status = 0;
      P.expert[0] = a.single_expert;
    }
    if (tid < kMaxT) P.w[0][tid] = 1.0f;
    __syncthreads();
    return;
  }
  const int N = a.T * a.top_k;
  const int nwords = (a.n_routed + 31) >> 5;
  for (int i = tid; i < nwords; i += nt) bitmap[i] = 0u;
  for (int i = tid; i < kMaxSlots * kMaxT; i += nt) (&P.w[0][0])[i] = 0.0f;
  if (tid == 0) P.status = 0;
  if (tid < N) {
    P.id[tid] = in.id;
    P.wi[tid] = in.w;
  }
  __syncthreads();

  const int id = in.id;
  const bool valid = tid < N && id >= 0 && id < a.n_routed;
  const int tok = tid < N ? tid / a.top_k : 0;
  const int base = tok * a.top_k;
  if (tid < N) {
    int st = 0;
    if (!valid) {
      st |= DUCKMOE_STATUS_BAD_ID;
    } else {
      atomicOr(&bitmap[id >> 5], 1u << (id & 31));
      for (int j = base; j < tid; ++j)
        if (P.id[j] == id) st |= DUCKMOE_STATUS_DUP_ID;
    }
    if (st) atomicOr(&P.status, st);
  }
  __syncthreads();
  for (int i = tid; i < nwords; i += nt) prefix[i] = __popc(bitmap[i]);
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int i = 0; i < nwords; ++i) {
      const int c = prefix[i];
      prefix[i] = run;
      run += c;
    }
    P.n_slots = run + 1;
    P.expert[run] = a.n_routed;
  }
  __syncthreads();
  if (valid) {
    const int wd = id >> 5;
    const int slot = prefix[wd] + __popc(bitmap[wd] & ((1u << (id & 31)) - 1u));
    P.expert[slot] = id;  // every lane holding this id writes the same value
    bool first = true;
    for (int j = base; j < tid; ++j)
      if (P.id[j] == id) first = false;
    if (first) {
      float sum = 0.0f;
      for (int j = base; j < base + a.top_k; ++j)
        if (P.id[j] == id) sum += P.wi[j];
      P.w[slot][tok] = sum;
    }
  }
  if (tid < a.T) P.w[P.n_slots - 1][tid] = 1.0f;
  __syncthreads();
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// ------------------------------------------------------------- gate / up ----
// Persistent: grid = resident workgroups, WA waves each.  The tasks are
// (expert slot, group of P intermediate rows); wave w of the grid takes tasks
// w, w + NW, w + 2 NW, ... (NW = all waves).  A wave streams its tasks as one
// sequence of (task, 1024-wide chunk of the hidden dim) units; with PF = 1 the
// loads of the next unit are issued before the current one is computed, so a
// wave keeps 2P rows of weights in flight while it decodes and multiplies.
// The TG tokens t0 .. t0+TG-1 of the call are handled; their activations sit in
// LDS for the whole kernel.  Dynamic LDS: max(TG * H, 2 * kMaxWords) floats.
template <int P>
struct GuTile {
  uint4 d[2][P];
  uint32_t s[2][P];
};

struct GuUnit {              // where one (task, chunk) unit reads from
  __amdgpu_buffer_rsrc_t rb, rs;
  uint32_t row0;             // first intermediate row of the task
  uint32_t kc;               // first weight of the chunk
  int slot;
  int task;
  int c;                     // chunk index
};

template <int P>
__device__ __forceinline__ GuUnit gu_unit(const LayerArgs &a, const PlanLds &plan, int task,
                                          int c) {
  const int NB = a.I / P;
  const int slot = task / NB;
  const int e = __builtin_amdgcn_readfirstlane(plan.expert[slot]);
  const uint32_t mat = (uint32_t)a.I * (uint32_t)a.H;
  GuUnit u;
  u.rb = make_rsrc(a.gu_body + (size_t)e * 2 * mat, 2 * mat);
  u.rs = make_rsrc(a.gu_sign + (size_t)e * 2 * (mat / 8), 2 * (mat / 8));
  u.row0 = (uint32_t)(task - slot * NB) * P;
  u.kc = (uint32_t)c * kChunk;
  u.slot = slot;
  u.task = task;
  u.c = c;
  return u;
}

// The unit after u in a wave's sequence: next chunk, or chunk 0 of task + NW.
template <int P>
__device__ __forceinline__ GuUnit gu_next(const LayerArgs &a, const PlanLds &plan,
                                          const GuUnit &u, int nc, int NW, int ntask) {
  if (u.c + 1 < nc) {
    GuUnit n = u;
    n.c = u.c + 1;
    n.kc = u.kc + kChunk;
    return n;
  }
  if (u.task + NW < ntask) return gu_unit<P>(a, plan, u.task + NW, 0);
  GuUnit n = u;
  n.task = ntask;  // past the end
  return n;
}

template <int P>
__device__ __forceinline__ void gu_issue(GuTile<P> &b, const GuUnit &u, const LayerArgs &a,
                                         int lane) {
  const uint32_t H = a.H, I = a.I;
  const bool kv = u.kc + lane * 16 < H;
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const uint32_t r = g * I + u.row0 + p;
      b.d[g][p] = buf_load16(u.rb, kv ? r * H + u.kc + lane * 16 : kOutOfRange);
      b.s[g][p] = buf_load2(u.rs, kv ? r * (H / 8) + (u.kc + lane * 16) / 8 : kOutOfRange);
    }
}

template <int TG, int P>
__device__ __forceinline__ void gu_consume(const GuTile<P> &b, const float4 *xs4, int Hp4,
                                           uint32_t kc, int lane, float (&acc)[2][P][TG][2]) {
  float xv[TG][16];
#pragma unroll
  for (int t = 0; t < TG; ++t) {
    const float4 *src = xs4 + t * Hp4 + kc / 4 + lane * 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 v = src[j];
      xv[t][4 * j + 0] = v.x;
      xv[t][4 * j + 1] = v.y;
      xv[t][4 * j + 2] = v.z;
      xv[t][4 * j + 3] = v.w;
    }
  }
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int p = 0; p < P; ++p) {
      h2_t h[8];
      fp9_decode16(b.d[g][p], b.s[g][p], h);
#pragma unroll
      for (int t = 0; t < TG; ++t) fma16(h, xv[t], acc[g][p][t][0], acc[g][p][t][1]);
    }
}

template <int TG, int P>
__device__ __forceinline__ void gu_finish(const LayerArgs &a, const PlanLds &plan, int slot,
                                          uint32_t row0, int t0, int lane,
                                          float (&acc)[2][P][TG][2]) {
#pragma unroll
  for (int p = 0; p < P; ++p)
#pragma unroll
    for (int t = 0; t < TG; ++t) {
      const float gsum = wave_sum(acc[0][p][t][0] + acc[0][p][t][1]);
      const float vsum = wave_sum(acc[1][p][t][0] + acc[1][p][t][1]);
      acc[0][p][t][0] = acc[0][p][t][1] = acc[1][p][t][0] = acc[1][p][t][1] = 0.0f;
      if (lane == 0) {
        const float wt = plan.w[slot][t0 + t];
        const float hv = (wt == 0.0f) ? 0.0f : wt * (silu(gsum) * vsum);
        a.hbuf[((size_t)slot * a.T + t0 + t) * a.I + row0 + p] = hv;
      }
    }
}

template <int TG, int P, int WA>
__global__ __launch_bounds__(WA * 64) void k_gate_up(const LayerArgs a, const int t0) {
  __shared__ PlanLds plan;
  extern __shared__ float4 xs4[];  // [TG][nc * 256]: rows padded with zeros to whole chunks
  constexpr int NT = WA * 64;
  constexpr int XR = 8;  // float4 of x per thread loaded before the plan
  const int H = a.H, H4 = a.H / 4;
  const int nc = (H + kChunk - 1) / kChunk;
  const int Hp4 = nc * (kChunk / 4);
  const int n4 = TG * Hp4;
  const float4 *xg = reinterpret_cast<const float4 *>(a.x + (size_t)t0 * H);

  // ids first, then x: the x loads' latency overlaps the plan
  const PlanIn pin = plan_load(a);
  float4 xr[XR];
#pragma unroll
  for (int j = 0; j < XR; ++j) {
    const int q = threadIdx.x + j * NT;
    const int t = q / Hp4, k4 = q - t * Hp4;
    xr[j] = (q < n4 && k4 < H4) ? xg[t * H4 + k4] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  build_plan(plan, a, pin, reinterpret_cast<uint32_t *>(xs4),
             reinterpret_cast<int *>(xs4) + kMaxWords);  // ends with a barrier
  if (blockIdx.x == 0 && t0 == 0) {
    int32_t *wsplan = reinterpret_cast<int32_t *>(reinterpret_cast<uint8_t *>(a.hdr) + kPlanOff);
    if (threadIdx.x == 0) {
      a.hdr->status = plan.status;
      a.hdr->n_slots = plan.n_slots;
      wsplan[0] = plan.n_slots;
    }
    for (int i = threadIdx.x; i < plan.n_slots; i += NT) wsplan[1 + i] = plan.expert[i];
  }

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int NW = gridDim.x * WA;
  const int gw = blockIdx.x * WA + wave;
  const int ntask = plan.n_slots * (a.I / P);

  GuTile<P> b0, b1;
  GuUnit u0, u1;
  u0.task = ntask;
  if (gw < ntask) {
    u0 = gu_unit<P>(a, plan, gw, 0);
    gu_issue(b0, u0, a, lane);
  }
  // activations into LDS (the first XR float4 per thread are already loaded)
#pragma unroll
  for (int j = 0; j < XR; ++j) {
    const int q = threadIdx.x + j * NT;
    if (q < n4) xs4[q] = xr[j];
  }
  for (int q = threadIdx.x + XR * NT; q < n4; q += NT) {
    const int t = q / Hp4, k4 = q - t * Hp4;
    xs4[q] = k4 < H4 ? xg[t * H4 + k4] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  __syncthreads();

  float acc[2][P][TG][2];
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
      for (int t = 0; t < TG; ++t) acc[g][p][t][0] = acc[g][p][t][1] = 0.0f;

  // Two units per trip so that the register buffers keep static names.
  while (u0.task < ntask) {
    u1 = gu_next<P>(a, plan, u0, nc, NW, ntask);
    if (DUCKMOE_GU_PREFETCH && u1.task < ntask) gu_issue(b1, u1, a, lane);
    gu_consume<TG, P>(b0, xs4, Hp4, u0.kc, lane, acc);
    if (u0.c == nc - 1) gu_finish<TG, P>(a, plan, u0.slot, u0.row0, t0, lane, acc);
    if (u1.task >= ntask) break;
    if (!DUCKMOE_GU_PREFETCH) gu_issue(b1, u1, a, lane);

    u0 = gu_next<P>(a, plan, u1, nc, NW, ntask);
    if (DUCKMOE_GU_PREFETCH && u0.task < ntask) gu_issue(b0, u0, a, lane);
    gu_consume<TG, P>(b1, xs4, Hp4, u1.kc, lane, acc);
    if (u1.c == nc - 1) gu_finish<TG, P>(a, plan, u1.slot, u1.row0, t0, lane, acc);
    if (!DUCKMOE_GU_PREFETCH && u0.task < ntask) gu_issue(b0, u0, a, lane);
  }
}

// ------------------------------------------------------------------ down ----
// Persistent: grid = resident workgroups of WB waves; workgroup g takes the
// blocks of R output rows g, g + G, ...  Within a block the waves split the
// (expert slot, 1024-wide chunk of the intermediate dim) items: wave w works
// on chunk c = w % nc for slots w / nc, w / nc + WB / nc, ...  A wave streams
// its items of all its blocks as one sequence, loading the next item while it
// computes the current one (also across blocks).  At the end of a block each
// wave reduces its lanes in groups as wide as a shard slice, the groups' sums
// meet in LDS, and the waves' sums are added in a fixed order: each output
// element is written once, no atomics, bit-reproducible.
// Dynamic LDS: max(WB * R * T * 16, 2 * kMaxWords) floats.
template <int G>
__device__ __forceinline__ void store_groups(float v, float *dst, int lane) {
  v = group_sum<G>(v);
  if ((lane & (G - 1)) == G - 1) dst[lane / G] = v;
}

template <int T, int R>
struct DnTile {
  uint4 d[R];
  uint32_t s[R];
  float4 h[T][4];  // the item's activations h'[slot][t][k .. k+16)
};

template <int T, int R>
__device__ __forceinline__ void dn_issue(DnTile<T, R> &b, const LayerArgs &a, const int32_t *plan,
                                         __amdgpu_buffer_rsrc_t rh, int slot, int row0,
                                         uint32_t k, bool kv) {
  const uint32_t H = a.H, I = a.I;
  const uint32_t mat = H * I;
  const int e = __builtin_amdgcn_readfirstlane(plan[1 + slot]);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(a.dn_body + (size_t)e * mat, mat);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.dn_sign + (size_t)e * (mat / 8), mat / 8);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t row = row0 + r;
    const bool ok = kv && row < H;
    b.d[r] = buf_load16(rb, ok ? row * I + k : kOutOfRange);
    b.s[r] = buf_load2(rs, ok ? row * (I / 8) + k / 8 : kOutOfRange);
  }
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const uint32_t off = kv ? ((uint32_t)(slot * a.T + t) * I + k) * 4u : kOutOfRange;
#pragma unroll
    for (int j = 0; j < 4; ++j) b.h[t][j] = buf_loadf4(rh, off + 16 * j);
  }
}

template <int T, int R>
__device__ __forceinline__ void dn_consume(const DnTile<T, R> &b, float (&acc)[R][T][2]) {
  float hv[T][16];
#pragma unroll
  for (int t = 0; t < T; ++t) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 v = b.h[t][j];
      hv[t][4 * j + 0] = v.x;
      hv[t][4 * j + 1] = v.y;
      hv[t][4 * j + 2] = v.z;
      hv[t][4 * j + 3] = v.w;
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    h2_t h[8];
    fp9_decode16(b.d[r], b.s[r], h);
#pragma unroll
    for (int t = 0; t < T; ++t) fma16(h, hv[t], acc[r][t][0], acc[r][t][1]);
  }
}

// The n_it items (slots s0, s0 + per_c, ...) of one block for one wave.  The
// first item is already in flight in b0; items alternate between b0 and b1,
// the next one always issued before the current one is computed.
template <int T, int R>
__device__ __forceinline__ void dn_block(DnTile<T, R> &b0, DnTile<T, R> &b1, const LayerArgs &a,
                                         const int32_t *plan, __amdgpu_buffer_rsrc_t rh,
                                         int blk, int s0, int per_c, int n_it, uint32_t k,
                                         bool kv, float (&acc)[R][T][2]) {
  for (int i = 0; i < n_it; i += 2) {
    const int slot = s0 + i * per_c;
    if (i + 1 < n_it) dn_issue<T, R>(b1, a, plan, rh, slot + per_c, blk * R, k, kv);
    dn_consume<T, R>(b0, acc);
    if (i + 1 >= n_it) break;
    if (i + 2 < n_it) dn_issue<T, R>(b0, a, plan, rh, slot + 2 * per_c, blk * R, k, kv);
    dn_consume<T, R>(b1, acc);
  }
}

template <int T, int R, int WB>
__global__ __launch_bounds__(WB * 64) void k_down(const LayerArgs a, const int G) {
  extern __shared__ float red[];
  // the plan the gate/up launch left in the workspace (uniform scalar loads)
  const int32_t *plan = reinterpret_cast<const int32_t *>(
      reinterpret_cast<const uint8_t *>(a.hdr) + kPlanOff);
  const int H = a.H, I = a.I;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nc = (I + kChunk - 1) / kChunk;
  const int per_c = WB / nc;  // waves per chunk
  const int S = __builtin_amdgcn_readfirstlane(plan[0]);
  const int nblk = (H + R - 1) / R;
  const int c = wave % nc;
  const uint32_t k = (uint32_t)c * kChunk + lane * 16;
  const bool kv = k < (uint32_t)I;
  const int s0 = wave / nc;  // first slot of this wave in every block
  // items per block for this wave (0 for waves beyond nc * per_c)
  const int n_it = (wave < nc * per_c && s0 < S) ? (S - s0 + per_c - 1) / per_c : 0;
  const __amdgpu_buffer_rsrc_t rh = make_rsrc(a.hbuf, (uint32_t)(S * a.T * I) * 4u);
  const int ns = a.n_shards;
  const int width = I / ns;

  DnTile<T, R> b0, b1;
  if (n_it > 0 && (int)blockIdx.x < nblk)
    dn_issue<T, R>(b0, a, plan, rh, s0, blockIdx.x * R, k, kv);

  for (int blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
    float acc[R][T][2];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int t = 0; t < T; ++t) acc[r][t][0] = acc[r][t][1] = 0.0f;

    if (n_it > 0) {
      dn_block<T, R>(b0, b1, a, plan, rh, blk, s0, per_c, n_it, k, kv, acc);
      // the next block's first item loads while this block is reduced
      if (blk + (int)gridDim.x < nblk)
        dn_issue<T, R>(b0, a, plan, rh, s0, (blk + gridDim.x) * R, k, kv);
    }

    // lane groups of G lanes -> 64/G partial sums per (wave, row, token)
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int t = 0; t < T; ++t) {
        float *dst = red + ((wave * R + r) * T + t) * 16;
        const float v = acc[r][t][0] + acc[r][t][1];
        switch (G) {
          case 4: store_groups<4>(v, dst, lane); break;
          case 8: store_groups<8>(v, dst, lane); break;
          case 16: store_groups<16>(v, dst, lane); break;
          case 32: store_groups<32>(v, dst, lane); break;
          default: store_groups<64>(v, dst, lane); break;
        }
      }
    __syncthreads();

    // combine: output (shard, t, row)
    const int row0 = blk * R;
    for (int q = threadIdx.x; q < ns * T * R; q += WB * 64) {
      const int shard = q / (T * R);
      const int rem = q - shard * (T * R);
      const int t = rem / R, r = rem - t * R;
      const int row = row0 + r;
      if (row >= H) continue;
      int c_lo, c_hi, grp;
      if (ns == 1) {
        c_lo = 0; c_hi = nc; grp = 0;
      } else if (width >= kChunk) {
        c_lo = shard * (width / kChunk); c_hi = c_lo + width / kChunk; grp = 0;
      } else {
        c_lo = (shard * width) / kChunk; c_hi = c_lo + 1;
        grp = ((shard * width) % kChunk) / (G * 16);
      }
      float sum = 0.0f;
      for (int w = 0; w < nc * per_c; ++w) {
        const int cw = w % nc;
        if (cw >= c_lo && cw < c_hi) sum += red[((w * R + r) * T + t) * 16 + grp];
      }
      a.out[((size_t)shard * T + t) * H + row] = sum;
    }
    __syncthreads();  // red is rewritten by the next block
  }
}

// ----------------------------------------------------------------- fused ----
// One launch for the whole layer (T <= 2).  The intermediate dimension is cut
// into n_xcd slices of Ix = I / n_xcd rows, one per XCD of the chip (logical
// XCD of workgroup b: b % n_xcd, which is where the hardware places it); each
// XCD is a tensor-parallel shard in the pages' sense:
//   A. its workgroups stream the gate/up rows of their slice for every plan
//      slot (balanced contiguous ranges of (row pair, 1024-chunk) units per
//      wave; a pair split between two waves is completed through LDS) and
//      write h' with write-through stores;
//   B. once every workgroup of the XCD has finished A (one counter per XCD),
//      each workgroup stages the XCD's h' slice in LDS and streams the down
//      matrices restricted to the slice's columns for a block of output rows,
//      all slots summed;
//   C. the XCD partials of a row block meet in the workspace; the XCD that
//      arrives last (a counter per row block) adds the n_xcd partials in XCD
//      order and writes the output.  In shard mode with one or more shards per
//      XCD, the shard sums are written directly instead.
// Producer/consumer traffic between workgroups uses write-through stores,
// device-coherent atomics and cache-bypassing loads, never a device-scope
// fence (those serialise across the chip).  Waits are bounded (kFuSpin); a
// timeout sets DUCKMOE_STATUS_TIMEOUT.  Every counter is back at zero when the
// launch ends, so a zero-filled workspace stays valid from call to call.
#ifndef DUCKMOE_FU_WAVES
#define DUCKMOE_FU_WAVES 8
#endif
constexpr int kFuSpin = 1 << 22;
constexpr size_t kFuDoneOff = 256;     // uint32 doneA[x] at 256 + 128 x
constexpr size_t kFuPassOff = 1280;    // uint32 passed[x] at 1280 + 128 x
constexpr size_t kFuCntOff = 8192;     // uint32 cnt[r] at 8192 + 64 r
constexpr int kFuMaxXcd = 8;
constexpr int kFuMaxBlocks = 128;      // row blocks (workgroups per XCD)

struct FuArgs {
  uint8_t *hdr;   // workspace header
  float *Y;       // [n_xcd][T][H] XCD partials
  int n_xcd;
  int G;          // lanes per reduction group in B (lane groups of one shard, or of one row)
};

// Phase timestamps (s_memrealtime, 100 MHz) per workgroup, for profiling builds
// only (-DDUCKMOE_FU_TRACE): 8 x u64 per workgroup after the workspace's end.
#ifdef DUCKMOE_FU_TRACE
#define FU_MARK(f, i)                                                                   \
  do {                                                                                \
    if (threadIdx.x == 0)                                                             \
      reinterpret_cast<unsigned long long *>((f).Y + (size_t)kFuMaxXcd * a.T * a.H)[  \
          blockIdx.x * 8 + (i)] = __builtin_amdgcn_s_memrealtime();                   \
  } while (0)
#else
#define FU_MARK(f, i) do { } while (0)
#endif

__device__ __forceinline__ uint32_t *fu_done(const FuArgs &f, int x) {
  return reinterpret_cast<uint32_t *>(f.hdr + kFuDoneOff + 128 * x);
}
__device__ __forceinline__ uint32_t *fu_pass(const FuArgs &f, int x) {
  return reinterpret_cast<uint32_t *>(f.hdr + kFuPassOff + 128 * x);
}
__device__ __forceinline__ uint32_t *fu_cnt(const FuArgs &f, int r) {
  return reinterpret_cast<uint32_t *>(f.hdr + kFuCntOff + 64 * r);
}
__device__ __forceinline__ void st_through(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ float ld_through(const float *p) {
  return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ uint32_t ld_ctr(uint32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_ctr(uint32_t *p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_ctr(uint32_t *p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// h' of one (slot, row) from the reduced gate/up sums
__device__ __forceinline__ float swiglu_w(float wt, float g, float v) {
  return (wt == 0.0f) ? 0.0f : wt * (silu(g) * v);
}

// B unit: M row groups of RPU rows (one slot's down matrix, the XCD slice's
// columns).  Lane l covers rows q*M*RPU + m*RPU + l / LR (m < M) and the 16
// columns at (l % LR) * 16 of the slice.
#ifndef DUCKMOE_FU_BROWS
#define DUCKMOE_FU_BROWS 4  // M: row groups per lane per B unit
#endif
template <int M>
struct FbTile {
  uint4 d[M];
  uint32_t s[M];
};

template <int M>
__device__ __forceinline__ void fb_issue(FbTile<M> &b, const LayerArgs &a,
                                         __amdgpu_buffer_rsrc_t rb, __amdgpu_buffer_rsrc_t rs,
                                         int q, int RPU, int LR, uint32_t kx, int lane) {
  const uint32_t H = a.H, I = a.I;
  const uint32_t k = kx + (uint32_t)(lane % LR) * 16;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const uint32_t row = (uint32_t)((q * M + m) * RPU + lane / LR);
    const bool ok = row < H;
    b.d[m] = buf_load16(rb, ok ? row * I + k : kOutOfRange);
    b.s[m] = buf_load2(rs, ok ? row * (I / 8) + k / 8 : kOutOfRange);
  }
}

template <int T, int M>
__device__ __forceinline__ void fb_consume(const FbTile<M> &b, const float *hs, int Ix, int slot,
                                           int LR, int lane, float (&acc)[M][T][2]) {
  float xv[T][16];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const float4 *src =
        reinterpret_cast<const float4 *>(hs + (slot * T + t) * Ix + (lane % LR) * 16);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 v = src[j];
      xv[t][4 * j] = v.x; xv[t][4 * j + 1] = v.y; xv[t][4 * j + 2] = v.z; xv[t][4 * j + 3] = v.w;
    }
  }
#pragma unroll
  for (int m = 0; m < M; ++m) {
    h2_t h[8];
    fp9_decode16(b.d[m], b.s[m], h);
#pragma unroll
    for (int t = 0; t < T; ++t) fma16(h, xv[t], acc[m][t][0], acc[m][t][1]);
  }
}

__device__ __forceinline__ float fb_reduce(float v, int G) {
  switch (G) {
    case 4: return group_sum<4>(v);
    case 8: return group_sum<8>(v);
    case 16: return group_sum<16>(v);
    case 32: return group_sum<32>(v);
    default: return group_sum<64>(v);
  }
}

// A cursor over (row pair, chunk) units; pr = pair index within the XCD's list
// (slot-major), ris = row of the pair inside its slot's slice.
struct FaCur {
  int u, pr, c, slot, ris;
};

__device__ __forceinline__ void fa_rsrc(const LayerArgs &a, const PlanLds &plan, int slot,
                                        __amdgpu_buffer_rsrc_t &rb, __amdgpu_buffer_rsrc_t &rs) {
  const int e = __builtin_amdgcn_readfirstlane(plan.expert[slot]);
  const uint32_t mat = (uint32_t)a.I * (uint32_t)a.H;
  rb = make_rsrc(a.gu_body + (size_t)e * 2 * mat, 2 * mat);
  rs = make_rsrc(a.gu_sign + (size_t)e * 2 * (mat / 8), 2 * (mat / 8));
}

template <int T, int WA>
__global__ __launch_bounds__(WA * 64) void k_fused(const LayerArgs a, const FuArgs f) {
  constexpr int M = DUCKMOE_FU_BROWS;
  __shared__ PlanLds plan;
  __shared__ int meta[WA][2];            // pair / row-block index of each wave's split ends
  __shared__ float pa[WA][2][T][2];      // A split partials (g, v)
  __shared__ float pb[WA][2][M][T][16];  // B split partials (64 / G groups per row group)
  __shared__ uint32_t bcast;
  extern __shared__ float4 lds4[];       // xs [T][Hp] | hs [S][T][Ix]
  constexpr int NT = WA * 64;
  constexpr int XR = 8;
  const int H = a.H, I = a.I, H4 = a.H / 4;
  const int nc = (H + kChunk - 1) / kChunk;
  const int Hp4 = nc * (kChunk / 4);
  const int n4 = T * Hp4;
  const float4 *xg = reinterpret_cast<const float4 *>(a.x);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  FU_MARK(f, 0);

  // ---- prologue: ids, then x loads overlapping the plan; x into LDS
  const PlanIn pin = plan_load(a);
  float4 xr[XR];
#pragma unroll
  for (int j = 0; j < XR; ++j) {
    const int q = threadIdx.x + j * NT;
    const int t = q / Hp4, k4 = q - t * Hp4;
    xr[j] = (q < n4 && k4 < H4) ? xg[t * H4 + k4] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  build_plan(plan, a, pin, reinterpret_cast<uint32_t *>(lds4),
             reinterpret_cast<int *>(lds4) + kMaxWords);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    a.hdr->status = plan.status;
    a.hdr->n_slots = plan.n_slots;
  }
#pragma unroll
  for (int j = 0; j < XR; ++j) {
    const int q = threadIdx.x + j * NT;
    if (q < n4) lds4[q] = xr[j];
  }
  for (int q = threadIdx.x + XR * NT; q < n4; q += NT) {
    const int t = q / Hp4, k4 = q - t * Hp4;
    lds4[q] = k4 < H4 ? xg[t * H4 + k4] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  if (threadIdx.x < 2 * WA) (&meta[0][0])[threadIdx.x] = -1;
  __syncthreads();
  FU_MARK(f, 1);

  const int S = plan.n_slots;
  const int nx = f.n_xcd;
  const int xcd = blockIdx.x % nx;
  const int r = blockIdx.x / nx;
  const int Gx = gridDim.x / nx;
  const int Ix = I / nx;
  const uint32_t kx = (uint32_t)xcd * Ix;
  float *hs = reinterpret_cast<float *>(lds4 + n4);

  // ---- A: gate/up pairs of this XCD's slice
  {
    const int PT = S * Ix;
    const int p0 = (int)((long)r * PT / Gx), p1 = (int)((long)(r + 1) * PT / Gx);
    const int U = (p1 - p0) * nc;
    const int u0 = (int)((long)wave * U / WA), u1 = (int)((long)(wave + 1) * U / WA);
    float acc[2][1][T][2];
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int t = 0; t < T; ++t) acc[g][0][t][0] = acc[g][0][t][1] = 0.0f;
    // at the last unit of a pair, or of the range: reduce, then finish or park
    auto pair_end = [&](const FaCur &cu) {
      const bool whole_start = cu.u - cu.c >= u0;  // the pair's chunk 0 is in range
      const bool done = cu.c == nc - 1;
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const float gs = wave_sum(acc[0][0][t][0] + acc[0][0][t][1]);
        const float vs = wave_sum(acc[1][0][t][0] + acc[1][0][t][1]);
        acc[0][0][t][0] = acc[0][0][t][1] = acc[1][0][t][0] = acc[1][0][t][1] = 0.0f;
        if (lane == 0) {
          if (whole_start && done) {
            st_through(a.hbuf + ((size_t)cu.slot * T + t) * I + kx + cu.ris,
                       swiglu_w(plan.w[cu.slot][t], gs, vs));
          } else {
            pa[wave][whole_start ? 1 : 0][t][0] = gs;
            pa[wave][whole_start ? 1 : 0][t][1] = vs;
          }
        }
      }
      if (!(whole_start && done) && lane == 0) meta[wave][whole_start ? 1 : 0] = cu.pr;
    };
    if (u0 < u1) {
      FaCur cur;
      cur.u = u0;
      cur.pr = p0 + u0 / nc;
      cur.c = u0 - (cur.pr - p0) * nc;
      cur.slot = cur.pr / Ix;
      cur.ris = cur.pr - cur.slot * Ix;
      __amdgpu_buffer_rsrc_t rb, rs;
      fa_rsrc(a, plan, cur.slot, rb, rs);
      auto unit = [&](const FaCur &cu) {
        GuUnit un;
        un.rb = rb;
        un.rs = rs;
        un.row0 = kx + (uint32_t)cu.ris;
        un.kc = (uint32_t)cu.c * kChunk;
        return un;
      };
      auto advance = [&](FaCur &cu) {
        ++cu.u;
        if (++cu.c == nc) {
          cu.c = 0;
          ++cu.pr;
          if (++cu.ris == Ix) {
            cu.ris = 0;
            ++cu.slot;
            if (cu.u < u1) fa_rsrc(a, plan, cu.slot, rb, rs);
          }
        }
      };
      GuTile<1> b0, b1;
      FaCur c0 = cur, c1;
      gu_issue(b0, unit(c0), a, lane);
      while (true) {
        c1 = c0;
        advance(c1);
        if (c1.u < u1) gu_issue(b1, unit(c1), a, lane);
        gu_consume<T, 1>(b0, lds4, Hp4, (uint32_t)c0.c * kChunk, lane, acc);
        if (c0.c == nc - 1 || c0.u + 1 == u1) pair_end(c0);
        if (c1.u >= u1) break;
        c0 = c1;
        advance(c0);
        if (c0.u < u1) gu_issue(b0, unit(c0), a, lane);
        gu_consume<T, 1>(b1, lds4, Hp4, (uint32_t)c1.c * kChunk, lane, acc);
        if (c1.c == nc - 1 || c1.u + 1 == u1) pair_end(c1);
        if (c0.u >= u1) break;
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  FU_MARK(f, 2);
  // pairs split between waves: sum the parts in wave order, then finish
  if (threadIdx.x < 2 * WA) {
    const int w = threadIdx.x >> 1, side = threadIdx.x & 1;
    const int pr = meta[w][side];
    bool first = pr >= 0;
    for (int w2 = 0; w2 <= w && first; ++w2)
      for (int s2 = 0; s2 < 2; ++s2)
        if ((w2 < w || s2 < side) && meta[w2][s2] == pr) first = false;
    if (first) {
      const int slot = pr / Ix;
      for (int t = 0; t < T; ++t) {
        float gs = 0.0f, vs = 0.0f;
        for (int w2 = 0; w2 < WA; ++w2)
          for (int s2 = 0; s2 < 2; ++s2)
            if (meta[w2][s2] == pr) { gs += pa[w2][s2][t][0]; vs += pa[w2][s2][t][1]; }
        st_through(a.hbuf + ((size_t)slot * T + t) * I + kx + (pr - slot * Ix),
                   swiglu_w(plan.w[slot][t], gs, vs));
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x < 2 * WA) (&meta[0][0])[threadIdx.x] = -1;

  // ---- B setup: this workgroup's row blocks; first unit in flight during the wait
  const int LR = Ix / 16;          // lanes per row
  const int RPU = 64 / LR;         // rows per row group
  const int nq = (H + M * RPU - 1) / (M * RPU);
  const int q0 = (int)((long)r * nq / Gx), q1 = (int)((long)(r + 1) * nq / Gx);
  const int UB = (q1 - q0) * S;
  const int ub0 = (int)((long)wave * UB / WA), ub1 = (int)((long)(wave + 1) * UB / WA);
  const uint32_t dmat = (uint32_t)H * (uint32_t)I;
  auto drsrc = [&](int slot, __amdgpu_buffer_rsrc_t &rb, __amdgpu_buffer_rsrc_t &rs) {
    const int e = __builtin_amdgcn_readfirstlane(plan.expert[slot]);
    rb = make_rsrc(a.dn_body + (size_t)e * dmat, dmat);
    rs = make_rsrc(a.dn_sign + (size_t)e * (dmat / 8), dmat / 8);
  };
  FbTile<M> t0, t1;
  int bq = 0, bs = 0;  // B cursor: row block, slot
  if (ub0 < ub1) {
    bq = q0 + ub0 / S;
    bs = ub0 - (bq - q0) * S;
    __amdgpu_buffer_rsrc_t rb, rs;
    drsrc(bs, rb, rs);
    fb_issue<M>(t0, a, rb, rs, bq, RPU, LR, kx, lane);
  }

  // ---- wait for the XCD's A phase; stage its h' slice
  if (threadIdx.x == 0) {
    add_ctr(fu_done(f, xcd), 1u);
    int it = 0;
    while (ld_ctr(fu_done(f, xcd)) < (uint32_t)Gx && it < kFuSpin) {
      __builtin_amdgcn_s_sleep(2);
      ++it;
    }
    if (it >= kFuSpin) atomicOr(&a.hdr->status, DUCKMOE_STATUS_TIMEOUT);
  }
  __syncthreads();
  FU_MARK(f, 3);
  if (threadIdx.x == 0) {
    if (add_ctr(fu_pass(f, xcd), 1u) == (uint32_t)Gx - 1) {  // everyone is past the wait
      st_ctr(fu_done(f, xcd), 0u);
      st_ctr(fu_pass(f, xcd), 0u);
    }
  }
  for (int q = threadIdx.x; q < S * T * Ix; q += NT) {
    const int st = q / Ix, i = q - st * Ix;  // st = slot * T + t
    hs[q] = ld_through(a.hbuf + (size_t)st * I + kx + i);
  }
  __syncthreads();
  FU_MARK(f, 4);

  // ---- B: down rows x slice columns, all slots; units (row block q, slot s)
  const int G = f.G;               // lanes per reduction group
  const int ns = a.n_shards;
  {
    float acc[M][T][2];
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
      for (int t = 0; t < T; ++t) acc[m][t][0] = acc[m][t][1] = 0.0f;
    auto emit = [&](int row, int t, int lanepos, float v) {
      if (row >= H) return;
      if (ns == 1) {
        st_through(f.Y + ((size_t)xcd * T + t) * H + row, v);
      } else {
        const int shard = (int)((kx + (lanepos % LR) / G * G * 16) / (uint32_t)(I / ns));
        a.out[((size_t)shard * T + t) * H + row] = v;
      }
    };
    // after the last slot of a row block, or at the end of the range
    auto block_end = [&](int u, int q, int sl) {
      const bool whole_start = u - sl >= ub0;
      const bool done = sl == S - 1;
#pragma unroll
      for (int m = 0; m < M; ++m)
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const float v = fb_reduce(acc[m][t][0] + acc[m][t][1], G);
          acc[m][t][0] = acc[m][t][1] = 0.0f;
          if ((lane & (G - 1)) == G - 1) {
            if (whole_start && done)
              emit((q * M + m) * RPU + lane / LR, t, lane, v);
            else
              pb[wave][whole_start ? 1 : 0][m][t][lane / G] = v;
          }
        }
      if (!(whole_start && done) && lane == 0) meta[wave][whole_start ? 1 : 0] = q;
    };
    if (ub0 < ub1) {
      __amdgpu_buffer_rsrc_t rb, rs;
      int u = ub0, q = bq, sl = bs;
      while (true) {
        // next unit's cursor
        int q1n = q, s1n = sl + 1;
        if (s1n == S) { s1n = 0; ++q1n; }
        if (u + 1 < ub1) { drsrc(s1n, rb, rs); fb_issue<M>(t1, a, rb, rs, q1n, RPU, LR, kx, lane); }
        fb_consume<T, M>(t0, hs, Ix, sl, LR, lane, acc);
        if (sl == S - 1 || u + 1 == ub1) block_end(u, q, sl);
        if (++u >= ub1) break;
        q = q1n; sl = s1n;
        int q2n = q, s2n = sl + 1;
        if (s2n == S) { s2n = 0; ++q2n; }
        if (u + 1 < ub1) { drsrc(s2n, rb, rs); fb_issue<M>(t0, a, rb, rs, q2n, RPU, LR, kx, lane); }
        fb_consume<T, M>(t1, hs, Ix, sl, LR, lane, acc);
        if (sl == S - 1 || u + 1 == ub1) block_end(u, q, sl);
        if (++u >= ub1) break;
        q = q2n; sl = s2n;
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  FU_MARK(f, 5);
  // row blocks split between waves: sum the parts in wave order
  for (int e = threadIdx.x; e < 2 * WA * 64; e += NT) {
    const int ws = e / 64, ln = e % 64;  // (wave, side) entry, lane position
    const int w = ws >> 1, side = ws & 1;
    const int q = meta[w][side];
    if (q < 0 || (ln & (G - 1)) != G - 1) continue;
    bool first = true;
    for (int w2 = 0; w2 <= w && first; ++w2)
      for (int s2 = 0; s2 < 2; ++s2)
        if ((w2 < w || s2 < side) && meta[w2][s2] == q) first = false;
    if (!first) continue;
    for (int m = 0; m < M; ++m) {
      const int row = (q * M + m) * RPU + ln / LR;
      if (row >= H) continue;
      for (int t = 0; t < T; ++t) {
        float v = 0.0f;
        for (int w2 = 0; w2 < WA; ++w2)
          for (int s2 = 0; s2 < 2; ++s2)
            if (meta[w2][s2] == q) v += pb[w2][s2][m][t][ln / G];
        if (ns == 1) {
          st_through(f.Y + ((size_t)xcd * T + t) * H + row, v);
        } else {
          const int shard = (int)((kx + (ln % LR) / G * G * 16) / (uint32_t)(I / ns));
          a.out[((size_t)shard * T + t) * H + row] = v;
        }
      }
    }
  }
  if (ns != 1) return;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // ---- C: the last XCD to finish this row range adds the partials in XCD order
  FU_MARK(f, 6);
  if (threadIdx.x == 0) bcast = add_ctr(fu_cnt(f, r), 1u);
  __syncthreads();
  if (bcast != (uint32_t)nx - 1) return;
  const int row_lo = q0 * M * RPU, row_hi = min(q1 * M * RPU, H);
  for (int q = threadIdx.x; q < (row_hi - row_lo) * T; q += NT) {
    const int t = q / (row_hi - row_lo), row = row_lo + q % (row_hi - row_lo);
    float v = 0.0f;
    for (int x2 = 0; x2 < nx; ++x2) v += ld_through(f.Y + ((size_t)x2 * T + t) * H + row);
    a.out[(size_t)t * H + row] = v;
  }
  if (threadIdx.x == 0) st_ctr(fu_cnt(f, r), 0u);
  FU_MARK(f, 7);
}

// ------------------------------------------------------ building blocks ----
__global__ __launch_bounds__(256) void k_decode(const uint8_t *__restrict__ body,
                                                const uint8_t *__restrict__ sign, int64_t n,
                                                float *__restrict__ out) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t groups = (n + 7) / 8;
  if (g >= groups) return;
  const int64_t base = g * 8;
  const int cnt = (int)min<int64_t>(8, n - base);
  uint32_t dw[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (i < cnt) dw[i >> 2] |= (uint32_t)body[base + i] << (8 * (i & 3));
  h2_t h[4];
  fp9_decode8(dw[0], dw[1], sign[g], h);
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (i < cnt) out[base + i] = (i & 1) ? (float)h[i >> 1].y : (float)h[i >> 1].x;
}

// y = W x: each wave owns R rows, lanes stride over groups of 8 weights.
template <int R>
__global__ __launch_bounds__(256) void k_gemv(const uint8_t *__restrict__ body,
                                              const uint8_t *__restrict__ sign, int rows,
                                              int cols, const float *__restrict__ x,
                                              float *__restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int row0 = (blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)) * R;
  if (row0 >= rows) return;  // whole wave
  const int ng = cols / 8;
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.0f;
  for (int g = lane; g < ng; g += 64) {
    const float4 xa = *reinterpret_cast<const float4 *>(x + 8 * g);
    const float4 xb = *reinterpret_cast<const float4 *>(x + 8 * g + 4);
    const float xv[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int row = row0 + r;
      if (row < rows) {
        const uint2 d = *reinterpret_cast<const uint2 *>(body + (size_t)row * cols + 8 * g);
        const uint32_t s = sign[(size_t)row * ng + g];
        h2_t h[4];
        fp9_decode8(d.x, d.y, s, h);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          acc[r] = __builtin_fmaf((float)h[p].x, xv[2 * p], acc[r]);
          acc[r] = __builtin_fmaf((float)h[p].y, xv[2 * p + 1], acc[r]);
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float v = wave_sum(acc[r]);
    if (lane == 0 && row0 + r < rows) y[row0 + r] = v;
  }
}

__global__ __launch_bounds__(64) void k_plan(const LayerArgs a, int32_t *uniq, int32_t *n_slots) {
  __shared__ PlanLds plan;
  __shared__ uint32_t scratch[2 * kMaxWords];
  build_plan(plan, a, plan_load(a), scratch, reinterpret_cast<int *>(scratch) + kMaxWords);
  for (int s = threadIdx.x; s < plan.n_slots; s += blockDim.x) uniq[s] = plan.expert[s];
  if (threadIdx.x == 0) *n_slots = plan.n_slots;
}

// ------------------------------------------------------------ host side ----
bool aligned(const void *p, size_t n) { return ((uintptr_t)p % n) == 0; }

constexpr size_t kGuXLds = 131072;  // LDS bytes for the activations of one gate/up pass

// tokens the gate/up kernel takes per pass for a given hidden size (0: too wide)
int gu_tokens_per_pass(int H) {
  const size_t hp = (size_t)((H + kChunk - 1) / kChunk) * kChunk;
  return (int)std::min<size_t>(kGuTokens, kGuXLds / (hp * sizeof(float)));
}



int check_layer(const duckmoe_layer *L) {
  if (!L || !L->gu_body || !L->gu_sign || !L->dn_body || !L->dn_sign) return DUCKMOE_EINVAL;
  if (L->hidden < 16 || L->hidden % 16 || L->inter < 16 || L->inter % 16 || L->inter > 4096 ||
      L->top_k < 1 || L->n_routed < 1 || L->n_routed > DUCKMOE_MAX_ROUTED)
    return DUCKMOE_ESHAPE;
  // one buffer descriptor spans an expert's gate+up bodies: 2*H*I < 2^31
  if (2ll * L->hidden * L->inter > 0x7fffffffll) return DUCKMOE_ESHAPE;
  if (gu_tokens_per_pass(L->hidden) < 1) return DUCKMOE_ESHAPE;
  if (!aligned(L->gu_body, 16) || !aligned(L->dn_body, 16) || !aligned(L->gu_sign, 2) ||
      !aligned(L->dn_sign, 2))
    return DUCKMOE_EINVAL;
  return DUCKMOE_OK;
}

int check_shards(int I, int ns) {
  if (ns < 1 || I % ns) return DUCKMOE_ESHAPE;
  if (ns == 1) return DUCKMOE_OK;
  const int w = I / ns;
  if (w % kChunk == 0) return DUCKMOE_OK;
  if (w >= 64 && w <= kChunk && (w & (w - 1)) == 0) return DUCKMOE_OK;
  return DUCKMOE_ESHAPE;
}

int group_width(int I, int ns) {
  if (ns == 1) return 64;
  const int w = I / ns;
  return w >= kChunk ? 64 : w / 16;
}

size_t hbuf_slots(const duckmoe_layer *L, int T, bool single) {
  return single ? 1 : (size_t)T * L->top_k + 1;
}

size_t hbuf_bytes(const duckmoe_layer *L, int T, bool single) {
  return hbuf_slots(L, T, single) * (size_t)T * L->inter * sizeof(float);
}

// header | h' [slots][T][I] | XCD partials [kFuMaxXcd][T][H] (fused path)
size_t ws_need(const duckmoe_layer *L, int T, bool single) {
  return kHdrBytes + hbuf_bytes(L, T, single) +
         (size_t)kFuMaxXcd * T * L->hidden * sizeof(float);
}

// Launch shape of the down kernel (compile-time; defaults measured on MI355X).
#ifndef DUCKMOE_DN_WAVES
#define DUCKMOE_DN_WAVES 2          // waves per workgroup
#endif
#ifndef DUCKMOE_DN_ROWS
#define DUCKMOE_DN_ROWS 7           // output rows per block at T = 1 (see down_rows)
#endif
#ifndef DUCKMOE_DN_WAVES_PER_CU
#define DUCKMOE_DN_WAVES_PER_CU 16  // target resident waves per CU (capped by occupancy)
#endif
constexpr int kWB = DUCKMOE_DN_WAVES;

// rows per down block: more rows share each h' load, fewer keep registers in check
template <int T>
constexpr int down_rows() {
  return T == 1 ? DUCKMOE_DN_ROWS : (T == 2 ? 2 * DUCKMOE_DN_ROWS : (T <= 4 ? DUCKMOE_DN_ROWS : 2));
}

// Compute units of the current device, cached per device id.
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return -1;
  if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

template <int TG>
hipError_t launch_gate_up_t(const LayerArgs &a, int t0, hipStream_t st) {
  constexpr int P = DUCKMOE_GU_PAIRS, WA = DUCKMOE_GU_WAVES;
  const auto kern = k_gate_up<TG, P, WA>;
  const size_t hp = (size_t)((a.H + kChunk - 1) / kChunk) * kChunk;
  const size_t lds = std::max((size_t)TG * hp * sizeof(float), (size_t)2 * kMaxWords * 4);
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (err != hipSuccess) return err;
  int per_cu = 0;
  err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, WA * 64, lds);
  if (err != hipSuccess) return err;
  const int cus = device_cus();
  if (cus <= 0 || per_cu <= 0) return hipErrorInvalidConfiguration;
  per_cu = std::max(1, std::min(per_cu, DUCKMOE_GU_WAVES_PER_CU / WA));
  hipLaunchKernelGGL(kern, dim3(cus * per_cu), dim3(WA * 64), lds, st, a, t0);
  return hipGetLastError();
}

template <int T>
hipError_t launch_down_t(const LayerArgs &a, hipStream_t st) {
  constexpr int R = down_rows<T>();
  const auto kern = k_down<T, R, kWB>;
  const size_t lds = (size_t)kWB * R * T * 16 * sizeof(float);
  int per_cu = 0;
  hipError_t err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kWB * 64, lds);
  if (err != hipSuccess) return err;
  const int cus = device_cus();
  if (cus <= 0 || per_cu <= 0) return hipErrorInvalidConfiguration;
  per_cu = std::max(1, std::min(per_cu, DUCKMOE_DN_WAVES_PER_CU / kWB));
  const int nblk = (a.H + R - 1) / R;
  const int grid = std::min(nblk, cus * per_cu);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kWB * 64), lds, st, a,
                     group_width(a.I, a.n_shards));
  return hipGetLastError();
}

hipError_t launch_gate_up(const LayerArgs &a, hipStream_t st) {
  const int tpp = gu_tokens_per_pass(a.H);
  for (int t0 = 0; t0 < a.T; t0 += tpp) {
    hipError_t err;
    switch (std::min(tpp, a.T - t0)) {
      case 1: err = launch_gate_up_t<1>(a, t0, st); break;
      case 2: err = launch_gate_up_t<2>(a, t0, st); break;
      case 3: err = launch_gate_up_t<3>(a, t0, st); break;
      default: err = launch_gate_up_t<4>(a, t0, st); break;
    }
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

hipError_t launch_down(const LayerArgs &a, hipStream_t st) {
  switch (a.T) {
    case 1: return launch_down_t<1>(a, st);
    case 2: return launch_down_t<2>(a, st);
    case 3: return launch_down_t<3>(a, st);
    case 4: return launch_down_t<4>(a, st);
    case 5: return launch_down_t<5>(a, st);
    case 6: return launch_down_t<6>(a, st);
    case 7: return launch_down_t<7>(a, st);
    default: return launch_down_t<8>(a, st);
  }
}

#ifndef DUCKMOE_FU_WAVES_PER_CU
#define DUCKMOE_FU_WAVES_PER_CU 16  // target resident waves per CU (capped by occupancy)
#endif
#ifndef DUCKMOE_FU_COOPERATIVE
#define DUCKMOE_FU_COOPERATIVE 0    // 1: cooperative launch (co-residency guaranteed, ~17 us slower)
#endif
#ifndef DUCKMOE_FUSED
#define DUCKMOE_FUSED 0             // 1: single-launch layer for T <= 2 (slower than two launches
                                    //    as measured on MI355X; kept for experiments)
#endif

// Logical XCDs the fused kernel splits the intermediate dimension over: the
// chip's 8 when the device is a whole MI355X (256 CUs, 32 per XCD).  Any value
// is correct; it only decides locality and balance.
int fused_xcds(int cus) { return (cus >= 64 && cus % 8 == 0) ? 8 : 1; }

// The fused kernel's LDS: x [T][Hp] + the XCD's h' slice [slots][T][Ix].
size_t fused_lds(const LayerArgs &a, int slots, int nx) {
  const size_t hp = (size_t)((a.H + kChunk - 1) / kChunk) * kChunk;
  return (size_t)a.T * hp * sizeof(float) + (size_t)slots * a.T * (a.I / nx) * sizeof(float);
}

bool fused_ok(const LayerArgs &a, int slots, int nx) {
  if (a.T > 2 || a.I % nx) return false;
  const int ix = a.I / nx;
  if (ix < 64 || ix > 1024 || (ix & (ix - 1))) return false;
  if (a.n_shards != 1) {
    const int w = a.I / a.n_shards;  // a power of two in [64, 1024] (check_shards)
    if (w > ix) return false;       // a shard spanning XCDs needs a cross-XCD reduce
  }
  return fused_lds(a, slots, nx) <= 150 * 1024;
}

template <int T>
hipError_t launch_fused_t(const LayerArgs &a, int slots, int nx, FuArgs f, hipStream_t st) {
  constexpr int WA = DUCKMOE_FU_WAVES;
  const auto kern = k_fused<T, WA>;
  const size_t lds = fused_lds(a, slots, nx);
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (err != hipSuccess) return err;
  int per_cu = 0;
  err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, WA * 64, lds);
  if (err != hipSuccess) return err;
  const int cus = device_cus();
  if (cus <= 0 || per_cu <= 0) return hipErrorInvalidConfiguration;
  per_cu = std::max(1, std::min(per_cu, DUCKMOE_FU_WAVES_PER_CU / WA));
  int grid = cus * per_cu;
  grid -= grid % nx;
  if (grid / nx > kFuMaxBlocks) grid = kFuMaxBlocks * nx;
  const int ix = a.I / nx;
  f.G = (a.n_shards == 1) ? ix / 16 : (a.I / a.n_shards) / 16;
  f.n_xcd = nx;
  if (DUCKMOE_FU_COOPERATIVE) {
    LayerArgs aa = a;
    void *args[] = {&aa, &f};
    return hipLaunchCooperativeKernel(reinterpret_cast<const void *>(kern), dim3(grid),
                                      dim3(WA * 64), args, (unsigned)lds, st);
  }
  hipLaunchKernelGGL(kern, dim3(grid), dim3(WA * 64), lds, st, a, f);
  return hipGetLastError();
}

enum Stages { kGateUp = 1, kDown = 2, kBoth = 3 };

// Shared argument checks and dispatch of the layer entry points.
int run_layer(const duckmoe_layer *L, const float *x, const int32_t *ids, const float *w,
              int single_expert, int32_t T, float *out, int32_t n_shards, void *ws,
              size_t ws_bytes, hipStream_t stream, int stages) {
  int rc = check_layer(L);
  if (rc) return rc;
  const bool single = ids == nullptr;
  if (T < 1 || T > kMaxT) return DUCKMOE_EINVAL;
  if (!single && !w) return DUCKMOE_EINVAL;
  if (!single && T * L->top_k > kMaxIds) return DUCKMOE_ESHAPE;
  if (single && (single_expert < 0 || single_expert > L->n_routed)) return DUCKMOE_EINVAL;
  if (!x || !out || !ws) return DUCKMOE_EINVAL;
  if (!aligned(x, 16) || !aligned(out, 4) || !aligned(ws, 256)) return DUCKMOE_EINVAL;
  rc = check_shards(L->inter, n_shards);
  if (rc) return rc;
  if (ws_bytes < ws_need(L, T, single)) return DUCKMOE_EWORKSPACE;

  LayerArgs a;
  a.H = L->hidden;
  a.I = L->inter;
  a.n_routed = L->n_routed;
  a.top_k = L->top_k;
  a.T = T;
  a.n_shards = n_shards;
  a.gu_body = L->gu_body;
  a.gu_sign = L->gu_sign;
  a.dn_body = L->dn_body;
  a.dn_sign = L->dn_sign;
  a.x = x;
  a.ids = ids;
  a.w = w;
  a.single_expert = single_expert;
  a.out = out;
  a.hdr = reinterpret_cast<WsHeader *>(ws);
  a.hbuf = reinterpret_cast<float *>(reinterpret_cast<uint8_t *>(ws) + kHdrBytes);

  if (DUCKMOE_FUSED && stages == kBoth) {
    const int slots = (int)hbuf_slots(L, T, single);
    const int nx = fused_xcds(device_cus());
    if (fused_ok(a, slots, nx)) {
      FuArgs f;
      f.hdr = reinterpret_cast<uint8_t *>(ws);
      f.Y = reinterpret_cast<float *>(reinterpret_cast<uint8_t *>(ws) + kHdrBytes +
                                      hbuf_bytes(L, T, single));
      const hipError_t err = T == 1 ? launch_fused_t<1>(a, slots, nx, f, stream)
                                    : launch_fused_t<2>(a, slots, nx, f, stream);
      return err == hipSuccess ? DUCKMOE_OK : DUCKMOE_EHIP;
    }
  }
  if (stages & kGateUp) {
    if (launch_gate_up(a, stream) != hipSuccess) return DUCKMOE_EHIP;
  }
  if (stages & kDown) {
    if (launch_down(a, stream) != hipSuccess) return DUCKMOE_EHIP;
  }
  return DUCKMOE_OK;
}

}  // namespace
}  // namespace duckmoe

using namespace duckmoe;

extern "C" {

size_t duckmoe_workspace_bytes(const duckmoe_layer *L, int32_t T, int32_t n_shards) {
  if (check_layer(L) || T < 1 || T > kMaxT || T * L->top_k > kMaxIds ||
      check_shards(L->inter, n_shards))
    return 0;
  return ws_need(L, T, false);
}

int duckmoe_moe_layer(const duckmoe_layer *L, const float *x, const int32_t *ids,
                      const float *w, int32_t T, float *out, int32_t n_shards, void *ws,
                      size_t ws_bytes, hipStream_t stream) {
  if (!ids) return DUCKMOE_EINVAL;
  return run_layer(L, x, ids, w, 0, T, out, n_shards, ws, ws_bytes, stream, kBoth);
}

int duckmoe_moe_gate_up(const duckmoe_layer *L, const float *x, const int32_t *ids,
                        const float *w, int32_t T, float *out, int32_t n_shards, void *ws,
                        size_t ws_bytes, hipStream_t stream) {
  if (!ids) return DUCKMOE_EINVAL;
  return run_layer(L, x, ids, w, 0, T, out, n_shards, ws, ws_bytes, stream, kGateUp);
}

int duckmoe_moe_down(const duckmoe_layer *L, const float *x, const int32_t *ids,
                     const float *w, int32_t T, float *out, int32_t n_shards, void *ws,
                     size_t ws_bytes, hipStream_t stream) {
  if (!ids) return DUCKMOE_EINVAL;
  return run_layer(L, x, ids, w, 0, T, out, n_shards, ws, ws_bytes, stream, kDown);
}

int duckmoe_expert_ffn(const duckmoe_layer *L, int32_t e, const float *x, int32_t T,
                       float *out, int32_t n_shards, void *ws, size_t ws_bytes,
                       hipStream_t stream) {
  return run_layer(L, x, nullptr, nullptr, e, T, out, n_shards, ws, ws_bytes, stream, kBoth);
}

int duckmoe_status(const void *ws, int32_t *status, hipStream_t stream) {
  if (!ws || !status) return DUCKMOE_EINVAL;
  WsHeader h;
  if (hipMemcpyAsync(&h, ws, sizeof(h), hipMemcpyDeviceToHost, stream) != hipSuccess)
    return DUCKMOE_EHIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return DUCKMOE_EHIP;
  *status = h.status;
  return DUCKMOE_OK;
}

int duckmoe_decode_fp9(const uint8_t *body, const uint8_t *sign, int64_t n, float *out,
                       hipStream_t stream) {
  if (n < 0 || !body || !sign || !out) return DUCKMOE_EINVAL;
  if (n == 0) return DUCKMOE_OK;
  const int64_t groups = (n + 7) / 8;
  const int64_t blocks = (groups + 255) / 256;
  if (blocks > 0x7fffffff) return DUCKMOE_ESHAPE;
  hipLaunchKernelGGL(k_decode, dim3((unsigned)blocks), dim3(256), 0, stream, body, sign, n, out);
  return hipGetLastError() == hipSuccess ? DUCKMOE_OK : DUCKMOE_EHIP;
}

int duckmoe_gemv_fp9(const uint8_t *body, const uint8_t *sign, int32_t rows, int32_t cols,
                     const float *x, float *y, hipStream_t stream) {
  if (!body || !sign || !x || !y || rows < 0 || cols < 0) return DUCKMOE_EINVAL;
  if (cols % 8) return DUCKMOE_ESHAPE;
  if (!aligned(body, 8) || !aligned(x, 16) || !aligned(y, 4)) return DUCKMOE_EINVAL;
  if (rows == 0) return DUCKMOE_OK;
  constexpr int R = 4;
  const int waves = (rows + R - 1) / R;
  const int blocks = (waves + 3) / 4;
  hipLaunchKernelGGL((k_gemv<R>), dim3(blocks), dim3(256), 0, stream, body, sign, rows, cols, x,
                     y);
  return hipGetLastError() == hipSuccess ? DUCKMOE_OK : DUCKMOE_EHIP;
}

int duckmoe_moe_plan(const int32_t *ids, int32_t T, int32_t top_k, int32_t n_routed,
                     int32_t *uniq, int32_t *n_slots, hipStream_t stream) {
  if (!ids || !uniq || !n_slots) return DUCKMOE_EINVAL;
  if (T < 1 || T > kMaxT || top_k < 1) return DUCKMOE_EINVAL;
  if (T * top_k > kMaxIds || n_routed < 1 || n_routed > DUCKMOE_MAX_ROUTED)
    return DUCKMOE_ESHAPE;
  LayerArgs a = {};
  a.ids = ids;
  a.T = T;
  a.top_k = top_k;
  a.n_routed = n_routed;
  a.w = nullptr;  // the slot list needs no weights; build_plan skips them
  hipLaunchKernelGGL(k_plan, dim3(1), dim3(64), 0, stream, a, uniq, n_slots);
  return hipGetLastError() == hipSuccess ? DUCKMOE_OK : DUCKMOE_EHIP;
}

}  // extern "C"
