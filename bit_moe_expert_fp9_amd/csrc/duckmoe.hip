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
// flops per weight byte at bsz 1), so it is HBM-bound and, at bsz 1-2, uses the
// vector ALUs, not MFMA.  Two launches per layer:
//   k_gate_up: persistent; each wave takes (expert slot, P intermediate rows)
//     tasks in a strided sequence and walks the hidden dimension in
//     1024-weight chunks: every lane loads 16 body bytes (one 128-bit load)
//     and 2 sign bytes per row (non-temporal: a wave's load covers whole
//     128-byte lines of a weight stream read once per call), decodes them in
//     registers and FMAs them against
//     the activation slice it reads from LDS (x is staged there once per
//     workgroup).  At a task's end the wave sums its lanes with DPP, applies
//     SwiGLU and the routing weight, and stores h' = w * silu(g) * v (f32) in
//     the workspace.  Block 0 also publishes the plan (the distinct experts).
//   k_down: persistent over blocks of R output rows.  A block's waves split the
//     (expert slot, 1024-wide chunk of the intermediate dimension) items, each
//     wave streaming the R down rows of its items and FMAing them against h'.
//     Because the routing weight is already folded into h', the weighted
//     combine is part of the same dot product.  Lanes are reduced in groups
//     whose width matches the shard slice, and the waves' partial sums are
//     added in LDS in a fixed order: every output element is written once, no
//     atomics, bit-reproducible run to run.
// From 3 tokens on (no shard partials) the two contractions run on the matrix
// cores instead (k_mx_xprep, k_gate_up_mx, k_down_mx, k_mx_reduce): the fp9
// weights decode exactly to fp16 A tiles, the activations are split into
// scaled fp16 hi and lo parts that share one B operand (x by k_mx_xprep, h' by
// the gate/up epilogue), and the sums are recombined and unscaled in f32.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>

#include "../../include/duckmoe.h"
#include "fp9_device.h"
#include "host_util.h"
#include "mfma_device.h"

namespace duckmoe {
namespace {

constexpr int kMaxT = DUCKMOE_MAX_TOKENS;
constexpr int kMaxIds = DUCKMOE_MAX_IDS;
constexpr int kChunk = 1024;          // weights per wave-row step: 64 lanes x 16
constexpr int kMaxInter = 32768;      // intermediate size limit (dense MLPs up to 32 chunks)
constexpr size_t kHdrBytes = 1024;    // workspace header (status word, plan)

// Launch shape of the gate/up kernel (compile-time; defaults measured on MI355X).
#ifndef DUCKMOE_GU_WAVES
#define DUCKMOE_GU_WAVES 8     // waves per workgroup
#endif
#ifndef DUCKMOE_GU_PAIRS
#define DUCKMOE_GU_PAIRS 1     // (gate, up) row pairs per wave task
#endif
#ifndef DUCKMOE_GU_DEPTH
#define DUCKMOE_GU_DEPTH 3     // units whose loads a wave keeps in flight (2 or 3)
#endif
#ifndef DUCKMOE_GU_WAVES_PER_CU
#define DUCKMOE_GU_WAVES_PER_CU 16  // target resident waves per CU (capped by occupancy)
#endif
#ifndef DUCKMOE_GU_MAP
#define DUCKMOE_GU_MAP 0
#endif
constexpr int kGuTokens = 4;   // tokens per gate/up pass (x of all of them sits in LDS)

// Workspace header, written by block 0 of the gate/up launch: the status word
// and, at kPlanOff, the plan (slot count and expert of each slot) that the down
// launch reads instead of rebuilding it.
struct WsHeader {
  int32_t status;
  int32_t n_slots;
};
constexpr size_t kPlanOff = 256;   // int32 n_slots, then expert[slot]
constexpr size_t kMaskOff = 640;   // int32 token mask of each slot (bit t: token t names it)

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
  int in_rms;          // 1: normalize each x row by its RMS first (stack glue)
  float in_eps;
  int cus;             // host only: CUs the launches may use (0: the device's)
};

// ----------------------------------------------------------------- plan ----
// Expert-selection plan.  Every wave builds it on its own from the <= 64
// routed ids, one per lane, with cross-lane operations only (no LDS, no
// barrier).  Slot 0 is the shared expert (index n_routed), or the one expert
// of single-expert mode; slots 1 .. n_slots-1 are the distinct valid ids in
// order of first appearance (token-major).  Slot 0 needs no ids, so work on it
// can start before they arrive.  A token's weight for a routed slot is the sum
// of its weights at the positions naming that expert (0 if none); its weight
// for slot 0 is 1.
struct PlanIn {
  int id;
  float w;
};

// Lane j < T * top_k loads position j's id and weight.  Unconditional buffer
// loads (lanes past the end read zero): a branch around a load makes the
// compiler drain every earlier load first.
__device__ __forceinline__ PlanIn plan_load(const LayerArgs &a) {
  const uint32_t n = a.ids != nullptr ? (uint32_t)(a.T * a.top_k) : 0u;
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t off = lane < n ? lane * 4u : kOutOfRange;
  const __amdgpu_buffer_rsrc_t ri = make_rsrc(a.ids, n * 4u);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.w, a.w != nullptr ? n * 4u : 0u);
  PlanIn in;
  in.id = (int)buf_load4(ri, off);
  in.w = __builtin_bit_cast(float, buf_load4(rw, off));
  return in;
}

struct WavePlan {
  int n_slots;  // uniform
  int status;   // uniform: DUCKMOE_STATUS_* bits
  int e0;       // uniform: expert of slot 0
  int slot;     // lane j < T * top_k: slot of position j, -1 if its id is invalid
  float w;      // lane j: routing weight at position j
  int expert;   // lane s < n_slots - 1: expert of slot s + 1
};

__device__ __forceinline__ int slot0_expert(const LayerArgs &a) {
  return a.ids != nullptr ? a.n_routed : a.single_expert;
}

__device__ __forceinline__ WavePlan wave_plan(const LayerArgs &a, const PlanIn in) {
  const int lane = threadIdx.x & 63;
  WavePlan p;
  p.e0 = slot0_expert(a);
  if (a.ids == nullptr) {
    p.n_slots = 1;
    p.status = 0;
    p.slot = -1;
    p.w = 0.0f;
    p.expert = 0;
    return p;
  }
  const int N = a.T * a.top_k;  // <= 64
  const int id = in.id;
  const bool valid = lane < N && id >= 0 && id < a.n_routed;
  const int tok = lane / a.top_k;
  // the earliest position with the same id, and repeats within one token
  int firstk = lane;
  bool dup = false;
  for (int k = 0; k < N; ++k) {
    const int idk = __builtin_amdgcn_readlane(id, k);
    const bool same = valid && k < lane && idk == id;
    if (same && firstk == lane) firstk = k;
    if (same && k / a.top_k == tok) dup = true;
  }
  const bool first = valid && firstk == lane;
  const uint64_t fmask = __builtin_amdgcn_ballot_w64(first);
  const int before = (int)__builtin_amdgcn_mbcnt_hi(
      (uint32_t)(fmask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)fmask, 0u));
  // a first occurrence takes slot 1 + (first occurrences before it); a repeat
  // takes its first occurrence's slot
  const int s = __builtin_amdgcn_ds_bpermute(firstk * 4, 1 + before);
  p.slot = valid ? s : -1;
  p.w = lane < N ? in.w : 0.0f;
  p.n_slots = 1 + (int)__builtin_popcountll(fmask);
  // lane r receives the id of the r-th first occurrence; the other lanes send
  // to lane 63, which holds a slot only when every position is a first one
  p.expert = __builtin_amdgcn_ds_permute((first ? before : 63) * 4, id);
  const uint64_t bad = __builtin_amdgcn_ballot_w64(lane < N && !valid);
  const uint64_t dups = __builtin_amdgcn_ballot_w64(dup);
  p.status = (bad ? DUCKMOE_STATUS_BAD_ID : 0) | (dups ? DUCKMOE_STATUS_DUP_ID : 0);
  return p;
}

// expert of slot s (s uniform, < n_slots)
__device__ __forceinline__ int plan_expert(const WavePlan &p, int s) {
  return s == 0 ? p.e0 : __builtin_amdgcn_readlane(p.expert, s - 1);
}

// token t's routing weight for slot s (s, t uniform)
__device__ __forceinline__ float plan_weight(const WavePlan &p, const LayerArgs &a, int s, int t) {
  if (s == 0) return 1.0f;
  float wt = 0.0f;
  for (int i = 0; i < a.top_k; ++i) {
    const int j = t * a.top_k + i;
    if (__builtin_amdgcn_readlane(p.slot, j) == s)
      wt += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, p.w), j));
  }
  return wt;
}

// Tokens t0 .. t0 + n - 1 that name slot s (bit t for token t0 + t): a token
// that names no position of a routed slot has weight 0 there, so its h' for
// the slot is 0 and its products can be skipped without changing any bit of
// the output (fp9 weights are finite).  Slot 0 serves every token.  s uniform.
__device__ __forceinline__ int slot_tokens(const WavePlan &p, const LayerArgs &a, int s, int t0,
                                           int n) {
  if (s == 0 || a.ids == nullptr) return (1 << n) - 1;
  int m = 0;
  for (int t = 0; t < n; ++t)
    for (int i = 0; i < a.top_k; ++i)
      if (__builtin_amdgcn_readlane(p.slot, (t0 + t) * a.top_k + i) == s) m |= 1 << t;
  return m;
}

// The plan as the down launch reads it from the workspace: int32 n_slots, then
// the expert of each slot; at kMaskOff the token mask of each slot (all T
// tokens).  Written by one wave.
__device__ __forceinline__ void plan_store(const WavePlan &p, const LayerArgs &a) {
  int32_t *dst = reinterpret_cast<int32_t *>(reinterpret_cast<uint8_t *>(a.hdr) + kPlanOff);
  int32_t *msk = reinterpret_cast<int32_t *>(reinterpret_cast<uint8_t *>(a.hdr) + kMaskOff);
  const int lane = threadIdx.x & 63;
  if (lane == 0) {
    a.hdr->status = p.status;
    a.hdr->n_slots = p.n_slots;
    dst[0] = p.n_slots;
    dst[1] = p.e0;
  }
  if (lane < p.n_slots - 1) dst[2 + lane] = p.expert;
  // lane s: the tokens naming slot s (a per-lane slot, so the loop compares
  // every position's slot with the lane's own)
  int m = 0;
  if (lane == 0 || a.ids == nullptr) {
    m = (1 << a.T) - 1;
  } else {
    const int N = a.T * a.top_k;
    for (int j = 0; j < N; ++j)
      if (__builtin_amdgcn_readlane(p.slot, j) == lane) m |= 1 << (j / a.top_k);
  }
  if (lane < p.n_slots) msk[lane] = m;
}

// The RMS glue's sum of squares of one row in a fixed order: thread j < 256
// adds x[j], x[j + 256], ... with fused multiply-adds; each of the 4 waves sums
// its lanes; the 4 wave sums are added as (w0 + w1) + (w2 + w3) by rms_divisor.
// k_rms and the gate/up prologue both use it, so normalizing inside the layer
// gives the same bits as normalizing before it.
__device__ __forceinline__ float rms_wave_part(const float *row, int H) {
  float ss = 0.0f;
  if (threadIdx.x < 256) {
#pragma unroll 8
    for (int i = threadIdx.x; i < H; i += 256) ss = __builtin_fmaf(row[i], row[i], ss);
  }
  return wave_sum(ss);
}

__device__ __forceinline__ float rms_divisor(const float part[4], int H, float eps) {
  return sqrtf(((part[0] + part[1]) + (part[2] + part[3])) / (float)H + eps);
}

// ------------------------------------------------------------- gate / up ----
// Persistent: grid = resident workgroups, WA waves each.  The tasks are
// (expert slot, group of P intermediate rows); wave w of the grid takes tasks
// w, w + NW, w + 2 NW, ... (NW = all waves).  A wave streams its tasks as one
// sequence of (task, 1024-wide chunk of the hidden dim) units and keeps the
// loads of the next DUCKMOE_GU_DEPTH - 1 units in flight while it decodes and
// multiplies the current one.
// The TG tokens t0 .. t0+TG-1 of the call are handled; their activations sit in
// LDS for the whole kernel.  Dynamic LDS: TG rows of H floats, padded to whole chunks.
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
  int tm;                    // tokens of the pass that name the slot (bit t), see slot_tokens
};

template <int P>
__device__ __forceinline__ GuUnit gu_unit(const LayerArgs &a, int e, int task, int c) {
  const int NB = a.I / P;
  const int slot = task / NB;
  const uint32_t mat = (uint32_t)a.I * (uint32_t)a.H;
  GuUnit u;
  u.rb = make_rsrc(a.gu_body + (size_t)e * 2 * mat, 2 * mat);
  u.rs = make_rsrc(a.gu_sign + (size_t)e * 2 * (mat / 8), 2 * (mat / 8));
  u.row0 = (uint32_t)(task - slot * NB) * P;
  u.kc = (uint32_t)c * kChunk;
  u.slot = slot;
  u.task = task;
  u.c = c;
  u.tm = -1;
  return u;
}

// The unit after u in a wave's sequence: next chunk, or chunk 0 of the wave's
// next task (with, from two tokens on, the pass's tokens that name its slot).
//
// Task order.  Tasks are dealt round robin: wave gw takes gw, gw + NW, ...  The
// two workgroups a CU holds do not progress at the same rate: the one
// dispatched first (blocks below gridDim.x / 2, waves below NW / 2) is served
// first.  Per-wave timestamps at two tokens (17 slots, 8.5 tasks per wave)
// had those waves, with 9 tasks each, end at a median of 82 us and the others,
// with 8, at 95 us, the launch ending at ~100 us.  So in a two-token pass
// (two workgroups per CU), when there are at least 4 rounds, the waves of the
// later workgroups stop one round early and the earlier ones take that
// round's tasks and the remainder with stride NW / 2 (10 against 7 tasks):
// gate/up at two tokens 100.8 -> 99.3 us; moving two rounds measured worse
// (103.0 us).  At one token the 5 / 4 split of the plain round robin already
// ends both groups within 1 us.
// Which wave computes a task does not change its result.
template <int TG, int P>
__device__ __forceinline__ GuUnit gu_next(const LayerArgs &a, const WavePlan &plan,
                                          const GuUnit &u, int nc, int NW, int ntask, int t0,
                                          int gw) {
  if (u.c + 1 < nc) {
    GuUnit n = u;
    n.c = u.c + 1;
    n.kc = u.kc + kChunk;
    return n;
  }
  int t = u.task + NW;
  if (TG == 2 && ntask / NW >= 4) {  // two tokens: two workgroups per CU
    const int shared = (ntask / NW - 1) * NW;  // the rounds every wave takes
    if (t >= shared) t = gw >= NW / 2 ? ntask : (u.task < shared ? shared + gw : u.task + NW / 2);
  }
  if (t < ntask) {
    const int slot = t / (a.I / P);
    GuUnit n = gu_unit<P>(a, plan_expert(plan, slot), t, 0);
    if (TG > 1) n.tm = slot_tokens(plan, a, slot, t0, TG);
    return n;
  }
  GuUnit n = u;
  n.task = ntask;  // past the end
  return n;
}

template <int P>
__device__ __forceinline__ void gu_issue(GuTile<P> &b, const GuUnit &u, const LayerArgs &a,
                                         int lane, bool live = true) {
  const uint32_t H = a.H, I = a.I;
  const bool kv = live && u.kc + lane * 16 < H;
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const uint32_t r = g * I + u.row0 + p;
      b.d[g][p] = buf_load16<kStream>(u.rb, kv ? r * H + u.kc + lane * 16 : kOutOfRange);
      b.s[g][p] = buf_load2<kStream>(u.rs, kv ? r * (H / 8) + (u.kc + lane * 16) / 8 : kOutOfRange);
    }
}

// tm: the tokens whose products are needed (bit t); the others' activations
// are not read and their accumulators stay zero (uniform branches).
template <int TG, int P>
__device__ __forceinline__ void gu_consume(const GuTile<P> &b, const float4 *xs4, int Hp4,
                                           uint32_t kc, int lane, float (&acc)[2][P][TG][2],
                                           int tm) {
  float xv[TG][16];
#pragma unroll
  for (int t = 0; t < TG; ++t) {
    if (TG > 1 && !((tm >> t) & 1)) continue;
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
      for (int t = 0; t < TG; ++t)
        if (TG == 1 || ((tm >> t) & 1)) fma16(h, xv[t], acc[g][p][t][0], acc[g][p][t][1]);
    }
}

template <int TG, int P>
__device__ __forceinline__ void gu_finish(const LayerArgs &a, const WavePlan &plan, int slot,
                                          uint32_t row0, int t0, int lane,
                                          float (&acc)[2][P][TG][2]) {
#pragma unroll
  for (int p = 0; p < P; ++p)
#pragma unroll
    for (int t = 0; t < TG; ++t) {
      const float gsum = wave_sum(acc[0][p][t][0] + acc[0][p][t][1]);
      const float vsum = wave_sum(acc[1][p][t][0] + acc[1][p][t][1]);
      acc[0][p][t][0] = acc[0][p][t][1] = acc[1][p][t][0] = acc[1][p][t][1] = 0.0f;
      const float wt = plan_weight(plan, a, slot, t0 + t);
      if (lane == 0) {
        const float hv = (wt == 0.0f) ? 0.0f : wt * (silu(gsum) * vsum);
        a.hbuf[((size_t)slot * a.T + t0 + t) * a.I + row0 + p] = hv;
      }
    }
}

template <int TG, int P, int WA>
__global__ __launch_bounds__(WA * 64) void k_gate_up(const LayerArgs a, const int t0) {
  extern __shared__ float4 xs4[];  // [TG][nc * 256]: rows padded with zeros to whole chunks
  constexpr int NT = WA * 64;
  constexpr int XR = 8;  // float4 of x per thread loaded before the plan
  const int H = a.H, H4 = a.H / 4;
  const int nc = (H + kChunk - 1) / kChunk;
  const int Hp4 = nc * (kChunk / 4);
  const int n4 = TG * Hp4;
  const int NB = a.I / P;  // tasks per slot
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int NW = gridDim.x * WA;
#if DUCKMOE_GU_MAP
  const int gw = wave * gridDim.x + blockIdx.x;
#else
  const int gw = blockIdx.x * WA + wave;
#endif

  // The ids and x first, then a wave whose first task lies in slot 0 (known
  // without the ids) issues its first weight loads at once.  In that order
  // the waits for the ids (the plan) and for x (the LDS staging) do not also
  // wait for those weights (loads complete in issue order).
  GuTile<P> b0, b1;
  GuUnit u0;
  const bool early = gw < NB;
  const PlanIn pin = plan_load(a);
  // x rows t0 .. t0 + TG - 1; unconditional buffer loads, zero past each row's end
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x + (size_t)t0 * H, (uint32_t)(TG * H) * 4u);
  auto x_off = [&](int q) -> uint32_t {
    const int t = q / Hp4, k4 = q - t * Hp4;
    return (q < n4 && k4 < H4) ? (uint32_t)(t * H4 + k4) * 16u : kOutOfRange;
  };
  float4 xr[XR];
#pragma unroll
  for (int j = 0; j < XR; ++j) xr[j] = buf_loadf4(rx, x_off(threadIdx.x + j * NT));
  if (early) {
    u0 = gu_unit<P>(a, slot0_expert(a), gw, 0);
    gu_issue(b0, u0, a, lane);
  }

  const WavePlan plan = wave_plan(a, pin);
  if (blockIdx.x == 0 && wave == 0 && t0 == 0) plan_store(plan, a);
  const int ntask = plan.n_slots * NB;
  if (!early) {
    if (gw < ntask) {
      u0 = gu_unit<P>(a, plan_expert(plan, gw / NB), gw, 0);
      if (TG > 1) u0.tm = slot_tokens(plan, a, gw / NB, t0, TG);
      gu_issue(b0, u0, a, lane);
    } else {
      u0 = gu_unit<P>(a, plan.e0, 0, 0);
      u0.task = ntask;  // no work: past the end
    }
  }

  // activations into LDS (the first XR float4 per thread are already loaded)
#pragma unroll
  for (int j = 0; j < XR; ++j) {
    const int q = threadIdx.x + j * NT;
    if (q < n4) xs4[q] = xr[j];
  }
#pragma unroll 4
  for (int q = threadIdx.x + XR * NT; q < n4; q += NT) xs4[q] = buf_loadf4(rx, x_off(q));
  __syncthreads();
  if (a.in_rms) {  // stack glue: x[t] /= sqrt(mean x[t]^2 + eps), in LDS
    __shared__ float part[TG][4];
    float *xs = reinterpret_cast<float *>(xs4);
#pragma unroll
    for (int t = 0; t < TG; ++t) {
      const float ss = rms_wave_part(xs + t * Hp4 * 4, H);
      if (lane == 0 && wave < 4) part[t][wave] = ss;
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < TG; ++t) {
      const float r = rms_divisor(part[t], H, a.in_eps);
      for (int i = threadIdx.x; i < H; i += NT) xs[t * Hp4 * 4 + i] /= r;
    }
    __syncthreads();
  }

  float acc[2][P][TG][2];
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
      for (int t = 0; t < TG; ++t) acc[g][p][t][0] = acc[g][p][t][1] = 0.0f;

  // The next DEPTH - 1 units' loads are in flight while a unit is computed.
  // DEPTH units per trip so that the register buffers keep static names.
  GuUnit u1 = gu_next<TG, P>(a, plan, u0, nc, NW, ntask, t0, gw);
#if DUCKMOE_GU_DEPTH == 3
  if (u1.task < ntask) gu_issue(b1, u1, a, lane);
  GuTile<P> b2;
  GuUnit u2;
  while (u0.task < ntask) {
    u2 = gu_next<TG, P>(a, plan, u1, nc, NW, ntask, t0, gw);
    if (u2.task < ntask) gu_issue(b2, u2, a, lane);
    gu_consume<TG, P>(b0, xs4, Hp4, u0.kc, lane, acc, u0.tm);
    if (u0.c == nc - 1) gu_finish<TG, P>(a, plan, u0.slot, u0.row0, t0, lane, acc);
    if (u1.task >= ntask) break;

    u0 = gu_next<TG, P>(a, plan, u2, nc, NW, ntask, t0, gw);
    if (u0.task < ntask) gu_issue(b0, u0, a, lane);
    gu_consume<TG, P>(b1, xs4, Hp4, u1.kc, lane, acc, u1.tm);
    if (u1.c == nc - 1) gu_finish<TG, P>(a, plan, u1.slot, u1.row0, t0, lane, acc);
    if (u2.task >= ntask) break;

    u1 = gu_next<TG, P>(a, plan, u0, nc, NW, ntask, t0, gw);
    if (u1.task < ntask) gu_issue(b1, u1, a, lane);
    gu_consume<TG, P>(b2, xs4, Hp4, u2.kc, lane, acc, u2.tm);
    if (u2.c == nc - 1) gu_finish<TG, P>(a, plan, u2.slot, u2.row0, t0, lane, acc);
  }
#else
  while (u0.task < ntask) {
    if (u1.task < ntask) gu_issue(b1, u1, a, lane);
    gu_consume<TG, P>(b0, xs4, Hp4, u0.kc, lane, acc, u0.tm);
    if (u0.c == nc - 1) gu_finish<TG, P>(a, plan, u0.slot, u0.row0, t0, lane, acc);
    if (u1.task >= ntask) break;

    u0 = gu_next<TG, P>(a, plan, u1, nc, NW, ntask, t0, gw);
    if (u0.task < ntask) gu_issue(b0, u0, a, lane);
    gu_consume<TG, P>(b1, xs4, Hp4, u1.kc, lane, acc, u1.tm);
    if (u1.c == nc - 1) gu_finish<TG, P>(a, plan, u1.slot, u1.row0, t0, lane, acc);
    u1 = gu_next<TG, P>(a, plan, u0, nc, NW, ntask, t0, gw);
  }
#endif
}

// Single-expert calls whose I / P tasks would leave more than half of the
// persistent grid idle (one expert of 2048 rows against 16 waves on each of
// 256 CUs): each task is split along the hidden dimension between the two
// waves of a pair in one workgroup.  Wave 2j of the grid takes the first
// ceil(nc / 2) 1024-wide chunks of task j, wave 2j + 1 the rest; a wave keeps
// up to three chunks' loads in flight.  The pair's row sums meet in LDS and
// are added in a fixed order (first half + second half) before SwiGLU, so the
// result does not depend on timing.  Needs 2 * (I / P) <= all waves.
template <int TG, int P, int WA>
__global__ __launch_bounds__(WA * 64) void k_gate_up_split(const LayerArgs a, const int t0) {
  extern __shared__ float4 xs4[];  // [TG][nc * 256], as in k_gate_up
  __shared__ float comb[WA / 2][2][P][TG];
  constexpr int NT = WA * 64;
  constexpr int XR = 8;
  const int H = a.H, H4 = a.H / 4;
  const int nc = (H + kChunk - 1) / kChunk;
  const int Hp4 = nc * (kChunk / 4);
  const int n4 = TG * Hp4;
  const int NB = a.I / P;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int gw = blockIdx.x * WA + wave;
  const int task = gw >> 1, half = gw & 1;
  const int cm = (nc + 1) / 2;
  const int c_lo = half ? cm : 0;
  const bool live = task < NB;
  const int n = live ? (half ? nc - cm : cm) : 0;  // chunks of this wave

  // x first, then the weights: the LDS staging waits for x only
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x + (size_t)t0 * H, (uint32_t)(TG * H) * 4u);
  auto x_off = [&](int q) -> uint32_t {
    const int t = q / Hp4, k4 = q - t * Hp4;
    return (q < n4 && k4 < H4) ? (uint32_t)(t * H4 + k4) * 16u : kOutOfRange;
  };
  float4 xr[XR];
#pragma unroll
  for (int j = 0; j < XR; ++j) xr[j] = buf_loadf4(rx, x_off(threadIdx.x + j * NT));

  const int e = a.single_expert;
  GuUnit u = gu_unit<P>(a, e, live ? task : 0, c_lo);
  auto unit = [&](int k) {  // chunk c_lo + k of the wave's task
    GuUnit v = u;
    v.c = c_lo + k;
    v.kc = (uint32_t)(c_lo + k) * kChunk;
    return v;
  };
  GuTile<P> b0, b1, b2;
  gu_issue(b0, unit(0), a, lane, 0 < n);
  gu_issue(b1, unit(1), a, lane, 1 < n);
  gu_issue(b2, unit(2), a, lane, 2 < n);

  if (blockIdx.x == 0 && wave == 0 && t0 == 0) plan_store(wave_plan(a, PlanIn{0, 0.0f}), a);
#pragma unroll
  for (int j = 0; j < XR; ++j) {
    const int q = threadIdx.x + j * NT;
    if (q < n4) xs4[q] = xr[j];
  }
  for (int q = threadIdx.x + XR * NT; q < n4; q += NT) xs4[q] = buf_loadf4(rx, x_off(q));
  __syncthreads();

  float acc[2][P][TG][2];
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
      for (int t = 0; t < TG; ++t) acc[g][p][t][0] = acc[g][p][t][1] = 0.0f;

  for (int k = 0; k < n; k += 3) {
    gu_consume<TG, P>(b0, xs4, Hp4, unit(k).kc, lane, acc, -1);
    gu_issue(b0, unit(k + 3), a, lane, k + 3 < n);
    if (k + 1 >= n) break;
    gu_consume<TG, P>(b1, xs4, Hp4, unit(k + 1).kc, lane, acc, -1);
    gu_issue(b1, unit(k + 4), a, lane, k + 4 < n);
    if (k + 2 >= n) break;
    gu_consume<TG, P>(b2, xs4, Hp4, unit(k + 2).kc, lane, acc, -1);
    gu_issue(b2, unit(k + 5), a, lane, k + 5 < n);
  }

  float gs[P][TG], vs[P][TG];
#pragma unroll
  for (int p = 0; p < P; ++p)
#pragma unroll
    for (int t = 0; t < TG; ++t) {
      gs[p][t] = wave_sum(acc[0][p][t][0] + acc[0][p][t][1]);
      vs[p][t] = wave_sum(acc[1][p][t][0] + acc[1][p][t][1]);
      if (half && lane == 0) {
        comb[wave >> 1][0][p][t] = gs[p][t];
        comb[wave >> 1][1][p][t] = vs[p][t];
      }
    }
  __syncthreads();
  if (half || !live || lane != 0) return;
#pragma unroll
  for (int p = 0; p < P; ++p)
#pragma unroll
    for (int t = 0; t < TG; ++t) {
      const float g = gs[p][t] + comb[wave >> 1][0][p][t];
      const float v = vs[p][t] + comb[wave >> 1][1][p][t];
      a.hbuf[(size_t)(t0 + t) * a.I + u.row0 + p] = silu(g) * v;
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
// Dynamic LDS: WB * R * T * 16 floats.
template <int G>
__device__ __forceinline__ void store_groups(float v, float *dst, int lane) {
  v = group_sum<G>(v);
  if ((lane & (G - 1)) == G - 1) dst[lane / G] = v;
}

// The sign words: at one token they stay 16-bit until the decode widens them,
// so the loop does not wait for the next item's loads right after issuing
// them (measured 0.4 us faster per bsz-1 layer); from two tokens on the early
// wait measured faster (0.9 us per bsz-2 layer), so they are widened at once.
template <int T>
using DnSign = typename std::conditional<T == 1, uint16_t, uint32_t>::type;

template <int T, int R>
struct DnTile {
  uint4 d[R];
  DnSign<T> s[R];
  float4 h[T][4];  // the item's activations h'[slot][t][k .. k+16)
  int tm;          // tokens naming the item's slot (bit t); the others' h' is 0
};

template <int T, int R>
__device__ __forceinline__ void dn_issue(DnTile<T, R> &b, const LayerArgs &a, int e,
                                         __amdgpu_buffer_rsrc_t rh, int slot, int row0,
                                         uint32_t k, bool kv, int tm) {
  const uint32_t H = a.H, I = a.I;
  const uint32_t mat = H * I;
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(a.dn_body + (size_t)e * mat, mat);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.dn_sign + (size_t)e * (mat / 8), mat / 8);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t row = row0 + r;
    const bool ok = kv && row < H;
    b.d[r] = buf_load16<kStream>(rb, ok ? row * I + k : kOutOfRange);
    b.s[r] = (DnSign<T>)buf_load2h<kStream>(rs, ok ? row * (I / 8) + k / 8 : kOutOfRange);
  }
  // h' rows of tokens that do not name the slot are zero: not read (the
  // out-of-range loads return zeros without touching memory)
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const bool tv = kv && (T == 1 || ((tm >> t) & 1));
    const uint32_t off = tv ? ((uint32_t)(slot * a.T + t) * I + k) * 4u : kOutOfRange;
#pragma unroll
    for (int j = 0; j < 4; ++j) b.h[t][j] = buf_loadf4(rh, off + 16 * j);
  }
  b.tm = tm;
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
  // a token that does not name the slot would add 0 * w = 0 (fp9 weights are
  // finite), so skipping it leaves every accumulator bit unchanged
#pragma unroll
  for (int r = 0; r < R; ++r) {
    h2_t h[8];
    fp9_decode16(b.d[r], b.s[r], h);
#pragma unroll
    for (int t = 0; t < T; ++t)
      if (T == 1 || ((b.tm >> t) & 1)) fma16(h, hv[t], acc[r][t][0], acc[r][t][1]);
  }
}

// The n_it items (slots s0, s0 + per_c, ...) of one block for one wave.  The
// first item is already in flight in b0; items alternate between b0 and b1,
// the next one always issued before the current one is computed.
// expert of slot s in the plan the gate/up launch left in the workspace
__device__ __forceinline__ int plan_at(const int32_t *plan, int s) {
  return __builtin_amdgcn_readfirstlane(plan[1 + s]);
}

// Item q of a block is (slot q / nc, chunk q % nc).  Wave w streams the items
// q = w, w + WB, ... < nq: the first is already in flight in b0; items
// alternate between b0 and b1, the next always issued before the current one
// is computed.  When WB is a multiple of nc every item of a wave has chunk
// w % nc (the shard combine relies on it).
template <int T, int R>
__device__ __forceinline__ void dn_item(DnTile<T, R> &b, const LayerArgs &a, const int32_t *plan,
                                        __amdgpu_buffer_rsrc_t rh, int q, int nc, int row0,
                                        int lane) {
  const int slot = q / nc;
  const uint32_t k = (uint32_t)(q - slot * nc) * kChunk + lane * 16;
  int tm = -1;
  if (T > 1)  // the slot's token mask, stored with the plan
    tm = __builtin_amdgcn_readfirstlane(
        plan[(int)((kMaskOff - kPlanOff) / sizeof(int32_t)) + slot]);
  dn_issue<T, R>(b, a, plan_at(plan, slot), rh, slot, row0, k, k < (uint32_t)a.I, tm);
}

template <int T, int R, int WB>
__device__ __forceinline__ void dn_block(DnTile<T, R> &b0, DnTile<T, R> &b1, const LayerArgs &a,
                                         const int32_t *plan, __amdgpu_buffer_rsrc_t rh,
                                         int blk, int w, int nq, int nc, int lane,
                                         float (&acc)[R][T][2]) {
  for (int q = w; q < nq; q += 2 * WB) {
    if (q + WB < nq) dn_item<T, R>(b1, a, plan, rh, q + WB, nc, blk * R, lane);
    dn_consume<T, R>(b0, acc);
    if (q + WB >= nq) break;
    if (q + 2 * WB < nq) dn_item<T, R>(b0, a, plan, rh, q + 2 * WB, nc, blk * R, lane);
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
  const int nblk = (H + R - 1) / R;
  // h' of every slot the workspace can hold; slots >= n_slots are never read
  const int max_slots = a.ids != nullptr ? a.T * a.top_k + 1 : 1;
  const __amdgpu_buffer_rsrc_t rh = make_rsrc(a.hbuf, (uint32_t)(max_slots * a.T * I) * 4u);
  const int ns = a.n_shards;
  const int width = I / ns;

  // A wave whose first item is in slot 0 (its expert is known without the
  // plan) issues it before the plan arrives.
  DnTile<T, R> b0, b1;
  const bool first_now = wave < nc && (int)blockIdx.x < nblk;
  if (first_now) {
    const uint32_t k = (uint32_t)wave * kChunk + lane * 16;
    dn_issue<T, R>(b0, a, slot0_expert(a), rh, 0, blockIdx.x * R, k, k < (uint32_t)I, -1);
  }
  const int nq = __builtin_amdgcn_readfirstlane(plan[0]) * nc;  // items per block
  if (!first_now && wave < nq && (int)blockIdx.x < nblk)
    dn_item<T, R>(b0, a, plan, rh, wave, nc, blockIdx.x * R, lane);

  for (int blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
    float acc[R][T][2];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int t = 0; t < T; ++t) acc[r][t][0] = acc[r][t][1] = 0.0f;

    if (wave < nq) {
      dn_block<T, R, WB>(b0, b1, a, plan, rh, blk, wave, nq, nc, lane, acc);
      // the next block's first item loads while this block is reduced
      if (blk + (int)gridDim.x < nblk)
        dn_item<T, R>(b0, a, plan, rh, wave, nc, (blk + gridDim.x) * R, lane);
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
      // with n_shards > 1, WB is a multiple of nc and wave w holds chunk w % nc
      float sum = 0.0f;
      for (int w = 0; w < WB; ++w) {
        const int cw = w % nc;
        if (ns == 1 || (cw >= c_lo && cw < c_hi)) sum += red[((w * R + r) * T + t) * 16 + grp];
      }
      a.out[((size_t)shard * T + t) * H + row] = sum;
    }
    __syncthreads();  // red is rewritten by the next block
  }
}

// -------------------------------------------------- matrix-core path ----
// For T >= 3 tokens the FMA count per weight (one per token) makes the vector
// kernels ALU-bound, so the contractions go to the matrix cores instead:
// v_mfma_f32_16x16x32_f16 takes a 16 x 32 fp16 A, a 32 x 16 fp16 B and an f32
// accumulator.  The fp9 weights decode exactly to fp16 (A).  The activations
// (B) are float32; each is split into two fp16 numbers, hi = fp16(v) and
// lo = fp16((v - hi) * 2^11), after scaling every token row (x) or (slot,
// token) row (h') by a power of two that puts its largest magnitude in
// [2^13, 2^14), so neither part overflows and the pair carries about 22 bits.
// With at most 8 tokens both parts fit one B operand: column j < 8 holds the hi
// part of token j and column 8 + j its lo part, so one MFMA per step gives
// both products, recombined in f32 as acc[j] + acc[8 + j] * 2^-11 and unscaled
// exactly.
//
// Lane layout (checked on gfx950): A[i][k] is in lane i + 16 * (k / 8), element
// k % 8; B[k][j] in lane j + 16 * (k / 8), element k % 8; the accumulator
// element D[i][j] in lane j + 16 * (i / 4), element i % 4.  The k index only has
// to agree between A and B.  Weights are loaded in whole 128-byte lines, 8
// lanes per row (lane 8r + q: 16-byte chunk q of rows r and r + 8 of the
// 128-column unit), with the non-temporal policy; ds_bpermute then gives lane
// i + 16g row i's chunks g and 4 + g, the MFMA's place for row i and lane
// group g (mfma_device.h).  So lane group g holds columns 16g .. 16g + 15
// (steps 0, 1) and 64 + 16g .. 64 + 16g + 15 (steps 2, 3), and the B loads
// follow the same columns.
constexpr int kMxGroups = 8;   // slot groups of the down pass (partials per row)
constexpr float kLoScale = 2048.0f;

// The hi/lo parts are stored as [column / 8][part][token][8] (part 0 hi, 1 lo):
// the 8 columns a lane takes for one MFMA step are 16 contiguous bytes, and the
// lanes of one lane group (hi of tokens 0 .. T-1, then their lo) read 16-byte
// pieces that are contiguous for T = 8.
static_assert(kMaxT <= 8, "hi and lo of every token share one 16-column B operand");
static_assert(kMaxIds + 1 <= 128, "the down pass keeps the slots' experts in two lane words");
struct MxArgs {
  _Float16 *xb;       // [Hp/8][2][T][8] scaled activations, hi and lo (zero padded)
  float *xinv;        // [T] 2^-k of each token's scale
  _Float16 *hb;       // [slots][Ip/8][2][T][8] scaled h'
  int8_t *hexp;       // [slots][T][EB] scale exponent of each 32-row block of h'
  float *part;        // [kMxGroups][T][H] down partials
  int Hp, Ip;         // H, I rounded up to whole units
  int EB;             // exponent bytes per (slot, token): 8 per unit pair
};

// h' is scaled per (slot, token, block of kHBlock rows of I), the rows one
// gate/up task owns, so each task's epilogue splits its own rows.  A block
// whose rows are all zero takes exponent kZeroExp, so that it never sets the
// common scale of a unit (below).
constexpr int kHBlock = 32;
constexpr int kZeroExp = 126;

__device__ __forceinline__ void mx_split(float v, _Float16 &hi, _Float16 &lo) {
  hi = (_Float16)v;
  lo = (_Float16)((v - (float)hi) * kLoScale);
}

// Split one token's row of n floats (optionally divided by r first) into scaled
// hi/lo parts of width np (zeros past n), stored as [np/8][2][T][8] at token t;
// returns 2^-k.  One workgroup of 256 threads.  Rows of up to 8192 floats are
// read once, into registers (all loads in flight together); longer rows are
// read twice.
constexpr int kPrepRegs = 8;  // float4s per thread held in registers

__device__ __forceinline__ void mx_prep_store(float4 v, float r, float sc, int i, _Float16 *dst,
                                              int T, int t) {
  const float e[4] = {v.x, v.y, v.z, v.w};
  _Float16 h[4], l[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) mx_split((e[q] / r) * sc, h[q], l[q]);
  typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
  const size_t o = ((size_t)(i >> 1) * 2 * T + t) * 8 + 4 * (i & 1);  // columns 4i .. 4i + 3
  *reinterpret_cast<h4_t *>(dst + o) = h4_t{h[0], h[1], h[2], h[3]};
  *reinterpret_cast<h4_t *>(dst + o + (size_t)T * 8) = h4_t{l[0], l[1], l[2], l[3]};
}

__device__ __forceinline__ float absmax4(float4 v, float r) {
  return fmaxf(fmaxf(fabsf(v.x / r), fabsf(v.y / r)), fmaxf(fabsf(v.z / r), fabsf(v.w / r)));
}

__device__ float mx_prep_row(const float *src, int n, int np, float r, _Float16 *dst, int T,
                             int t, float *red) {
  // n and np are multiples of 4 (of 16 and 128): float4 loads
  const float4 *s4 = reinterpret_cast<const float4 *>(src);
  const int n4 = n / 4, np4 = np / 4;
  const bool in_regs = np4 <= kPrepRegs * 256;
  float4 v[kPrepRegs];
  float m = 0.0f;
  if (in_regs) {
#pragma unroll
    for (int q = 0; q < kPrepRegs; ++q) {
      const int i = threadIdx.x + 256 * q;
      v[q] = i < n4 ? s4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int q = 0; q < kPrepRegs; ++q) m = fmaxf(m, absmax4(v[q], r));
  } else {
#pragma unroll 4
    for (int i = threadIdx.x; i < n4; i += 256) m = fmaxf(m, absmax4(s4[i], r));
  }
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  const int k = mx_scale_exp(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])));
  const float sc = ldexpf(1.0f, k);
  if (in_regs) {
#pragma unroll
    for (int q = 0; q < kPrepRegs; ++q) {
      const int i = threadIdx.x + 256 * q;
      if (i < np4) mx_prep_store(v[q], r, sc, i, dst, T, t);
    }
  } else {
#pragma unroll 4
    for (int i = threadIdx.x; i < np4; i += 256)
      mx_prep_store(i < n4 ? s4[i] : make_float4(0.f, 0.f, 0.f, 0.f), r, sc, i, dst, T, t);
  }
  return ldexpf(1.0f, -k);
}

// One workgroup per token: x (or its RMS-normalized form, the stack glue) ->
// scaled hi/lo parts.  The glue divides by the same divisor as k_rms.
__global__ __launch_bounds__(256) void k_mx_xprep(const LayerArgs a, const MxArgs m) {
  __shared__ float red[4];
  __shared__ float part[4];
  const int t = blockIdx.x;
  const float *row = a.x + (size_t)t * a.H;
  float r = 1.0f;
  if (a.in_rms) {
    const float ss = rms_wave_part(row, a.H);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
    __syncthreads();
    r = rms_divisor(part, a.H, a.in_eps);
  }
  const float inv = mx_prep_row(row, a.H, m.Hp, r, m.xb, a.T, t, red);
  if (threadIdx.x == 0) m.xinv[t] = inv;
}

// A stack's glue between two layers on the matrix-core path, in one launch:
// the previous layer's output row of token t (its kMxGroups down partials added
// in group order, as k_mx_reduce adds them) is normalized by its RMS and split
// as k_mx_xprep splits it.  The row is never written out; it sits in LDS so
// that the sum of squares runs in rms_wave_part's order, and the results are
// bit-identical to k_mx_reduce followed by k_mx_xprep.  One workgroup of 1024
// threads per token; rows of up to kChainMaxH floats.
constexpr int kChainMaxH = 8192;

__global__ __launch_bounds__(1024) void k_mx_reduce_xprep(const LayerArgs a, const MxArgs m) {
  __shared__ float4 row4[kChainMaxH / 4];
  __shared__ float part[4];
  __shared__ float red[16];
  const int t = blockIdx.x;
  const int n4 = a.H / 4, np4 = m.Hp / 4;
  const size_t plane4 = (size_t)a.T * n4;  // float4s of one group's [T][H] partials
  const float4 *p4 = reinterpret_cast<const float4 *>(m.part) + (size_t)t * n4;
  float4 v[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int i = threadIdx.x + 1024 * q;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i < n4) {
#pragma unroll
      for (int g = 0; g < kMxGroups; ++g) {
        const float4 p = p4[(size_t)g * plane4 + i];
        s.x += p.x;
        s.y += p.y;
        s.z += p.z;
        s.w += p.w;
      }
      row4[i] = s;
    }
    v[q] = s;
  }
  __syncthreads();
  const float ss = rms_wave_part(reinterpret_cast<const float *>(row4), a.H);
  if (threadIdx.x < 256 && (threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float r = rms_divisor(part, a.H, a.in_eps);
  float mx = fmaxf(absmax4(v[0], r), absmax4(v[1], r));
  mx = wave_max(mx);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  mx = red[0];
#pragma unroll
  for (int w = 1; w < 16; ++w) mx = fmaxf(mx, red[w]);
  const int k = mx_scale_exp(mx);
  const float sc = ldexpf(1.0f, k);
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int i = threadIdx.x + 1024 * q;
    if (i < np4) mx_prep_store(v[q], r, sc, i, m.xb, a.T, t);
  }
  if (threadIdx.x == 0) m.xinv[t] = ldexpf(1.0f, -k);
}

struct MxAct {      // the lane's 32 B values of one unit (hi or lo of one token)
  uint4 v[4];
};

// B for lane (column j, group g): part j / 8 of token j % 8, columns
// c0 + 16g + 8s (s = 0, 1) and c0 + 64 + 16g + 8(s - 2) (s = 2, 3), from a
// [cols/8][2][T][8] block at byte base; zeros for tokens at or past T, for
// columns at or past ncol (CLIP), and everywhere when live is false (the
// loads are issued either way).
template <bool CLIP>
__device__ __forceinline__ void mx_load_b(MxAct &b, __amdgpu_buffer_rsrc_t r, uint32_t base,
                                          uint32_t c0, int T, bool live, uint32_t ncol) {
  const int j = threadIdx.x & 15, g = (threadIdx.x & 63) >> 4;
  const uint32_t row = (uint32_t)(j >> 3) * (uint32_t)T + (uint32_t)(j & 7);
  const bool v = live && (j & 7) < T;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const uint32_t kb = (c0 + 16 * g) / 8 + (s & 1) + 8 * (s >> 1);
    const uint32_t o = base + (kb * 2u * (uint32_t)T + row) * 16u;
    b.v[s] = buf_load16(r, v && (!CLIP || kb * 8u < ncol) ? o : kOutOfRange);
  }
}

// acc += A * B over the unit's 4 steps (columns j: hi of token j, 8 + j: its lo)
__device__ __forceinline__ void mx_mma_frag(const MxFrag &w, const MxAct &b, f4v_t &acc) {
  h2_t d[16];
  fp9_decode16(w.b0, w.s0, d);
  fp9_decode16(w.b1, w.s1, d + 8);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const half8_t A = __builtin_bit_cast(half8_t, make_uint4(
        __builtin_bit_cast(uint32_t, d[4 * s]), __builtin_bit_cast(uint32_t, d[4 * s + 1]),
        __builtin_bit_cast(uint32_t, d[4 * s + 2]), __builtin_bit_cast(uint32_t, d[4 * s + 3])));
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, __builtin_bit_cast(half8_t, b.v[s]), acc, 0, 0, 0);
  }
}

// A wave's work in the two matrix-core kernels is one flat stream of items:
// for each task of its workgroup (in order), the unit pairs p = wave,
// wave + WA, ... of the task (units 2p and 2p + 1, the second one empty past
// the task's last unit), or one empty pair (p = -1) when the wave has no pair
// in it, so that every wave closes every task exactly once (the close has a
// barrier).  A pair is two items, one per unit; the sign words of both units
// come with the first item's loads (mx_load_signs) and are kept in one of two
// alternating register sets.  The loads of the next item, possibly in the
// next task, are issued before the current one is computed.  Every item
// issues the same loads, an empty item or one past the last task with
// out-of-range offsets (they read zeros and touch no memory): with a branch
// around them the compiler could not know how many loads are in flight behind
// the current item's, and its waits would drain the next item's loads as well.
struct MxItem {
  int task;
  int u;  // pair index, -1 for the empty pair
};


// Gate/up: a workgroup of WA waves takes whole tasks (slot, block of 16 * RT
// rows) and splits the task's unit pairs (256 columns of H) over its waves; the
// waves' partial accumulators meet in LDS, wave 0 sums them in a fixed order and
// writes h' = w * silu(gate) * up for the block's rows and every token.
template <int RT>
struct GuMxBuf {
  MxBody g[RT], u[RT];
  MxAct b;
};

template <int RT>
struct GuMxSigns {
  MxSigns g[RT], u[RT];
};

template <int WA, int RT, int SM>
__global__ __launch_bounds__(WA * 64) void k_gate_up_mx(const LayerArgs a, const MxArgs m) {
  static_assert(16 * RT == kHBlock, "a gate/up task owns one scale block of h' rows");
  __shared__ f4v_t red[2][WA][RT * 2][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int H = a.H, I = a.I, T = a.T;
  const int nu = m.Hp / kMxUnit;
  const int np = (nu + 1) / 2;
  const int NB = (I + 16 * RT - 1) / (16 * RT);  // row blocks per slot (last may be partial)
  const PlanIn pin = plan_load(a);
  const WavePlan plan = wave_plan(a, pin);
  if (blockIdx.x == 0 && wave == 0) plan_store(plan, a);
  const int ntask = plan.n_slots * NB;
  // tasks blockIdx.x, blockIdx.x + gridDim.x, ...
  auto first = [&]() { return MxItem{(int)blockIdx.x, wave < np ? wave : -1}; };
  auto next = [&](MxItem it) {
    if (it.u >= 0 && it.u + WA < np) return MxItem{it.task, it.u + WA};
    return MxItem{it.task + (int)gridDim.x, wave < np ? wave : -1};
  };
  const int j = lane & 15, g = lane >> 4;
  const uint32_t mat = (uint32_t)I * (uint32_t)H;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(m.xb, (uint32_t)(2 * T * m.Hp) * 2u);
  const bool jv = j < T;  // lanes that finish token j (j < 8)
  // token j's unscale factor, loaded once: a load in the task epilogue would
  // wait for every load issued before it, the next item's included
  float xs = __builtin_bit_cast(float, buf_load4(make_rsrc(m.xinv, (uint32_t)T * 4u),
                                                 jv ? (uint32_t)j * 4u : kOutOfRange));

  // unit 2p + half of the item's pair; the first half also loads both units' signs
  auto issue = [&](GuMxBuf<RT> &bf, GuMxSigns<RT> &sg, MxItem it, int half) {
    const bool live = it.u >= 0 && it.task < ntask && 2 * it.u + half < nu;
    const int task = live ? it.task : 0, u = live ? 2 * it.u : 0;
    const int slot = task / NB, r0 = (task - slot * NB) * 16 * RT;
    const int e = plan_expert(plan, slot);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(a.gu_body + (size_t)e * 2 * mat, 2 * mat);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.gu_sign + (size_t)e * 2 * (mat / 8), 2 * (mat / 8));
    const uint32_t c0 = (uint32_t)(u * kMxUnit);
    const uint32_t ch = c0 + (uint32_t)(half * kMxUnit);
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const int row = r0 + 16 * t + (lane >> 2);
      const bool rv = live && row < I;
      mx_load_body_ln<kStream>(bf.g[t], rb, 0u, r0 + 16 * t, I, H, ch, live);
      mx_load_body_ln<kStream>(bf.u[t], rb, (uint32_t)I, r0 + 16 * t, I, H, ch, live);
      if (half == 0) {
        mx_load_signs<SM>(sg.g[t], rs, (uint32_t)row, H, c0, rv);
        mx_load_signs<SM>(sg.u[t], rs, (uint32_t)(I + row), H, c0, rv);
      }
    }
    mx_load_b<false>(bf.b, rx, 0u, ch, T, live, 0u);
  };

  f4v_t acc[RT][2];  // gate, up
  auto zero = [&]() {
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int f = 0; f < 2; ++f) acc[t][f] = f4v_t{0, 0, 0, 0};
  };
  zero();
  int parity = 0;

  // An empty item's tiles are zeros and add nothing; computing them anyway
  // consumes every load, so no register of the item is still being written
  // when the next issue reuses it.  The second half closes the task.
  auto consume0 = [&](const GuMxBuf<RT> &bf, const GuMxSigns<RT> &sg) {
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      mx_mma_frag(mx_to_mfma_pair<SM, 0>(bf.g[t], sg.g[t]), bf.b, acc[t][0]);
      mx_mma_frag(mx_to_mfma_pair<SM, 0>(bf.u[t], sg.u[t]), bf.b, acc[t][1]);
    }
  };
  auto consume1 = [&](const GuMxBuf<RT> &bf, const GuMxSigns<RT> &sg, MxItem it) {
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      mx_mma_frag(mx_to_mfma_pair<SM, 1>(bf.g[t], sg.g[t]), bf.b, acc[t][0]);
      mx_mma_frag(mx_to_mfma_pair<SM, 1>(bf.u[t], sg.u[t]), bf.b, acc[t][1]);
    }
    if (it.task >= ntask || (it.u >= 0 && it.u + WA < np)) return;
    // close the task: partials to LDS, wave 0 reduces them and writes the
    // block's h' as scaled hi/lo parts with the block's exponent per token (lane
    // j < 8 adds the hi sums of its own column and the lo sums of column 8 + j;
    // lanes j + 16g, g < 4, hold token j's 32 rows)
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int f = 0; f < 2; ++f) red[parity][wave][2 * t + f][lane] = acc[t][f];
    zero();
    __syncthreads();
    if (wave == 0) {
      const int slot = it.task / NB, r0 = (it.task - slot * NB) * 16 * RT;
      float wt = 0.0f;
      for (int t = 0; t < T; ++t) {
        const float w_t = plan_weight(plan, a, slot, t);
        if (t == j) wt = w_t;
      }
      float hv[RT][4];
      float mx = 0.0f;
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        f4v_t G = {0, 0, 0, 0}, Gl = G, U = G, Ul = G;
        if (jv) {
#pragma unroll
          for (int w = 0; w < WA; ++w) {
            G += red[parity][w][2 * t + 0][lane];
            Gl += red[parity][w][2 * t + 0][lane + 8];
            U += red[parity][w][2 * t + 1][lane];
            Ul += red[parity][w][2 * t + 1][lane + 8];
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = r0 + 16 * t + 4 * g + r;
          const float gs = (G[r] + Gl[r] * (1.0f / kLoScale)) * xs;
          const float us = (U[r] + Ul[r] * (1.0f / kLoScale)) * xs;
          hv[t][r] = (!jv || wt == 0.0f || row >= I) ? 0.0f : wt * (silu(gs) * us);
          mx = fmaxf(mx, fabsf(hv[t][r]));
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const int k = mx > 0.0f ? mx_scale_exp(mx) : kZeroExp;
      if (jv) {
        const float sc = ldexpf(1.0f, k);
        _Float16 *dst = m.hb + (size_t)slot * 2 * T * m.Ip;
#pragma unroll
        for (int t = 0; t < RT; ++t)
          mx_prep_store(make_float4(hv[t][0], hv[t][1], hv[t][2], hv[t][3]), 1.0f, sc,
                        (r0 + 16 * t + 4 * g) / 4, dst, T, j);
        int8_t *ex = m.hexp + ((size_t)slot * T + j) * m.EB;
        if (g == 0) ex[r0 / kHBlock] = (int8_t)k;
        // blocks past the last one (to the end of the unit pair) hold no rows:
        // the all-zero exponent keeps them out of their unit's common scale
        if (r0 / kHBlock == NB - 1)
          for (int q = NB + g; q < m.EB; q += 4) ex[q] = (int8_t)kZeroExp;
      }
    }
    parity ^= 1;
  };

  GuMxBuf<RT> b0, b1;
  GuMxSigns<RT> s0, s1;
  MxItem p0 = first(), p1;
  issue(b0, s0, p0, 0);
  asm volatile("" : "+v"(xs));  // xs arrives here, the first item stays in flight
  // Two pairs per trip; the second may lie past the last task (zeros, no
  // close).  No exit inside a trip: a path that leaves with one buffer's loads
  // unconsumed would make the compiler's waits at the loop head assume those
  // loads may still be writing their registers.
  while (p0.task < ntask) {
    issue(b1, s0, p0, 1);
    consume0(b0, s0);
    p1 = next(p0);
    issue(b0, s1, p1, 0);
    consume1(b1, s0, p0);
    issue(b1, s1, p1, 1);
    consume0(b0, s1);
    p0 = next(p1);
    issue(b0, s0, p0, 0);
    consume1(b1, s1, p1);
  }
}

// Down: a workgroup takes tasks (block of 16 * RT rows of H, slot group q) and
// splits the (slot, unit pair of I) items of the group's slots over its waves;
// each unit's B values are first brought to the unit's common scale
// (mx_unit_rescale), and its accumulator is unscaled into the wave's running
// sum (column j by that scale, column 8 + j by it times 2^-11); the waves' sums
// meet in LDS and wave 0 writes the group's partial for the block's rows,
// adding columns j and 8 + j.  The groups' partials are added by k_mx_reduce in
// a fixed order.
template <int RT>
struct DnMxBuf {
  MxBody w[RT];
  MxAct b;
};

template <int RT>
struct DnMxSigns {
  MxSigns w[RT];
  uint2 ex;  // exponents of the 8 h' blocks of the pair's two units, the lane's token
};

// 2^-d (d >= 0) as two fp16 halves: normal to d = 14, subnormal to 24, then 0.
__device__ __forceinline__ uint32_t pow2neg_h2(int d) {
  const uint32_t h = d <= 14 ? (uint32_t)(15 - d) << 10 : (d <= 24 ? 1u << (24 - d) : 0u);
  return h | (h << 16);
}

__device__ __forceinline__ uint4 mul_h2(uint4 v, uint32_t f) {
  typedef _Float16 h2v __attribute__((ext_vector_type(2)));
  const h2v m = __builtin_bit_cast(h2v, f);
  return make_uint4(__builtin_bit_cast(uint32_t, __builtin_bit_cast(h2v, v.x) * m),
                    __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2v, v.y) * m),
                    __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2v, v.z) * m),
                    __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2v, v.w) * m));
}

// One unit of h' as B: its 4 blocks were scaled by 2^e0 .. 2^e3 (signed bytes
// of ew); lane group g's steps 0, 1 hold block g / 2 and steps 2, 3 block
// 2 + g / 2.  Each value is brought to the unit's common scale 2^ku, ku the
// smallest exponent (the block with the largest magnitude), by an exact
// power-of-two step, and 2^-ku is returned to unscale the unit's products.
__device__ __forceinline__ float mx_unit_rescale(MxAct &b, uint32_t ew, int g) {
  const int e0 = (int8_t)(ew & 0xff), e1 = (int8_t)((ew >> 8) & 0xff);
  const int e2 = (int8_t)((ew >> 16) & 0xff), e3 = (int8_t)(ew >> 24);
  const int ku = min(min(e0, e1), min(e2, e3));
  const uint32_t fa = pow2neg_h2(((g >> 1) ? e1 : e0) - ku);
  const uint32_t fb = pow2neg_h2(((g >> 1) ? e3 : e2) - ku);
  b.v[0] = mul_h2(b.v[0], fa);
  b.v[1] = mul_h2(b.v[1], fa);
  b.v[2] = mul_h2(b.v[2], fb);
  b.v[3] = mul_h2(b.v[3], fb);
  return ldexpf(1.0f, -max(-126, min(126, ku)));
}

template <int WA, int RT, int SM, int WPE>
__global__ __launch_bounds__(WA * 64) __attribute__((amdgpu_waves_per_eu(WPE)))
void k_down_mx(const LayerArgs a, const MxArgs m) {
  __shared__ f4v_t red[2][WA][RT][64];
  const int32_t *plan = reinterpret_cast<const int32_t *>(
      reinterpret_cast<const uint8_t *>(a.hdr) + kPlanOff);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int H = a.H, I = a.I, T = a.T;
  const int S = __builtin_amdgcn_readfirstlane(plan[0]);
  // lane l holds the expert of slot l (slots past 64 from a second word): a
  // load per item would be a wait for every load in flight before it
  const int eslot_lo = plan[1 + lane];
  const int eslot_hi = plan[1 + min(64 + lane, kMaxIds)];
  const int nv = m.Ip / kMxUnit;
  const int npv = (nv + 1) / 2;  // unit pairs per slot
  const int NBH = (H + 16 * RT - 1) / (16 * RT);
  const int ntask = NBH * kMxGroups;
  const int j = lane & 15, g = lane >> 4;
  const bool jv = j < T;             // lanes that finish token j (j < 8)
  const bool bv = (j & 7) < T;       // lanes whose column holds a token's part
  const float part_scale = j < 8 ? 1.0f : 1.0f / kLoScale;
  const uint32_t mat = (uint32_t)I * (uint32_t)H;
  const int max_slots = a.ids != nullptr ? T * a.top_k + 1 : 1;
  const __amdgpu_buffer_rsrc_t rh = make_rsrc(m.hb, (uint32_t)(max_slots * 2 * T * m.Ip) * 2u);
  const __amdgpu_buffer_rsrc_t rex = make_rsrc(m.hexp, (uint32_t)(max_slots * T * m.EB));
  // pairs of the task's group: (slot q + s * G, unit pair vp) for s < ns_q, vp < npv
  auto n_pairs = [&](int task) {
    const int q = task / NBH;
    return (S > q ? (S - q + kMxGroups - 1) / kMxGroups : 0) * npv;
  };
  // the stream of pairs as in k_gate_up_mx, with a per-task pair count
  auto first = [&]() {
    const int t = blockIdx.x;
    return MxItem{t, (t < ntask && wave < n_pairs(t)) ? wave : -1};
  };
  auto next = [&](MxItem it) {
    if (it.u >= 0 && it.u + WA < n_pairs(it.task)) return MxItem{it.task, it.u + WA};
    const int t = it.task + (int)gridDim.x;
    return MxItem{t, (t < ntask && wave < n_pairs(t)) ? wave : -1};
  };

  auto issue = [&](DnMxBuf<RT> &bf, DnMxSigns<RT> &sg, MxItem it, int half) {
    const bool pl = it.u >= 0 && it.task < ntask;
    const int task = pl ? it.task : 0, p = pl ? it.u : 0;
    const int q = task / NBH, blk = task - q * NBH;
    const int si = p / npv, vp = p - si * npv;
    const bool live = pl && 2 * vp + half < nv;
    const int slot = pl ? q + si * kMxGroups : 0;
    const int e = slot < 64 ? __builtin_amdgcn_readlane(eslot_lo, slot)
                            : __builtin_amdgcn_readlane(eslot_hi, slot - 64);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(a.dn_body + (size_t)e * mat, mat);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.dn_sign + (size_t)e * (mat / 8), mat / 8);
    const uint32_t c0 = (uint32_t)(2 * vp * kMxUnit);
    const uint32_t ch = c0 + (uint32_t)(half * kMxUnit);
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const int row = blk * 16 * RT + 16 * t + (lane >> 2);
      mx_load_body_ln<kStream>(bf.w[t], rb, 0u, blk * 16 * RT + 16 * t, H, I, ch, live);
      if (half == 0) mx_load_signs<SM>(sg.w[t], rs, (uint32_t)row, I, c0, pl && row < H);
    }
    mx_load_b<true>(bf.b, rh, (uint32_t)(slot * 2 * T * m.Ip) * 2u, ch, T, live, (uint32_t)I);
    if (half == 0)
      sg.ex = buf_load8(rex, pl && bv ? (uint32_t)((slot * T + (j & 7)) * m.EB + 8 * vp)
                                      : kOutOfRange);
  };

  f4v_t acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) acc[t] = f4v_t{0, 0, 0, 0};
  int parity = 0;

  auto consume0 = [&](const DnMxBuf<RT> &bf, const DnMxSigns<RT> &sg) {  // empty items add zeros
    MxAct b = bf.b;
    const float hs = mx_unit_rescale(b, sg.ex.x, g) * part_scale;
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      f4v_t d = {0, 0, 0, 0};
      mx_mma_frag(mx_to_mfma_pair<SM, 0>(bf.w[t], sg.w[t]), b, d);
      acc[t] += d * hs;
    }
  };
  auto consume1 = [&](const DnMxBuf<RT> &bf, const DnMxSigns<RT> &sg, MxItem it) {
    MxAct b = bf.b;
    const float hs = mx_unit_rescale(b, sg.ex.y, g) * part_scale;
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      f4v_t d = {0, 0, 0, 0};
      mx_mma_frag(mx_to_mfma_pair<SM, 1>(bf.w[t], sg.w[t]), b, d);
      acc[t] += d * hs;
    }
    if (it.task >= ntask || (it.u >= 0 && it.u + WA < n_pairs(it.task))) return;
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      red[parity][wave][t][lane] = acc[t];
      acc[t] = f4v_t{0, 0, 0, 0};
    }
    __syncthreads();
    if (wave == 0 && jv) {
      const int q = it.task / NBH, blk = it.task - q * NBH;
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        f4v_t sum = {0, 0, 0, 0}, lo = sum;
#pragma unroll
        for (int w = 0; w < WA; ++w) {
          sum += red[parity][w][t][lane];
          lo += red[parity][w][t][lane + 8];
        }
        sum += lo;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int orow = blk * 16 * RT + 16 * t + 4 * g + r;
          if (orow < H) m.part[((size_t)q * T + j) * H + orow] = sum[r];
        }
      }
    }
    parity ^= 1;
  };

  DnMxBuf<RT> b0, b1;
  DnMxSigns<RT> s0, s1;
  MxItem p0 = first(), p1;
  issue(b0, s0, p0, 0);
  while (p0.task < ntask) {  // two pairs per trip, as in k_gate_up_mx
    issue(b1, s0, p0, 1);
    consume0(b0, s0);
    p1 = next(p0);
    issue(b0, s1, p1, 0);
    consume1(b1, s0, p0);
    issue(b1, s1, p1, 1);
    consume0(b0, s1);
    p0 = next(p1);
    issue(b0, s0, p0, 0);
    consume1(b1, s1, p1);
  }
}

// out[t][row] = the kMxGroups partials added in group order.
__global__ __launch_bounds__(256) void k_mx_reduce(const LayerArgs a, const MxArgs m) {
  const int n = a.T * a.H;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = 0.0f;
#pragma unroll
  for (int q = 0; q < kMxGroups; ++q) s += m.part[(size_t)q * n + i];
  a.out[i] = s;
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
  const WavePlan p = wave_plan(a, plan_load(a));
  const int lane = threadIdx.x;
  if (lane == 0) {
    uniq[0] = p.e0;
    *n_slots = p.n_slots;
  }
  if (lane < p.n_slots - 1) uniq[1 + lane] = p.expert;
}

// y[t] = x[t] / sqrt(mean_i x[t][i]^2 + eps): one workgroup of 256 threads per
// token, sum of squares in f32 in the order of rms_wave_part; every element is
// read before any is written, so y may be x.
__global__ __launch_bounds__(256) void k_rms(const float *x, int H, float eps, float *y) {
  __shared__ float part[4];
  const float *xr = x + (size_t)blockIdx.x * H;
  float *yr = y + (size_t)blockIdx.x * H;
  const float ss = rms_wave_part(xr, H);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float r = rms_divisor(part, H, eps);
  for (int i = threadIdx.x; i < H; i += 256) yr[i] = xr[i] / r;
}

// Calibration: a plain streaming read of n1k blocks of 1 KB.  Wave w of the
// grid reads a contiguous slab of blocks with 8 loads in flight (non-temporal,
// the policy of the weight streams) and folds the words into a value that is
// stored only if it matches a constant it never matches, so the loads cannot
// be dropped.  This is the ceiling a pure weight stream reaches on the device,
// the reference the layer kernels are held to.
__global__ __launch_bounds__(512) void k_read_probe(const uint4 *__restrict__ p, uint32_t n1k,
                                                   uint32_t *sink) {
  typedef uint32_t u4v __attribute__((ext_vector_type(4)));
  const uint32_t nw = gridDim.x * (blockDim.x / 64);
  const uint32_t w = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t per = (n1k + nw - 1) / nw;
  const uint32_t b0 = min(n1k, w * per), b1 = min(n1k, b0 + per);
  const u4v *q = reinterpret_cast<const u4v *>(p);
  uint32_t acc = 0;
  for (uint32_t b = b0; b < b1; b += 8) {
    u4v v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      v[u] = u4v{0u, 0u, 0u, 0u};
      if (b + u < b1) v[u] = __builtin_nontemporal_load(q + (size_t)(b + u) * 64 + lane);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

// ------------------------------------------------------------ host side ----

constexpr size_t kGuXLds = 131072;  // LDS bytes for the activations of one gate/up pass

// tokens the gate/up kernel takes per pass for a given hidden size (0: too wide)
int gu_tokens_per_pass(int H) {
  const size_t hp = (size_t)((H + kChunk - 1) / kChunk) * kChunk;
  return (int)std::min<size_t>(kGuTokens, kGuXLds / (hp * sizeof(float)));
}



int check_layer(const duckmoe_layer *L) {
  if (!L || !L->gu_body || !L->gu_sign || !L->dn_body || !L->dn_sign) return DUCKMOE_EINVAL;
  if (L->hidden < 16 || L->hidden % 16 || L->inter < 16 || L->inter % 16 ||
      L->inter > kMaxInter || L->top_k < 1 || L->n_routed < 0 ||
      L->n_routed > DUCKMOE_MAX_ROUTED)
    return DUCKMOE_ESHAPE;
  // one buffer descriptor spans an expert's gate+up bodies: 2*H*I < 2^31
  if (2ll * L->hidden * L->inter > 0x7fffffffll) return DUCKMOE_ESHAPE;
  if (gu_tokens_per_pass(L->hidden) < 1) return DUCKMOE_ESHAPE;
  if (!aligned(L->gu_body, 16) || !aligned(L->dn_body, 16) || !aligned(L->gu_sign, 2) ||
      !aligned(L->dn_sign, 2))
    return DUCKMOE_EINVAL;
  return DUCKMOE_OK;
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

int check_shards(int I, int ns) {
  if (ns < 1 || I % ns) return DUCKMOE_ESHAPE;
  if (ns == 1) return DUCKMOE_OK;
  // shard partials need every down wave on one 1024-wide chunk
  const int nc = (I + kChunk - 1) / kChunk;
  if (kWB % nc) return DUCKMOE_ESHAPE;
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

// Matrix-core path (T >= kMxMinT, no shard partials): launch shape and the
// workspace it adds after h'.
#ifndef DUCKMOE_MX_MIN_T
#define DUCKMOE_MX_MIN_T 3          // smallest T that takes the matrix-core path
#endif
#ifndef DUCKMOE_MX_GU_WAVES
#define DUCKMOE_MX_GU_WAVES 4       // waves per gate/up workgroup
#endif
#ifndef DUCKMOE_MX_DN_WAVES
#define DUCKMOE_MX_DN_WAVES 4       // waves per down workgroup
#endif
#ifndef DUCKMOE_MX_GU_ROW_TILES
#define DUCKMOE_MX_GU_ROW_TILES 2   // 16-row MFMA tiles per gate/up task (they share B loads)
#endif
// Down task shapes: 16-row MFMA tiles per task (they share the B loads) and
// the waves per SIMD the registers must allow.  Below DUCKMOE_MX_DN_WIDE_T
// tokens 2 tiles at 4 waves; from it on 3 tiles at 3 waves (150 registers; 3
// tiles at 4 waves spill), which measured 0.4-1% faster at 6-8 tokens and
// the same at 5.
#ifndef DUCKMOE_MX_DN_WIDE_T
#define DUCKMOE_MX_DN_WIDE_T 6
#endif
#ifndef DUCKMOE_MX_WAVES_PER_CU
#define DUCKMOE_MX_WAVES_PER_CU 16  // target resident waves per CU (capped by occupancy)
#endif

bool use_mx(int T, int n_shards) { return T >= DUCKMOE_MX_MIN_T && n_shards == 1; }

size_t align256(size_t n) { return (n + 255) / 256 * 256; }

struct MxLayout {
  size_t xb, xinv, hb, hexp, part, end;
  int Hp, Ip, EB;
};

MxLayout mx_layout(const duckmoe_layer *L, int T, bool single, size_t base) {
  MxLayout m;
  m.Hp = (L->hidden + kMxUnit - 1) / kMxUnit * kMxUnit;
  m.Ip = (L->inter + kMxUnit - 1) / kMxUnit * kMxUnit;
  const size_t slots = hbuf_slots(L, T, single);
  size_t off = align256(base);
  m.xb = off;   off = align256(off + (size_t)2 * T * m.Hp * 2);
  m.xinv = off; off = align256(off + (size_t)T * 4);
  m.EB = (m.Ip / kMxUnit + 1) / 2 * 8;
  m.hb = off;   off = align256(off + slots * 2 * T * m.Ip * 2);
  m.hexp = off; off = align256(off + slots * T * m.EB);
  m.part = off; off = align256(off + (size_t)kMxGroups * T * L->hidden * 4);
  m.end = off;
  return m;
}

// header | h' [slots][T][I] | (T >= kMxMinT) matrix-core buffers
size_t ws_need(const duckmoe_layer *L, int T, bool single) {
  const size_t base = kHdrBytes + hbuf_bytes(L, T, single);
  return T >= DUCKMOE_MX_MIN_T ? mx_layout(L, T, single, base).end : base;
}

// rows per down block: more rows share each h' load, fewer give more blocks (waves
// in flight) and keep registers in check; 7 measured best at bsz 1 and 2
// (1024 blocks of the 7168 output rows)
template <int T>
constexpr int down_rows() {
  return T <= 4 ? DUCKMOE_DN_ROWS : 2;
}

template <int TG>
hipError_t launch_gate_up_t(const LayerArgs &a, int t0, hipStream_t st) {
  constexpr int P = DUCKMOE_GU_PAIRS, WA = DUCKMOE_GU_WAVES;
  const auto kern = k_gate_up<TG, P, WA>;
  const size_t hp = (size_t)((a.H + kChunk - 1) / kChunk) * kChunk;
  const size_t lds = (size_t)TG * hp * sizeof(float);
  static OccCache occ;
  int per_cu = 0;
  hipError_t err = occupancy(occ, kern, WA * 64, lds, kGuXLds, per_cu);
  if (err != hipSuccess) return err;
  const int cus = cu_budget(a.cus);
  if (cus <= 0) return hipErrorInvalidConfiguration;
  per_cu = std::max(1, std::min(per_cu, DUCKMOE_GU_WAVES_PER_CU / WA));
  const int grid = cus * per_cu;
  if (a.ids == nullptr && !a.in_rms && 2 * (a.I / P) <= grid * WA) {
    // one expert: tasks split between wave pairs (same launch shape and LDS)
    const auto split = k_gate_up_split<TG, P, WA>;
    static OccCache occ_split;
    int per_cu_split = 0;
    err = occupancy(occ_split, split, WA * 64, lds, kGuXLds, per_cu_split);
    if (err != hipSuccess) return err;
    const int grid_split = cus * std::max(1, std::min(per_cu_split, DUCKMOE_GU_WAVES_PER_CU / WA));
    if (2 * (a.I / P) <= grid_split * WA) {
      hipLaunchKernelGGL(split, dim3(grid_split), dim3(WA * 64), lds, st, a, t0);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL(kern, dim3(grid), dim3(WA * 64), lds, st, a, t0);
  return hipGetLastError();
}

#ifndef DUCKMOE_DN_ROWS_SINGLE
#define DUCKMOE_DN_ROWS_SINGLE 4
#endif
template <int T, int R>
hipError_t launch_down_tr(const LayerArgs &a, hipStream_t st) {
  const auto kern = k_down<T, R, kWB>;
  const size_t lds = (size_t)kWB * R * T * 16 * sizeof(float);
  static OccCache occ;
  int per_cu = 0;
  hipError_t err = occupancy(occ, kern, kWB * 64, lds, 0, per_cu);
  if (err != hipSuccess) return err;
  const int cus = cu_budget(a.cus);
  if (cus <= 0) return hipErrorInvalidConfiguration;
  per_cu = std::max(1, std::min(per_cu, DUCKMOE_DN_WAVES_PER_CU / kWB));
  const int nblk = (a.H + R - 1) / R;
  const int grid = std::min(nblk, cus * per_cu);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kWB * 64), lds, st, a,
                     group_width(a.I, a.n_shards));
  return hipGetLastError();
}

// One slot of at most two 1024-wide chunks (a single expert of the DeepSeek-V3
// shape) gives a block of down_rows<1>() rows only two items, one per wave,
// and the grid then holds half the resident waves: such calls take smaller
// blocks.
template <int T>
hipError_t launch_down_t(const LayerArgs &a, hipStream_t st) {
  if constexpr (T == 1) {
    if (a.ids == nullptr && a.I <= 2 * kChunk)
      return launch_down_tr<1, DUCKMOE_DN_ROWS_SINGLE>(a, st);
  }
  return launch_down_tr<T, down_rows<T>()>(a, st);
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

template <int SM>
hipError_t launch_mx_gate_up_sm(const LayerArgs &a, const MxArgs &m, hipStream_t st) {
  constexpr int WA = DUCKMOE_MX_GU_WAVES, RT = DUCKMOE_MX_GU_ROW_TILES;
  const auto kern = k_gate_up_mx<WA, RT, SM>;
  const int max_slots = a.ids != nullptr ? a.T * a.top_k + 1 : 1;
  static OccCache occ;
  int grid = 0;
  hipError_t err = persistent_grid(occ, kern, WA * 64, DUCKMOE_MX_WAVES_PER_CU,
                                   max_slots * ((a.I + 16 * RT - 1) / (16 * RT)), a.cus, grid);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(WA * 64), 0, st, a, m);
  return hipSuccess;
}

// chain_in: x is the previous layer's output, still as its down partials in
// the same workspace (a stack's layers l > 0, H <= kChainMaxH, in_rms set).
hipError_t launch_mx_gate_up(const LayerArgs &a, const MxArgs &m, hipStream_t st, bool chain_in) {
  if (chain_in)
    hipLaunchKernelGGL(k_mx_reduce_xprep, dim3(a.T), dim3(1024), 0, st, a, m);
  else
    hipLaunchKernelGGL(k_mx_xprep, dim3(a.T), dim3(256), 0, st, a, m);
  const int sm = mx_sign_mode(a.H, a.gu_sign);
  const hipError_t err = sm == 2   ? launch_mx_gate_up_sm<2>(a, m, st)
                         : sm == 1 ? launch_mx_gate_up_sm<1>(a, m, st)
                                   : launch_mx_gate_up_sm<0>(a, m, st);
  if (err != hipSuccess) return err;
  return hipGetLastError();
}

template <int SM, int RT, int WPE>
hipError_t launch_mx_down_shape(const LayerArgs &a, const MxArgs &m, hipStream_t st) {
  constexpr int WA = DUCKMOE_MX_DN_WAVES;
  const auto kern = k_down_mx<WA, RT, SM, WPE>;
  static OccCache occ;
  int grid = 0;
  hipError_t err = persistent_grid(occ, kern, WA * 64, DUCKMOE_MX_WAVES_PER_CU,
                                   (a.H + 16 * RT - 1) / (16 * RT) * kMxGroups, a.cus, grid);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(WA * 64), 0, st, a, m);
  return hipSuccess;
}

template <int SM>
hipError_t launch_mx_down_sm(const LayerArgs &a, const MxArgs &m, hipStream_t st) {
  return a.T >= DUCKMOE_MX_DN_WIDE_T ? launch_mx_down_shape<SM, 3, 3>(a, m, st)
                                      : launch_mx_down_shape<SM, 2, 4>(a, m, st);
}

// chain_out: the partials stay for the next layer's k_mx_reduce_xprep, and out
// is not written.
hipError_t launch_mx_down(const LayerArgs &a, const MxArgs &m, hipStream_t st, bool chain_out) {
  const int sm = mx_sign_mode(a.I, a.dn_sign);
  const hipError_t err = sm == 2   ? launch_mx_down_sm<2>(a, m, st)
                         : sm == 1 ? launch_mx_down_sm<1>(a, m, st)
                                   : launch_mx_down_sm<0>(a, m, st);
  if (err != hipSuccess) return err;
  if (!chain_out)
    hipLaunchKernelGGL(k_mx_reduce, dim3((a.T * a.H + 255) / 256), dim3(256), 0, st, a, m);
  return hipGetLastError();
}

enum Stages { kGateUp = 1, kDown = 2, kBoth = 3 };

// Stack chaining on the matrix-core path: kChainIn, the layer's input is the
// previous layer's down partials in the same workspace; kChainOut, the layer
// leaves its partials there instead of writing out.
enum Chain { kChainIn = 1, kChainOut = 2 };

bool chain_ok(const duckmoe_layer *L, int T) {
  return use_mx(T, 1) && L->hidden <= kChainMaxH;
}

// Shared argument checks and dispatch of the layer entry points.
int run_layer(const duckmoe_layer *L, const float *x, const int32_t *ids, const float *w,
              int single_expert, int32_t T, float *out, int32_t n_shards, void *ws,
              size_t ws_bytes, hipStream_t stream, int stages, int in_rms = 0,
              float in_eps = 0.0f, int cus = 0, int chain = 0) {
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
  a.in_rms = in_rms;
  a.in_eps = in_eps;
  a.cus = cus;

  if (use_mx(T, n_shards)) {
    const MxLayout l = mx_layout(L, T, single, kHdrBytes + hbuf_bytes(L, T, single));
    uint8_t *b = reinterpret_cast<uint8_t *>(ws);
    MxArgs m;
    m.xb = reinterpret_cast<_Float16 *>(b + l.xb);
    m.xinv = reinterpret_cast<float *>(b + l.xinv);
    m.hb = reinterpret_cast<_Float16 *>(b + l.hb);
    m.hexp = reinterpret_cast<int8_t *>(b + l.hexp);
    m.part = reinterpret_cast<float *>(b + l.part);
    m.Hp = l.Hp;
    m.Ip = l.Ip;
    m.EB = l.EB;
    if ((stages & kGateUp) &&
        launch_mx_gate_up(a, m, stream, (chain & kChainIn) && in_rms) != hipSuccess)
      return DUCKMOE_EHIP;
    if ((stages & kDown) && launch_mx_down(a, m, stream, chain & kChainOut) != hipSuccess)
      return DUCKMOE_EHIP;
    return DUCKMOE_OK;
  }
  if (stages & kGateUp) {
    if (launch_gate_up(a, stream) != hipSuccess) return DUCKMOE_EHIP;
  }
  if (stages & kDown) {
    if (launch_down(a, stream) != hipSuccess) return DUCKMOE_EHIP;
  }
  return DUCKMOE_OK;
}

// ------------------------------------------------- allocation-free entry ----
// The workspace of duckmoe_moe_layer_noalloc: a file-scope device array, one
// copy per GPU the library runs on, held until the process ends.  On the host
// the array's name only stands in for it, so it is never passed to a kernel:
// its device address is looked up once per device (with that device current)
// by hipGetSymbolAddress, kept, and passed instead.  Every call on a GPU
// shares that GPU's array; the layer kernels write everything they read there
// (plan, status, h'), so nothing has to start at zero.
static __device__ __align__(256) uint8_t scratch[DUCKMOE_NOALLOC_WS_BYTES];

std::atomic<void *> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_ptr(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DUCKMOE_EHIP;
  void *p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DUCKMOE_EHIP;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
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

int duckmoe_moe_layer_noalloc(const duckmoe_layer *L, const float *x, const int32_t *ids,
                              const float *w, int32_t T, float *out, int32_t n_shards,
                              hipStream_t stream) {
  if (!ids) return DUCKMOE_EINVAL;
  void *ws = nullptr;
  const int rc = scratch_ptr(&ws);
  if (rc) return rc;
  return run_layer(L, x, ids, w, 0, T, out, n_shards, ws, DUCKMOE_NOALLOC_WS_BYTES, stream, kBoth);
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

int duckmoe_rms_normalize(const float *x, int32_t T, int32_t H, float eps, float *y,
                          hipStream_t stream) {
  if (!x || !y || T < 0 || H < 1 || !(eps >= 0.0f)) return DUCKMOE_EINVAL;
  if (T == 0) return DUCKMOE_OK;
  hipLaunchKernelGGL(k_rms, dim3(T), dim3(256), 0, stream, x, H, eps, y);
  return hipGetLastError() == hipSuccess ? DUCKMOE_OK : DUCKMOE_EHIP;
}

// stack workspace: one layer's workspace, then two [T][H] activation buffers
static size_t stack_act_off(const duckmoe_layer *L, int T) {
  return (ws_need(L, T, false) + 255) / 256 * 256;
}

static size_t stack_act_bytes(const duckmoe_layer *L, int T) {
  return ((size_t)T * L->hidden * sizeof(float) + 255) / 256 * 256;
}

static int check_stack(const duckmoe_layer *layers, int32_t n_layers, int32_t T) {
  if (!layers || n_layers < 1 || T < 1 || T > kMaxT) return DUCKMOE_EINVAL;
  for (int l = 0; l < n_layers; ++l) {
    const int rc = check_layer(&layers[l]);
    if (rc) return rc;
    const duckmoe_layer &a = layers[0], &b = layers[l];
    if (b.hidden != a.hidden || b.inter != a.inter || b.n_routed != a.n_routed ||
        b.top_k != a.top_k)
      return DUCKMOE_ESHAPE;
  }
  if (T * layers[0].top_k > kMaxIds) return DUCKMOE_ESHAPE;
  return DUCKMOE_OK;
}

size_t duckmoe_stack_workspace_bytes(const duckmoe_layer *layers, int32_t n_layers, int32_t T) {
  if (check_stack(layers, n_layers, T)) return 0;
  return stack_act_off(&layers[0], T) + 2 * stack_act_bytes(&layers[0], T);
}

int duckmoe_moe_stack(const duckmoe_layer *layers, int32_t n_layers, const float *x,
                      const int32_t *ids, const float *w, int32_t T, float eps, float *out,
                      void *ws, size_t ws_bytes, hipStream_t stream) {
  int rc = check_stack(layers, n_layers, T);
  if (rc) return rc;
  if (!x || !ids || !w || !out || !ws || !(eps >= 0.0f)) return DUCKMOE_EINVAL;
  if (!aligned(ws, 256)) return DUCKMOE_EINVAL;
  const duckmoe_layer *L0 = &layers[0];
  if (ws_bytes < duckmoe_stack_workspace_bytes(layers, n_layers, T)) return DUCKMOE_EWORKSPACE;
  uint8_t *base = reinterpret_cast<uint8_t *>(ws);
  float *act[2] = {reinterpret_cast<float *>(base + stack_act_off(L0, T)),
                   reinterpret_cast<float *>(base + stack_act_off(L0, T) +
                                             stack_act_bytes(L0, T))};
  // Layer l > 0 reads layer l-1's raw output and normalizes it in its gate/up
  // prologue (bit-identical to duckmoe_rms_normalize followed by the layer).
  // On the matrix-core path the raw output is never written between layers:
  // the next layer's first launch adds layer l-1's partials itself.
  const size_t per = (size_t)T * L0->top_k;
  const bool chained = chain_ok(L0, T);
  const float *in = x;
  for (int l = 0; l < n_layers; ++l) {
    float *y = l == n_layers - 1 ? out : act[l & 1];
    const int chain = !chained ? 0 : (l > 0 ? kChainIn : 0) | (l < n_layers - 1 ? kChainOut : 0);
    rc = run_layer(&layers[l], in, ids + l * per, w + l * per, 0, T, y, 1, ws,
                   stack_act_off(L0, T), stream, kBoth, l > 0, eps, 0, chain);
    if (rc) return rc;
    in = y;
  }
  return DUCKMOE_OK;
}

int duckmoe_read_probe(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream) {
  if (!buf || !sink) return DUCKMOE_EINVAL;
  if (!aligned(buf, 16) || bytes % 1024) return DUCKMOE_EINVAL;
  if (bytes / 1024 > 0xffffffffull) return DUCKMOE_ESHAPE;
  if (bytes == 0) return DUCKMOE_OK;
  hipLaunchKernelGGL(k_read_probe, dim3(1024), dim3(512), 0, stream,
                     reinterpret_cast<const uint4 *>(buf), (uint32_t)(bytes / 1024), sink);
  return hipGetLastError() == hipSuccess ? DUCKMOE_OK : DUCKMOE_EHIP;
}

// CUs a stream's CU mask enables (0: the query failed or the mask is empty,
// which the launches read as "the whole device").
static int stream_cus(hipStream_t s) {
  uint32_t mask[32] = {0};
  if (hipExtStreamGetCUMask(s, 32, mask) != hipSuccess) return 0;
  int n = 0;
  for (uint32_t m : mask) n += __builtin_popcount(m);
  return n;
}

int duckmoe_lane_init(duckmoe_lane *lane) {
  if (!lane) return DUCKMOE_EINVAL;
  lane->ready = nullptr;
  lane->done = nullptr;
  // a budget the caller set stays (capped by the stream's CU mask); 0 takes the mask's
  const int mask_cus = stream_cus(lane->stream);
  if (lane->cus < 0) return DUCKMOE_EINVAL;
  if (lane->cus == 0 || (mask_cus > 0 && mask_cus < lane->cus)) lane->cus = mask_cus;
  if (hipEventCreateWithFlags(&lane->ready, hipEventDisableTiming) != hipSuccess)
    return DUCKMOE_EHIP;
  if (hipEventCreateWithFlags(&lane->done, hipEventDisableTiming) != hipSuccess) {
    (void)hipEventDestroy(lane->ready);
    lane->ready = nullptr;
    return DUCKMOE_EHIP;
  }
  return DUCKMOE_OK;
}

int duckmoe_lane_destroy(duckmoe_lane *lane) {
  if (!lane) return DUCKMOE_EINVAL;
  int rc = DUCKMOE_OK;
  if (lane->ready && hipEventDestroy(lane->ready) != hipSuccess) rc = DUCKMOE_EHIP;
  if (lane->done && hipEventDestroy(lane->done) != hipSuccess) rc = DUCKMOE_EHIP;
  lane->ready = lane->done = nullptr;
  return rc;
}

int duckmoe_lane_begin(duckmoe_lane *lane, const duckmoe_layer *L, const float *x,
                       const int32_t *ids, const float *w, int32_t T, float *out,
                       hipStream_t producer) {
  if (!lane || !lane->ready || !lane->done || !ids) return DUCKMOE_EINVAL;
  // argument checks first: nothing is recorded for a call that would fail
  int rc = run_layer(L, x, ids, w, 0, T, out, 1, lane->ws, lane->ws_bytes, lane->stream, 0, 0,
                     0.0f, lane->cus);
  if (rc) return rc;
  if (hipEventRecord(lane->ready, producer) != hipSuccess) return DUCKMOE_EHIP;
  if (hipStreamWaitEvent(lane->stream, lane->ready, 0) != hipSuccess) return DUCKMOE_EHIP;
  rc = run_layer(L, x, ids, w, 0, T, out, 1, lane->ws, lane->ws_bytes, lane->stream, kBoth, 0,
                 0.0f, lane->cus);
  if (rc) return rc;
  return hipEventRecord(lane->done, lane->stream) == hipSuccess ? DUCKMOE_OK : DUCKMOE_EHIP;
}

int duckmoe_lane_finish(duckmoe_lane *lane, hipStream_t consumer) {
  if (!lane || !lane->done) return DUCKMOE_EINVAL;
  if (!consumer) return hipEventSynchronize(lane->done) == hipSuccess ? DUCKMOE_OK : DUCKMOE_EHIP;
  return hipStreamWaitEvent(consumer, lane->done, 0) == hipSuccess ? DUCKMOE_OK : DUCKMOE_EHIP;
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
  a.w = nullptr;  // the slot list needs no weights
  hipLaunchKernelGGL(k_plan, dim3(1), dim3(64), 0, stream, a, uniq, n_slots);
  return hipGetLastError() == hipSuccess ? DUCKMOE_OK : DUCKMOE_EHIP;
}

}  // extern "C"
