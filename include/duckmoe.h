/*
 * duckmoe.h - C ABI of libduckmoe: the fp9 routed-expert MoE FFN on gfx950.
 *
 * Sources (cited by page title and section):
 *  [fp9]   duck-llm memoir page "一鸭三吃：我把评测鸭变成了满血 DeepSeek-V3.2
 *          推理系统", section "在只有 AVX2 的 N100 上，我先做出了单核 MLP fp9":
 *          9-bit layout figure (sign bit 8, exponent bits 7..3 with bias 15,
 *          mantissa bits 2..0), body byte + packed sign bitplane storage
 *          (8 weights in 9 bytes), decode by placing the bits into fp16.
 *  [afd]   same page, section "真正埋下伏笔的是内存；R1 之后，问题第一次被改写":
 *          the FFN/MoE expert weights are the part held outside the GPU.
 *  [tp]    same page, section "真正难的不是把参数塞下，而是通信": tensor
 *          parallelism is the split that cuts per-token latency at bsz 1;
 *          section "先用 Qwen3 练级，再让 Qwen3.5 充当高压试炼场": slices
 *          narrower than 128 (multiple_of 64/32).
 *  [brk]   same page, section "16 tok/s 之后：一段没有跑通的路": MoE forward
 *          breakdown (prepare / send / per-box compute / fetch / host reduce).
 *  [route] chapter page "第 9 章 MTP1 dual-lane overlap", section 9.2
 *          "两条路线的判断": 8 routed experts per token (top_k = 8); the sets of
 *          two tokens barely overlap, so bsz 2 reads about twice the weights.
 *  [fp8]   memoir page, sections "真正埋下伏笔的是内存；R1 之后，问题第一次被改写"
 *          (the released checkpoints are fp8) and "先用 Qwen3 练级，再让
 *          Qwen3.5 充当高压试炼场" (the fp8 format uses 128 x 128 block scales).
 *  [lane]  chapter page "第 9 章 MTP1 dual-lane overlap", section 9.5
 *          "pair runtime：stage0/stage1 调度": per decoder layer, a GPU stage
 *          (attention, layernorm, residual add) precedes the FFN/MoE stage,
 *          and layer i+1 of a lane waits for layer i's MoE result.
 *  [pair]  same chapter page, section 9.5: lanes keep separate input and
 *          output buffers, and one lane's MoE stage is dispatched only after
 *          an event recorded behind the work that produced its input; section
 *          9.6 "Rust overlap 接口": begin starts a lane's MoE forward and returns
 *          at once, finish waits for it and hands over the result.
 *  [pf]    memoir page, section "限制条件": the fp9 prefill kernel is the part
 *          still far from the machine's peak, and contexts were tested up to
 *          2048 tokens; prefill is the same routed layer over many tokens.
 *  [f32]   ds4 glossary page "张量并行（Tensor Parallelism, TP）", section
 *          "形态一：Mac-to-Mac 张量并行（RDMA）": TP partial sums travel as f32.
 *
 * Conventions shared by every entry point:
 *  - Return 0 (DUCKMOE_OK) or a negative DUCKMOE_E* code; nothing throws.
 *  - Argument errors are detected on the host and returned before anything is
 *    launched; no output is written then.
 *  - Device entry points are asynchronous on the given stream (0 = the null
 *    stream).  A device fault surfaces at the caller's next synchronisation.
 *  - All memory is caller-owned, except the static device workspace of
 *    duckmoe_moe_layer_noalloc.  The library allocates no device memory.  Its
 *    only global state is per-device caches (compute-unit counts, launch
 *    shapes, that workspace's address), each filled once and then only read,
 *    so calls on different streams may run concurrently as long as they use
 *    different workspaces and outputs.
 *  - Device pointers must satisfy the alignment stated for them
 *    (DUCKMOE_EINVAL otherwise).
 */
#ifndef DUCKMOE_H
#define DUCKMOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DUCKMOE_OK          0
#define DUCKMOE_EINVAL     -1  /* null/misaligned pointer, T out of [1,8], bad index   */
#define DUCKMOE_ESHAPE     -2  /* a size the kernels do not support (see each call)    */
#define DUCKMOE_ENONFINITE -3  /* NaN given to the quantizer                           */
#define DUCKMOE_EWORKSPACE -4  /* ws_bytes < duckmoe_workspace_bytes(...)              */
#define DUCKMOE_EHIP       -5  /* the HIP runtime refused a launch or a copy           */

/* Bits of the device status word (duckmoe_status). */
#define DUCKMOE_STATUS_BAD_ID  1  /* a routed id outside [0, n_routed): entry skipped   */
#define DUCKMOE_STATUS_DUP_ID  2  /* a token lists an id twice: its weights were added  */

#define DUCKMOE_MAX_TOKENS 8      /* T, tokens per call                                 */
#define DUCKMOE_MAX_IDS    64     /* T * top_k                                          */
#define DUCKMOE_MAX_ROUTED 8192   /* n_routed                                           */

/*
 * One MoE layer's expert weights, resident in device memory, in the [fp9]
 * split storage.  Expert index n_routed is the shared expert.  H = hidden,
 * I = inter.  Rows are row-major along the contraction dimension:
 *   gu_body [n_routed+1][2][I][H]    uint8  gate rows (g=0) then up rows (g=1)
 *   gu_sign [n_routed+1][2][I][H/8]  uint8  sign byte j of a row: elements 8j..8j+7,
 *                                            element 8j+i in bit i
 *   dn_body [n_routed+1][H][I]       uint8  down rows
 *   dn_sign [n_routed+1][H][I/8]     uint8
 * Requirements: H and I multiples of 16, 16 <= I <= 32768, H >= 16,
 * 2 * H * I < 2^31, 1 <= top_k, 0 <= n_routed <= DUCKMOE_MAX_ROUTED
 * (DUCKMOE_ESHAPE otherwise).  n_routed = 0 describes a dense MLP: its only
 * expert is index 0, run with duckmoe_expert_ffn (the pages' first fp9
 * workload was a dense MLP, [fp9]);
 * body pointers 16-byte aligned, sign pointers 2-byte aligned (DUCKMOE_EINVAL).
 * In the matrix-core kernels (layer calls of 3 tokens and more, prefill),
 * sign planes aligned to 8 bytes and matrices whose rows are multiples of 64
 * elements let the kernels fetch more sign bytes per load; other layouts give
 * the same results more slowly.
 * The struct itself is read on the host during the call only.
 */
typedef struct duckmoe_layer {
  int32_t hidden;
  int32_t inter;
  int32_t n_routed;
  int32_t top_k;
  const uint8_t *gu_body;
  const uint8_t *gu_sign;
  const uint8_t *dn_body;
  const uint8_t *dn_sign;
} duckmoe_layer;

/* Text for a return code (static storage; never NULL). */
const char *duckmoe_strerror(int code);

/*
 * [fp9] Host quantizer and packer, synchronous, HOST pointers.
 *   w    [rows][cols] float32 (read only)
 *   body [rows][cols]   uint8  <- bits 7..0 of each code (exponent, mantissa)
 *   sign [rows][cols/8] uint8  <- sign bits, element 8j+i of a row in bit i of byte j
 * Rounding: to nearest, ties to even, computed directly from the float32 value
 * (never via fp16).  |w| >= 61440 and +-inf saturate to +-61440 (exponent 30,
 * mantissa 7); exponent 31 is never produced; the sign of zero is kept.
 * Errors: DUCKMOE_EINVAL for null pointers or rows/cols < 0; DUCKMOE_ESHAPE if
 * cols % 8 != 0; DUCKMOE_ENONFINITE if any element is NaN (the outputs are
 * then unspecified).  rows or cols == 0 is a no-op.
 */
int duckmoe_quantize_fp9(const float *w, int64_t rows, int64_t cols,
                         uint8_t *body, uint8_t *sign);

/*
 * [fp9] The same quantizer and packer on the GPU (bit-identical results),
 * asynchronous on `stream`; w, body, sign DEVICE pointers.
 *   w    [rows][cols] float32, 16-byte aligned
 *   body [rows][cols] uint8, 8-byte aligned;  sign [rows][cols/8] uint8
 *   nonfinite: device int32 or NULL; set to 1 if any element is NaN (never
 *              cleared by the call; the codes of NaN elements are unspecified)
 * Errors (host-side, nothing launched): DUCKMOE_EINVAL for negative sizes or
 * null or misaligned pointers, DUCKMOE_ESHAPE if cols % 8 != 0.  rows or
 * cols == 0 is a no-op (the pointers may then be null).
 */
int duckmoe_quantize_fp9_device(const float *w, int64_t rows, int64_t cols,
                                uint8_t *body, uint8_t *sign, int32_t *nonfinite,
                                hipStream_t stream);

/*
 * [fp8][fp9] Convert an fp8 weight matrix with block scales to fp9 planes on
 * the GPU, asynchronous on `stream`; all pointers DEVICE.
 *   fp8   [rows][cols] uint8, finite-only E4M3 codes (exponent bias 7,
 *         subnormals, no infinities, NaN = 0x7F/0xFF), 8-byte aligned
 *   scale [ceil(rows/block)][ceil(cols/block)] float32, row-major, 4-byte aligned;
 *         element (r, c) has weight value(code) * scale[r/block][c/block]
 *   body  [rows][cols] uint8 (8-byte aligned), sign [rows][cols/8] uint8:
 *         the fp9 planes, rounded once from the exact product (nearest, ties to
 *         even, saturating at +-61440: the quantizer's rounding)
 *   nonfinite: device int32 or NULL; set to 1 if a code is NaN or a product is
 *         NaN (never cleared by the call)
 * Errors (host-side): DUCKMOE_EINVAL for negative sizes, block < 8, null or
 * misaligned pointers; DUCKMOE_ESHAPE if cols or block is not a multiple of 8.
 * rows or cols == 0 is a no-op.
 */
int duckmoe_fp8_to_fp9(const uint8_t *fp8, const float *scale, int64_t rows, int64_t cols,
                       int32_t block, uint8_t *body, uint8_t *sign, int32_t *nonfinite,
                       hipStream_t stream);

/*
 * Bytes of device workspace duckmoe_expert_ffn / duckmoe_moe_layer need for T
 * tokens (the same figure covers both).  Returns 0 if the arguments are
 * invalid.  The workspace holds the status word, the expert-selection plan
 * and the per-(expert, token) SwiGLU activations (f32).  It needs no
 * initialisation: every call writes what it later reads.  Calls that may run
 * at the same time need separate workspaces.
 */
size_t duckmoe_workspace_bytes(const duckmoe_layer *L, int32_t T, int32_t n_shards);

/*
 * [afd][route][brk] Full routed layer for T tokens (1 <= T <= 8):
 *   out_t = shared(x_t) + sum_i w[t][i] * expert_{ids[t][i]}(x_t),
 *   expert(x) = W_down (silu(W_gate x) * (W_up x)),  silu(z) = z / (1 + e^-z).
 * Only the experts named in ids (their union over the batch) and the shared
 * expert are read from memory, each once per call.
 *   x   [T][H]          float32, device, 16-byte aligned
 *   ids [T][top_k]      int32,   device; ids of one token should be distinct
 *   w   [T][top_k]      float32, device
 *   out n_shards == 1:  [T][H] float32, device
 *       n_shards  > 1:  [n_shards][T][H]: shard r is the same sum restricted to
 *                       the intermediate slice [r*I/n_shards, (r+1)*I/n_shards)
 *                       of every expert ([tp][f32]); the shards add up to the
 *                       n_shards == 1 output.
 *   n_shards >= 1 must divide I, the slice width I / n_shards must be a
 *   multiple of 1024 or a power of two in [64, 1024], and n_shards > 1 needs
 *   I <= 2048 (DUCKMOE_ESHAPE otherwise); for I = 2048 that is n_shards in
 *   {1, 2, 4, 8, 16, 32}.
 *   ws  device workspace, 256-byte aligned, >= duckmoe_workspace_bytes(L,T,n_shards)
 * Ids outside [0, n_routed) are skipped and flag DUCKMOE_STATUS_BAD_ID; an id
 * repeated within a token has its weights added and flags DUCKMOE_STATUS_DUP_ID.
 */
int duckmoe_moe_layer(const duckmoe_layer *L, const float *x, const int32_t *ids,
                      const float *w, int32_t T, float *out, int32_t n_shards,
                      void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * duckmoe_moe_layer without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The call allocates nothing: it runs the
 * same kernels on a static device array of DUCKMOE_NOALLOC_WS_BYTES bytes that
 * the library holds on each GPU it runs on until the process ends (its address
 * is looked up on the first call on a device).  Arguments, results and errors
 * are those of duckmoe_moe_layer, plus DUCKMOE_EWORKSPACE when the call needs
 * more than DUCKMOE_NOALLOC_WS_BYTES of workspace (duckmoe_workspace_bytes)
 * and DUCKMOE_EHIP if the array's address cannot be obtained.  Every call on
 * one GPU shares that GPU's array, and the array keeps the last call's
 * contents: calls that overlap on one GPU (concurrent streams or host
 * threads) race, so the caller serialises them.  duckmoe_status cannot read
 * this call's status word (it is in the library's array).
 */
#define DUCKMOE_NOALLOC_WS_BYTES (16u << 20)  /* 16 MiB: DeepSeek-V3 layers up to 8 tokens */
int duckmoe_moe_layer_noalloc(const duckmoe_layer *L, const float *x, const int32_t *ids,
                              const float *w, int32_t T, float *out, int32_t n_shards,
                              hipStream_t stream);

/*
 * The two launches duckmoe_moe_layer makes, for callers that time or overlap
 * them separately.  Same arguments and checks as duckmoe_moe_layer.
 *   gate_up: plan + gate/up GEMVs + SwiGLU, the routing weight folded in;
 *            writes only the workspace.
 *   down:    down GEMVs + routing-weighted combine; reads the workspace the
 *            gate_up call left (same L, x, ids, w, T, ws) and writes out.
 */
int duckmoe_moe_gate_up(const duckmoe_layer *L, const float *x, const int32_t *ids,
                        const float *w, int32_t T, float *out, int32_t n_shards,
                        void *ws, size_t ws_bytes, hipStream_t stream);
int duckmoe_moe_down(const duckmoe_layer *L, const float *x, const int32_t *ids,
                     const float *w, int32_t T, float *out, int32_t n_shards,
                     void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * One expert e in [0, n_routed] (n_routed = the shared expert) for T tokens,
 * weight 1: out_t = expert_e(x_t).  Layouts, n_shards and ws as for
 * duckmoe_moe_layer; DUCKMOE_EINVAL if e is out of range.
 */
int duckmoe_expert_ffn(const duckmoe_layer *L, int32_t e, const float *x, int32_t T,
                       float *out, int32_t n_shards, void *ws, size_t ws_bytes,
                       hipStream_t stream);

/*
 * [lane] Glue between stacked layers: y[t] = x[t] / sqrt(mean_i x[t][i]^2 + eps)
 * for t < T, i < H, in float32.  x, y [T][H] device float32 (y may equal x).
 * DUCKMOE_EINVAL for null pointers, T < 0, H < 1 or eps < 0 (or NaN).  With
 * eps = 0 an all-zero row gives 0/0 = NaN, as the formula does.
 */
int duckmoe_rms_normalize(const float *x, int32_t T, int32_t H, float eps, float *y,
                          hipStream_t stream);

/*
 * [lane][afd] A stack of n_layers routed layers chained through the glue above:
 *   h_0 = x;  y_l = moe_layer(layers[l], h_l, ids[l], w[l]);
 *   h_{l+1} = rms_normalize(y_l, eps);  out = y_{n_layers-1}.
 *   layers  host array of n_layers descriptors with equal hidden, inter,
 *           n_routed and top_k (DUCKMOE_ESHAPE otherwise)
 *   x [T][H], out [T][H] float32 device; ids, w [n_layers][T][top_k] device
 *   ws      device workspace of duckmoe_stack_workspace_bytes(...) bytes,
 *           256-byte aligned, needing no initialisation
 * The status word (duckmoe_status on ws) is that of the last layer.  The glue
 * runs inside the next layer's first kernel (no launch of its own) with the
 * same arithmetic in the same order, so the result equals calling
 * duckmoe_moe_layer and duckmoe_rms_normalize in turn, bit for bit.  At T >= 3
 * with H <= 8192 that kernel also finishes the previous layer (its fixed-order
 * sum of the down pass's partial results), so the inner layers' outputs y_l
 * never go to memory: one launch fewer per layer.
 */
size_t duckmoe_stack_workspace_bytes(const duckmoe_layer *layers, int32_t n_layers, int32_t T);
int duckmoe_moe_stack(const duckmoe_layer *layers, int32_t n_layers, const float *x,
                      const int32_t *ids, const float *w, int32_t T, float eps, float *out,
                      void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * [pf][route][fp9] Prefill: the routed layer of duckmoe_moe_layer for many
 * tokens at once, with the tokens grouped by expert so that each selected
 * expert's weights are streamed once per tile of up to 64 of its tokens, and
 * the contractions run on the matrix cores (fp9 weights decoded to fp16,
 * activations carried as scaled fp16 hi/lo pairs, f32 accumulation).
 *   x [T][H], out [T][H]  float32 device, 16-byte aligned, 1 <= T <= 32768
 *   ids, w [T][top_k]     int32 / float32 device; ids == NULL runs the shared
 *                         (or, for n_routed = 0, the only) expert alone and
 *                         ignores w
 *   ws   device workspace of at least duckmoe_prefill_workspace_bytes(L, T,
 *        ids != NULL) bytes, 256-byte aligned, needing no initialisation;
 *        holds the per-expert token lists, the staged activations, h' and the
 *        per-entry outputs (about T * (top_k + 1) * (4 H + 4 I) bytes)
 * out_t = shared(x_t) + sum_i w[t][i] * expert_{ids[t][i]}(x_t); an id listed
 * twice by one token adds its weights (status bit DUCKMOE_STATUS_DUP_ID), an
 * id outside [0, n_routed) is skipped (DUCKMOE_STATUS_BAD_ID); the status word
 * is read with duckmoe_status on ws.  Each output element is a sum in a fixed
 * order: repeated calls give identical bits.
 * Requirements beyond the layer's: n_routed <= 1024, top_k <= 32 when ids is
 * given, T * roundup(H, 128) * 2 and T * (top_k + 1) * roundup(I, 128) * 2
 * below 2^31 (DUCKMOE_ESHAPE).  DUCKMOE_EINVAL for T outside [1, 32768], null
 * or misaligned pointers (w null with ids given); DUCKMOE_EWORKSPACE if
 * ws_bytes is too small.  duckmoe_prefill_workspace_bytes returns 0 for an
 * invalid layer or T.
 */
size_t duckmoe_prefill_workspace_bytes(const duckmoe_layer *L, int32_t T, int32_t routed);
int duckmoe_moe_prefill(const duckmoe_layer *L, const float *x, const int32_t *ids,
                        const float *w, int32_t T, float *out, void *ws, size_t ws_bytes,
                        hipStream_t stream);

/*
 * [pf] Test export: the per-expert token lists of a prefill call, written to
 * caller buffers (device, asynchronous on stream).
 *   ids, w [T][top_k] device (may be NULL when top_k == 0)
 *   offsets   [n_routed + 2] int32: first entry of list p; list 0 is the
 *             shared expert (every token, weight 1), list p >= 1 routed
 *             expert p - 1; offsets[n_routed + 1] = number of entries
 *   tokens    [T * (top_k + 1)] int32: entry -> token, ascending in a list
 *   weights   [T * (top_k + 1)] float32: entry -> routing weight (summed in
 *             id order for a repeated id)
 *   tok_entry [T][top_k + 1] int32: token t's shared entry, then the entry of
 *             ids[t][i] for the first position of each valid id, -1 for a
 *             repeat or an id out of range
 *   status    [1] int32: the status bits of the ids
 * Errors: DUCKMOE_EINVAL for T outside [1, 32768], top_k outside [0, 32],
 * n_routed outside [0, 1024] or null pointers.
 */
int duckmoe_prefill_plan(const int32_t *ids, const float *w, int32_t T, int32_t top_k,
                         int32_t n_routed, int32_t *offsets, int32_t *tokens, float *weights,
                         int32_t *tok_entry, int32_t *status, hipStream_t stream);

/*
 * [pair] Asynchronous lanes.  A lane owns a stream, a workspace and two HIP
 * events, so two tokens (two lanes) can have their layers in flight at once
 * while other work runs on the caller's streams.  The struct is caller-owned;
 * duckmoe_lane_init fills the events (no device memory is allocated) and
 * duckmoe_lane_destroy releases them.
 *   stream    the lane's stream (created by the caller, default priority).  A
 *             stream limited to a CU subset (hipExtStreamCreateWithCUMask)
 *             keeps the lane's kernels there: two lanes on complementary
 *             halves of the CUs run side by side instead of each filling the
 *             whole device and waiting for the other's workgroups.  Without
 *             a mask, a CU budget in `cus` (say half the device for each of
 *             two lanes) sizes each lane's persistent grids so that the two
 *             together fill the device once.  The results do not depend on
 *             the CU count (each output is computed in the same order on any
 *             grid).
 *   ws        the lane's workspace: >= duckmoe_workspace_bytes(L, T, 1) for the
 *             largest T it will run, 256-byte aligned; one lane per workspace
 * duckmoe_lane_begin records an event on `producer` (the stream that wrote x,
 * ids and w; 0 = the null stream), makes the lane's stream wait for it, runs
 * duckmoe_moe_layer there and records the lane's done event.  It returns
 * without waiting.  x, ids, w and out must stay valid until finish.
 * duckmoe_lane_finish makes `consumer` wait for the done event (no host
 * blocking); consumer == NULL blocks the host until the lane's layer is done.
 * Errors: DUCKMOE_EINVAL for a null lane or stream fields, plus the errors of
 * duckmoe_moe_layer (checked before anything is recorded); DUCKMOE_EHIP if the
 * runtime refuses an event operation.
 */
typedef struct duckmoe_lane {
  hipStream_t stream;
  void *ws;
  size_t ws_bytes;
  hipEvent_t ready;  /* set by duckmoe_lane_init */
  hipEvent_t done;   /* set by duckmoe_lane_init */
  int32_t cus;       /* CUs the lane's launches size their grids to (0 = all).  Set
                        by the caller before duckmoe_lane_init as a budget, or 0;
                        lane_init caps it by the stream's CU mask (or takes the
                        mask's count when it is 0) */
} duckmoe_lane;

int duckmoe_lane_init(duckmoe_lane *lane);
int duckmoe_lane_destroy(duckmoe_lane *lane);
int duckmoe_lane_begin(duckmoe_lane *lane, const duckmoe_layer *L, const float *x,
                       const int32_t *ids, const float *w, int32_t T, float *out,
                       hipStream_t producer);
int duckmoe_lane_finish(duckmoe_lane *lane, hipStream_t consumer);

/*
 * Reads the status word the last layer call on this workspace wrote
 * (DUCKMOE_STATUS_* bits).  Synchronises `stream` first.  status: host pointer.
 */
int duckmoe_status(const void *ws, int32_t *status, hipStream_t stream);

/* ---- building blocks, exported for parity tests ---------------------------- */

/*
 * [fp9] Decode n codes from the split planes to float32 through the fp16 route
 * (code << 7 is an fp16 pattern, converted by hardware).
 *   body [n] uint8, sign [(n+7)/8] uint8, out [n] float32; all device, any alignment.
 * n == 0 is a no-op; n < 0 or a null pointer -> DUCKMOE_EINVAL.
 */
int duckmoe_decode_fp9(const uint8_t *body, const uint8_t *sign, int64_t n,
                       float *out, hipStream_t stream);

/*
 * [fp9] y = W x, W [rows][cols] in split storage (body [rows][cols],
 * sign [rows][cols/8]), x [cols], y [rows] float32; all device.
 * cols % 8 == 0 (DUCKMOE_ESHAPE); body/x 8-byte aligned (DUCKMOE_EINVAL).
 */
int duckmoe_gemv_fp9(const uint8_t *body, const uint8_t *sign, int32_t rows, int32_t cols,
                     const float *x, float *y, hipStream_t stream);

/*
 * [route] Expert-selection plan, in the slot order the layer kernels use:
 * n_routed (the shared expert) first, then the distinct valid ids of
 * ids[T][top_k] in order of first appearance (token-major).  Invalid ids
 * (outside [0, n_routed)) are left out.
 *   uniq [T*top_k+1] int32 device <- plan entries (the rest untouched)
 *   n_slots [1] int32 device      <- number of entries written (distinct + 1)
 */
int duckmoe_moe_plan(const int32_t *ids, int32_t T, int32_t top_k, int32_t n_routed,
                     int32_t *uniq, int32_t *n_slots, hipStream_t stream);

/*
 * Calibration: a plain streaming read of `bytes` device bytes (16-byte
 * aligned buf, bytes a multiple of 1024; DUCKMOE_EINVAL otherwise) with
 * non-temporal dwordx4 loads, 8 in flight per lane, 32 waves per CU.  It computes nothing
 * of the method; its duration is the read ceiling that the weight-streaming
 * kernels above are compared with.  sink: device uint32, written only in a case
 * that does not occur (it keeps the loads alive).
 */
int duckmoe_read_probe(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DUCKMOE_H */
