/*
 * skinny_gemm.h - C ABI of the MI355X (gfx950) decode-phase linear layer.
 *
 * Operation (every entry point):  y[M x N] = x[M x K] . W^T,  M = 1..16 tokens.
 *
 *   The decode-phase linear layer is a tall-skinny product of a few token
 *   rows with a weight matrix that is read from HBM once per step
 *   ("Developing a custom Qwen2.5 72B inference engine from scratch - what is
 *   the real bottleneck?", section 2 "The two-phase reality" and section 6.1
 *   "Decode GEMV: already near the roofline").  A linear layer computes
 *   y = x W with one row of x per token ("Multi-GPU Inference and Serving at
 *   Scale", Example 2); here W is stored one row per output feature, so the
 *   product is x . W^T.
 *
 *   FP8 weights are weight-only: activations stay 16-bit and each FP8 weight
 *   is dequantized with the fp32 scale of the 128 x 128 block it lies in
 *   ("9% faster GLM-5.3-Flash prefill with GPU-to-GPU IPC (and why TileLang
 *   didn't help)", section "TileLang: twice as fast, and no faster"; the
 *   Qwen2.5 72B engine report, section 6.2).
 *
 * Layouts (all row-major, contiguous, device memory):
 *   x        [M][K]                    bf16
 *   W        [N][K]                    bf16, or OCP E4M3FN bytes (FP8)
 *   w_scale  [ceil(N/128)][ceil(K/128)] fp32; weight (n, k) uses
 *                                       w_scale[n/128][k/128] (FP8 only)
 *   y        [M][N]                    bf16, round-to-nearest-even
 *   Accumulation is fp32.  Results are within 2e-3 * sum_k |x w| + 1e-6 of
 *   the exact product, and bitwise reproducible for a given device and plan.
 *
 * Requirements checked on the host before anything is enqueued:
 *   1 <= M <= SKINNY_MAX_M, N >= 1, K >= 1; K % 8 == 0 (bf16) or
 *   K % 16 == 0 (FP8); x, W, y and the workspace 16-byte aligned; w_scale
 *   4-byte aligned; no NULL operand.  Violations return a status and enqueue
 *   nothing.
 *
 * Ownership and concurrency:
 *   The caller owns every buffer (x, W, w_scale, y, workspace) and keeps it
 *   alive until the work on `stream` has finished.  The library allocates
 *   nothing and keeps no pointer after a call returns.  Host arrays passed in
 *   (the `linears` of a stack) are read during the call only.  y must not
 *   overlap x, W, w_scale, the workspace or another linear's y, and the
 *   workspace must not overlap x, W or w_scale (checked:
 *   SKINNY_ERR_INVALID_ARG).  Calls enqueue work on `stream` (a hipStream_t;
 *   NULL is the default stream) and return without waiting for it; execution
 *   faults surface at the caller's next synchronization.  Calls on different streams need separate workspaces.
 *   Workspace contents are undefined after a call.  Entry points may be
 *   called from several host threads at once: the library's only shared
 *   state is a per-device cache of device properties, occupancy results and
 *   granted LDS sizes, filled on first use under a lock.
 */
#ifndef SKINNY_GEMM_H
#define SKINNY_GEMM_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SKINNY_ABI_VERSION 2
#define SKINNY_MAX_M 16
/* Linears whose descriptors travel in a main-kernel launch's arguments; a
 * launch over more linears reads them from a table in the workspace. */
#define SKINNY_MAX_LINEARS_PER_LAUNCH 32
/* Smallest workspace any call asks for (bytes). */
#define SKINNY_MIN_WORKSPACE_BYTES 256

typedef enum skinny_status {
  SKINNY_OK = 0,
  SKINNY_ERR_INVALID_ARG = 1, /* NULL operand, M outside 1..16, N < 1, K < 1, count < 1,
                                 unknown dtype or variant, overlapping output             */
  SKINNY_ERR_UNSUPPORTED = 2, /* K not a multiple of 8 (bf16) / 16 (FP8), misaligned
                                 pointer, shape too large, device is not gfx950            */
  SKINNY_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than the *_workspace_bytes value */
  SKINNY_ERR_HIP = 4          /* a HIP call failed (device query or kernel launch)          */
} skinny_status;

enum skinny_dtype { SKINNY_BF16 = 0, SKINNY_FP8_BS128 = 1 };

/* Compute variant of the main kernel.  VECTOR streams one row per wave and
 * multiplies on the vector ALUs (M <= 8); MFMA streams 16-row tiles and
 * multiplies on the matrix cores (any M).  AUTO picks per (dtype, M) from
 * measurement. */
enum skinny_variant { SKINNY_VARIANT_AUTO = 0, SKINNY_VARIANT_VECTOR = 1, SKINNY_VARIANT_MFMA = 2 };

/* One linear of a stack.  All pointers are device pointers. */
typedef struct skinny_linear {
  int dtype;            /* SKINNY_BF16 or SKINNY_FP8_BS128                  */
  int N;                /* output features: rows of W, columns of y         */
  int K;                /* input features: columns of W and x               */
  int reserved;         /* must be 0                                        */
  const void* w;        /* W[N][K] bf16 or E4M3FN bytes                     */
  const float* w_scale; /* FP8: [ceil(N/128)][ceil(K/128)] fp32; bf16: NULL */
  const void* x;        /* x[M][K] bf16                                     */
  void* y;              /* y[M][N] bf16                                     */
} skinny_linear;

/* Main kernel of a launch, as the plan queries report it. */
enum skinny_kernel {
  SKINNY_KERNEL_NONE = 0,
  SKINNY_KERNEL_ROWS = 1,         /* skinny_rows (VECTOR), deep instance; MoE form      */
  SKINNY_KERNEL_ROWS_LEAN = 2,    /* skinny_rows, lean instance (bf16 launches >= 0.4 GB) */
  SKINNY_KERNEL_ROWS_FLAT = 3,    /* skinny_rows_flat (loads streamed across units):
                                     launches < 0.4 GB of up to 4 (bf16) or 2 (FP8)
                                     tokens, one-token FP8 launches >= 1 GB             */
  SKINNY_KERNEL_TILES = 4,        /* skinny_tiles (MFMA), 4-wave workgroups; MoE form  */
  SKINNY_KERNEL_TILES_WIDE = 5,   /* skinny_tiles, 8-wave workgroups                    */
  SKINNY_KERNEL_TILES_KSPLIT = 6, /* skinny_tiles' K-split form (one-token MoE slices)  */
  SKINNY_KERNEL_MOE_MLP1 = 7      /* skinny_moe_mlp1 (the experts' MLP in one launch)   */
};

/* Launch plan override, for tests and benchmarks.  Zero-initialised = automatic. */
typedef struct skinny_plan {
  int variant;          /* enum skinny_variant                               */
  int waves;            /* persistent waves per main launch; 0 = automatic   */
  int kernel;           /* enum skinny_kernel, filled by the plan queries;
                           ignored on input                                  */
  int reserved[5];      /* must be 0                                         */
} skinny_plan;

/* Bytes of workspace a single linear needs: at least SKINNY_MIN_WORKSPACE_BYTES
 * for valid arguments, 0 for invalid ones.  Pure host arithmetic, no HIP call.
 * The workspace holds the fp32 partial sums of K-chunks that the second pass
 * adds: for every row group of a linear that the launch splits into C > 1
 * K-chunks, C slots of [M][band rows] floats.  The value covers the largest
 * split either variant may choose.  The split is the long dimension cut
 * across workgroups so that a skinny launch still streams on the whole chip
 * ("9% faster GLM-5.3-Flash prefill with GPU-to-GPU IPC (and why TileLang
 * didn't help)", section "TileLang: twice as fast, and no faster"); a
 * K-split's partial results add up to the product ("Multi-GPU Inference and
 * Serving at Scale", Example 3, the row-split second linear). */
size_t skinny_workspace_bytes(int dtype, int M, int N, int K);

/* Bytes of workspace decode_linear_stack needs for these linears at this M:
 * the partial sums of its launches (for a launch of more than
 * SKINNY_MAX_LINEARS_PER_LAUNCH linears, bounded at the largest grid any
 * launch runs) plus that launch's descriptor table. */
size_t skinny_stack_workspace_bytes(const skinny_linear* linears, int count, int M);

/* y = x . W^T with bf16 W: one linear layer of the decode step, x the
 * [M][K] activations of M tokens, W the layer's [N][K] weights ("Multi-GPU
 * Inference and Serving at Scale", Example 2: a linear's product, worked on
 * a small matrix; "Developing a custom Qwen2.5 72B inference engine from
 * scratch - what is the real bottleneck?", section 6.1: the decode GEMV).
 *   x, y       device, [M][K] and [M][N] bf16 row-major, 16-byte aligned
 *   w          device, [N][K] bf16 row-major (the nn.Linear layout)
 *   workspace  device, >= skinny_workspace_bytes(SKINNY_BF16, M, N, K)
 * Argument errors are returned before anything is enqueued; the call is
 * asynchronous on `stream`. */
skinny_status skinny_gemm_bf16(const void* x, const void* w, void* y, int M, int N, int K,
                               void* workspace, size_t workspace_bytes, void* stream);

/* y = x . (e4m3(W) * block scale)^T: weight-only FP8, each weight an OCP
 * E4M3FN byte times the fp32 scale of its 128 x 128 block, activations and
 * outputs bf16 ("9% faster GLM-5.3-Flash prefill with GPU-to-GPU IPC (and why
 * TileLang didn't help)", section "TileLang: twice as fast, and no faster":
 * FP8 weights with 128 x 128 block scales against 16-bit activations).
 *   w_fp8      device, [N][K] bytes row-major
 *   w_scale    device, [ceil(N/128)][ceil(K/128)] fp32 row-major; the scale
 *              of W[n][k] is w_scale[n / 128][k / 128]
 *   x, y, workspace as skinny_gemm_bf16 (workspace for SKINNY_FP8_BS128) */
skinny_status skinny_gemm_fp8_bs128(const void* x, const void* w_fp8, const float* w_scale,
                                    void* y, int M, int N, int K, void* workspace,
                                    size_t workspace_bytes, void* stream);

/* Runs `count` independent linears that share M, e.g. the QKV, O, gate_up
 * and down projections of every decoder layer: the decode step streams every
 * layer's weights once per generated token ("Developing a custom Qwen2.5 72B
 * inference engine from scratch - what is the real bottleneck?", section 1
 * (80 layers, each with attention and MLP projections) and section 2 "The
 * two-phase reality" (decode reads the whole model from HBM per token)).
 *   linears    host array of `count` >= 1 skinny_linear, read during the call
 *   M          tokens, 1..SKINNY_MAX_M, the rows of every x and y
 *   workspace  device, 16-byte aligned, >= skinny_stack_workspace_bytes(linears,
 *              count, M); contents undefined afterwards
 * Each linear reads its own x and writes its own y; no y may overlap any x,
 * W, w_scale, other y or the workspace (checked).  The linears of each dtype,
 * in call order, are streamed by one persistent launch (one per 4096 linears
 * of a dtype, should a call have more); a launch of more than
 * SKINNY_MAX_LINEARS_PER_LAUNCH linears reads their descriptors from a table
 * that the call copies from host memory into the workspace on `stream` just
 * before it.  On a stream under graph capture (where such a copy would read
 * this call's host memory at every replay) the call instead makes launches of
 * at most SKINNY_MAX_LINEARS_PER_LAUNCH linears.  Each launch's split-K
 * partial sums are combined by a second, deterministic pass.  Errors (any
 * linear failing the checks of a single linear) are returned before anything
 * is enqueued. */
skinny_status decode_linear_stack(const skinny_linear* linears, int count, int M,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* decode_linear_stack for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): no workspace argument; the split-K partial sums go to a static
 * device buffer of SKINNY_STATIC_SCRATCH_BYTES that the library holds on each
 * GPU it runs on until the process ends.  Nothing is allocated on the call
 * path (the first call on a device only looks up the buffer's address there),
 * and nothing is copied: its launches hold at most
 * SKINNY_MAX_LINEARS_PER_LAUNCH linears each, descriptors in the arguments.
 *   A call is accepted only if skinny_stack_workspace_bytes of each of its
 *   launches (every SKINNY_MAX_LINEARS_PER_LAUNCH consecutive linears of one
 *   dtype, in call order) is <= SKINNY_STATIC_SCRATCH_BYTES (a bound from the
 *   shapes alone, so the same call is accepted on every device); otherwise
 *   SKINNY_ERR_WORKSPACE, returned before anything is enqueued.  Every other argument rule and
 *   error is that of decode_linear_stack.
 *   All calls on one GPU share its buffer, which keeps the last call's
 *   contents: calls on one stream are ordered and safe, but calls that may
 *   overlap on one GPU (other streams, other host threads) race on it and
 *   give wrong results.  No part of the buffer needs to start at zero. */
#define SKINNY_STATIC_SCRATCH_BYTES (64u << 20)
skinny_status decode_linear_stack_noalloc(const skinny_linear* linears, int count, int M,
                                          void* stream);

/* decode_linear_stack with an explicit plan (plan may be NULL = automatic). */
skinny_status skinny_linear_run(const skinny_linear* linears, int count, int M,
                                const skinny_plan* plan, void* workspace,
                                size_t workspace_bytes, void* stream);

/* Number of main-kernel launches a call over these linears makes on a stream
 * not under graph capture: one per dtype present (per 4096 linears of it);
 * 0 if invalid. */
int skinny_launch_count(const skinny_linear* linears, int count);

/* skinny_linear_run that also records events around each main-kernel launch,
 * for benchmarks: events[2 g] just before and events[2 g + 1] just after
 * launch g, on `stream`.  `events` is a host array of hipEvent_t created by
 * the caller; event_count must be >= 2 * skinny_launch_count(linears, count).
 * The second (combine) pass of each launch is enqueued after events[2 g + 1]. */
skinny_status skinny_linear_run_timed(const skinny_linear* linears, int count, int M,
                                      const skinny_plan* plan, void* const* events,
                                      int event_count, void* workspace,
                                      size_t workspace_bytes, void* stream);

/* Rows of W in one row group of the main kernel of this dtype, variant
 * (VECTOR or MFMA; 0 for AUTO, whose choice depends on the shapes) and M; 0 if
 * invalid.  For MFMA this is the 4-wave workgroup's 64; FP8 launches of M >= 2
 * tokens with at least 8 row groups of 128 rows per compute unit run 8-wave
 * workgroups with 128-row groups instead.  The split-K workspace holds fp32 partial sums laid out
 * [slot][M][band rows]: one slot per K-chunk of each row group of a linear the
 * launch splits; linears in order, then row groups, then K-chunks in K order. */
int skinny_band_rows(int dtype, int variant, int M);

/* The automatic plan (fills *out) of the launch of linears[0]'s dtype on
 * the current device: a call launches its linears grouped by dtype (one
 * launch per dtype, or launches of at most SKINNY_MAX_LINEARS_PER_LAUNCH under
 * graph capture), and each launch chooses its own variant (it can depend on
 * the launch's size).  out->variant, ->waves
 * (persistent waves of the main launch) and ->kernel (its form) are set. */
skinny_status skinny_plan_query(const skinny_linear* linears, int count, int M,
                                skinny_plan* out);

/* Greedy next token: idx[m] = the smallest n such that y[m][n] is the largest
 * of y[m][0..N), comparing the bf16 values (NaN ranks below every number,
 * -inf included, so a row of NaNs gives 0).  This is the decode step's on-device argmax
 * ("Developing a custom Qwen2.5 72B inference engine from scratch - what is
 * the real bottleneck?", section 5, third lever: pick the next token on the
 * GPU rather than copying the logits back to the host).
 *   y          [M][N] bf16, device, 2-byte aligned (read 16 bytes at a time
 *              when y is 16-byte aligned and N % 8 == 0)
 *   idx        [M] int32, device, 4-byte aligned, written
 *   workspace  device, 16-byte aligned, >= skinny_argmax_workspace_bytes(M, N)
 *              (a (value, index) pair per 4096 logits of a row)
 * y, idx and the workspace must not overlap.  1 <= M <= SKINNY_MAX_M, N >= 1;
 * errors are returned before anything is enqueued.  Two launches, no
 * atomics; the result does not depend on the launch. */
size_t skinny_argmax_workspace_bytes(int M, int N);
skinny_status skinny_argmax_bf16(const void* y, int M, int N, int* idx, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* The vocabulary projection and its greedy token in one call (same section
 * and lever): runs the one linear `head` (N = vocabulary size, K = hidden
 * size, head->y = the logits [M][N], written) exactly as decode_linear_stack
 * would, and writes into next_token[M] (device int32) what skinny_argmax_bf16
 * over those logits gives.  Where the linear runs on the vector kernel with K
 * unsplit, its launch also leaves one (value, index) pair per workgroup and
 * token and a single pass reduces them; otherwise the two argmax passes run
 * after the linear.  next_token must not overlap x, W, w_scale, y or the
 * workspace.  The workspace serves the linear and the argmax (stream order),
 * so it needs skinny_lm_head_workspace_bytes(head, M) bytes (0 for invalid
 * arguments); less returns SKINNY_ERR_WORKSPACE before anything is enqueued. */
size_t skinny_lm_head_workspace_bytes(const skinny_linear* head, int M);
skinny_status skinny_lm_head_argmax(const skinny_linear* head, int M, int* next_token,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* One gated MLP of a decoder layer (Qwen2.5's SiLU-gated unit): y = down(h),
 * h = silu(g) * u, [g | u] = x . W_gate_up^T ("Multi-GPU Inference and
 * Serving at Scale", Example 3: a column-split linear, the activation, then a
 * row-split linear; the Qwen2.5 72B engine report, section 3, the MLP of each
 * layer).  All pointers are device pointers:
 *   x          [M][H] bf16                    y          [M][H] bf16, written
 *   w_gate_up  [2I][H] bf16 or E4M3FN: rows 0..I-1 the gate, I..2I-1 the up
 *   w_down     [H][I] bf16 or E4M3FN
 *   s_gate_up  [ceil(2I/128)][ceil(H/128)] fp32, s_down [ceil(H/128)][ceil(I/128)]
 *              fp32 (FP8 only; NULL for bf16)
 * g and u are the gate_up linear's bf16 outputs; h = bf16(silu(g) * u) is
 * computed in fp32 (silu(g) = g / (1 + e^-g)) while down stages its input, so
 * no separate activation pass runs.  Both linears accumulate in fp32 and are
 * within the bound of each linear.  The intermediate [M][2I] bf16 lives in
 * the workspace (skinny_mlp_workspace_bytes(mlp, M), 0 for invalid
 * arguments).  H % 8 == 0 and I % 8 == 0 (bf16) or % 16 (FP8); y must not
 * overlap x, the weights, the scales or the workspace, and x must not overlap
 * the workspace.  reserved must be 0. */
typedef struct skinny_mlp {
  int dtype;
  int H;
  int I;
  int reserved;
  const void* w_gate_up;
  const float* s_gate_up;
  const void* w_down;
  const float* s_down;
  const void* x;
  void* y;
} skinny_mlp;
size_t skinny_mlp_workspace_bytes(const skinny_mlp* mlp, int M);
skinny_status skinny_mlp_swiglu(const skinny_mlp* mlp, int M, void* workspace,
                                size_t workspace_bytes, void* stream);

/* One linear of a mixture-of-experts layer over the routes of a decode or
 * verify batch.  A router sends each of T tokens to topk experts, every
 * expert being its own small network ("Multi-GPU Inference and Serving at
 * Scale", Example 8); a verify step passes a handful of tokens through the
 * weight-only FP8 expert matmuls ("9% faster GLM-5.3-Flash prefill with
 * GPU-to-GPU IPC (and why TileLang didn't help)", section "TileLang: twice as
 * fast, and no faster").  Route r = t * topk + j is token t's j-th choice,
 * e = ids[r]:
 *   y[r] = x_r . W_e^T, x_r = x[t] (default) or x[r] (SKINNY_MOE_X_PER_ROUTE),
 *   y[r] = 0 for every r whose e is outside [0, E).
 * With SKINNY_MOE_SWIGLU each x row holds [g | u] (2K values) and x_r is
 * bf16(silu(g) * u) computed in fp32 as the input is staged: the experts'
 * down projection reads their gate_up outputs directly.
 *   experts->w        [E][N][K] bf16 or E4M3FN (expert e at e * N * K)
 *   experts->w_scale  [E][ceil(N/128)][ceil(K/128)] fp32 (FP8), NULL (bf16)
 *   x                 [T][K] bf16, or [T * topk][K]; 2K columns with SWIGLU
 *   ids               [T][topk] int32, device, read by the kernel (no host
 *                     synchronization); any values (duplicates included)
 *   y                 [T * topk][N] bf16, written
 * Each chosen expert's weights are streamed once for all of its routes, in
 * one persistent launch that finds the routes per expert itself (plus a
 * second pass when K is split).  Accumulation is fp32 with the single-linear
 * bound per route.  Requirements as for a linear (K % 8 or % 16, 16-byte
 * aligned x, y, w and workspace; 4-byte aligned ids and w_scale), plus
 * 1 <= T <= SKINNY_MAX_M, 1 <= topk <= SKINNY_MAX_TOPK, E >= 1; y must not
 * overlap x, ids, the weights, the scales or the workspace, and the
 * workspace must not overlap x or ids.  Workspace:
 * skinny_moe_workspace_bytes(experts, T, topk, flags), 0 for invalid
 * arguments. */
#define SKINNY_MAX_TOPK 16
enum skinny_moe_flags { SKINNY_MOE_X_PER_ROUTE = 1, SKINNY_MOE_SWIGLU = 2 };
typedef struct skinny_experts {
  int dtype;            /* SKINNY_BF16 or SKINNY_FP8_BS128 */
  int E;                /* experts                          */
  int N;                /* rows of each expert's W          */
  int K;                /* columns of each expert's W       */
  const void* w;
  const float* w_scale;
} skinny_experts;
size_t skinny_moe_workspace_bytes(const skinny_experts* experts, int T, int topk, int flags);
skinny_status skinny_moe_linear(const skinny_experts* experts, const void* x, const int* ids,
                                int T, int topk, int flags, void* y, void* workspace,
                                size_t workspace_bytes, void* stream);
/* skinny_moe_linear recording events[0] / events[1] (hipEvent_t, created by
 * the caller) just before and after its main launch, for benchmarks. */
skinny_status skinny_moe_linear_timed(const skinny_experts* experts, const void* x,
                                      const int* ids, int T, int topk, int flags, void* y,
                                      void* const* events, void* workspace,
                                      size_t workspace_bytes, void* stream);
/* The main kernel skinny_moe_linear takes for these experts and routes, for
 * tests and benchmarks: out->variant is SKINNY_VARIANT_VECTOR (the row
 * kernel, for one-token slices of rows long enough to keep its loads in
 * flight) or SKINNY_VARIANT_MFMA (the tile kernel); out->kernel names the
 * kernel's form; out->waves and out->reserved are 0.  Host logic only (no device call).  Errors: the
 * argument checks of skinny_moe_linear on experts, T, topk and flags, and
 * SKINNY_ERR_INVALID_ARG for a NULL out. */
skinny_status skinny_moe_plan_query(const skinny_experts* experts, int T, int topk, int flags,
                                    skinny_plan* out);

/* The experts' gated MLP over the routes of a batch (the same sources as
 * skinny_moe_linear: the router's top-k experts, each its own small MLP whose
 * SiLU-gated activation sits between its two linears, "Multi-GPU Inference
 * and Serving at Scale", Examples 3 and 8).  For route r = t * topk + j,
 * e = ids[r]:
 *   [g | u] = bf16(x[t] . Wgu_e^T),  y[r] = bf16(silu(g) * u) . Wdn_e^T,
 * exactly skinny_moe_linear(gate_up, x, ids, ..., flags 0) into a
 * [T * topk][2I] buffer followed by skinny_moe_linear(down, that buffer, ids,
 * ..., SKINNY_MOE_X_PER_ROUTE | SKINNY_MOE_SWIGLU, y).  y[r] = 0 for routes
 * whose e is outside [0, E).
 *   gate_up  E experts of N = 2I rows, K = H columns
 *   down     the same E experts (same dtype or not) of N rows, K = I columns
 *   x        [T][H] bf16;  ids [T][topk] int32, device;  y [T * topk][N] bf16
 * One token (T = 1, topk <= 16, both linears of one dtype, and each
 * workgroup's rows within the one-token kernel's registers) runs as one
 * launch: every wave issues the loads of all its gate_up and down rows at its
 * start, and the workgroups (one or two per CU, all resident) meet once
 * between the linears through a counter in the workspace.  A wait there gives
 * up after a bounded number of polls (skinny_moe_mlp_set_spin_limit) and then
 * sets the flag word, leaving y invalid; it never hangs.  Other calls make the
 * two launches.
 *   Workspace: skinny_moe_mlp_workspace_bytes(gate_up, down, T, topk) bytes,
 * 256-byte aligned; 0 for invalid arguments.  Its first
 * SKINNY_MOE_MLP_COUNTER_BYTES hold a counter (bytes 0-7: workgroups of the
 * one-launch form finished over all calls, a multiple of the grid between
 * calls) and a flag (bytes 8-11, nonzero once a wait gave up; the caller
 * clears it): zero them once before the first call on that workspace, do not
 * hand the workspace to other calls in between, and do not run two calls on
 * it at once.  The gate_up outputs follow: [T * topk][2I] bf16 (two launches),
 * or [topk][I] 64-bit words, each this call's number (low 32 bits of the
 * counter / grid + 1) above two bf16 values (one launch; rows of routes with
 * no expert keep what they held). */
#define SKINNY_MOE_MLP_COUNTER_BYTES 256
/* Requirements and errors as for skinny_moe_linear on both linears, plus gate_up->E ==
 * down->E and gate_up->N == 2 * down->K (else SKINNY_ERR_INVALID_ARG); y
 * must not overlap x, ids, the weights, the scales or the workspace, and the
 * workspace must not overlap x, ids, the weights or the scales. */
size_t skinny_moe_mlp_workspace_bytes(const skinny_experts* gate_up, const skinny_experts* down,
                                      int T, int topk);
skinny_status skinny_moe_mlp_swiglu(const skinny_experts* gate_up, const skinny_experts* down,
                                    const void* x, const int* ids, int T, int topk, void* y,
                                    void* workspace, size_t workspace_bytes, void* stream);
/* skinny_moe_mlp_swiglu recording events[0] / events[1] just before and after
 * its main launch (the one launch, or gate_up's), for benchmarks. */
skinny_status skinny_moe_mlp_swiglu_timed(const skinny_experts* gate_up,
                                          const skinny_experts* down, const void* x,
                                          const int* ids, int T, int topk, void* y,
                                          void* const* events, void* workspace,
                                          size_t workspace_bytes, void* stream);
/* Polls before the one-token launch's wait gives up (default 4194304; a
 * negative value makes it give up without waiting).  Process-wide; read when
 * a call is enqueued.  For tests of that path. */
void skinny_moe_mlp_set_spin_limit(long long polls);
/* The plan of skinny_moe_mlp_swiglu's main launch on the current device:
 * kernel SKINNY_KERNEL_MOE_MLP1 (variant VECTOR, waves of its grid) for the
 * one launch, else skinny_moe_plan_query's answer for the gate_up launch. */
skinny_status skinny_moe_mlp_plan_query(const skinny_experts* gate_up, const skinny_experts* down,
                                        int T, int topk, skinny_plan* out);

/* Static text for a status code; never NULL. */
const char* skinny_status_string(int status);

/* SKINNY_ABI_VERSION of the loaded library. */
int skinny_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SKINNY_GEMM_H */
