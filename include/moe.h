/*
 * moe.h -- C ABI of libmoe: one GPU's share of a sparse Mixture-of-Experts layer on
 * AMD Instinct MI355X (gfx950).
 *
 * The layer, in the notation of the "EP / DeepEP explanation" page (section 2): N tokens
 * with hidden states x in R^{N x H}, E routed experts, router logits z in R^{N x E}, for
 * each token t an index set I_t of k experts with gates g_{t,e}, and
 *
 *     y_t = sum_{e in I_t} g_{t,e} * Expert_e(x_t),     n_e = |{(t, e) : e in I_t}|.
 *
 * The calls run in the order the pages give for a MoE layer ("MoE part 4: DeepEP and
 * GroupedGEMM", section 4: permute by expert -> grouped GEMM over tokens-per-expert ->
 * unpermute and weighted sum; section 4.2: router top-k with correction bias and grouped
 * top-k first):
 *
 *     moe_router_logits -> moe_route -> moe_dispatch_layout -> moe_permute -> moe_grouped_ffn
 *         -> moe_combine
 *
 * On one GPU the dispatch and combine all-to-alls of expert parallelism become the
 * on-device permute and unpermute.
 *
 * Conventions (all entry points):
 *   - Every array argument is a DEVICE pointer to row-major, contiguous memory.  Row
 *     bases must be 16-byte aligned (every row length below is a multiple of 16 bytes).
 *   - The caller owns every buffer, workspaces included.  The library never allocates
 *     or frees device memory and keeps no pointer after a call returns; it holds no
 *     state and may be called from several host threads.  (One exception, by design:
 *     moe_dispatch_layout_noalloc keeps its counts in a fixed device array of the
 *     library, see there.)
 *   - Work is enqueued asynchronously on `stream` (0 = the null stream).  There is no
 *     host synchronisation and no device-to-host copy inside any call; stream order is
 *     the completion signal.  Buffers may be reused once later work on the stream runs.
 *   - Arguments are validated on the host before anything is enqueued; a failed check
 *     returns an error status and enqueues nothing.  A launch failure reported by the
 *     HIP runtime returns MOE_ERR_HIP.  No C++ exception crosses the ABI.
 *   - N == 0 (or rows == 0) is valid and enqueues nothing.
 *   - Non-finite logits or activations give unspecified (but memory-safe) results.
 *   - Index arrays are int32 (N * k < 2^31); byte offsets inside kernels are 64-bit.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* a size, pointer or combination of arguments is invalid   */
  MOE_ERR_UNSUPPORTED = 2, /* valid request outside what this library implements       */
  MOE_ERR_WORKSPACE = 3,   /* workspace pointer missing or smaller than required       */
  MOE_ERR_HIP = 4          /* the HIP runtime reported an error while enqueuing         */
} moe_status;

typedef enum {
  MOE_F32 = 0,
  MOE_BF16 = 1,
  MOE_FP8_E4M3 = 2 /* OCP e4m3fn: 1 sign, 4 exponent (bias 7), 3 mantissa bits, max 448 */
} moe_dtype;

/* Workspace query ids for moe_workspace_bytes(). */
typedef enum {
  MOE_OP_DISPATCH_LAYOUT = 0,
  MOE_OP_GROUPED_FFN = 1, /* includes the [rows, I] intermediate h                      */
  MOE_OP_EXPERT_GEMM = 2, /* moe_expert_gate_up / moe_expert_down: tile schedule (fp8 gate/up: and a bf16 copy of a) */
  MOE_OP_ROUTER = 3,      /* moe_router_logits: fp32 partial sums (N, H, E, a_dt = x_dt) */
  MOE_OP_EXPERT_DGRAD = 4 /* moe_expert_dgrad: tile schedule (N = rows, E)               */
} moe_op;

/* Limits of this implementation. */
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOPK 32
#define MOE_MAX_GROUPS 64
#define MOE_FP8_BLOCK 128 /* columns per fp32 scale of an fp8 row */

/*
 * moe_router_logits -- z = x W_r^T, the router's logits for every token and expert.
 *
 * Definition: "EP / DeepEP explanation" page, section 2 (the router maps each token's
 * hidden state to logits z in R^{N x E}); "MoE part 4" page, section 4.2 (the router's
 * top-k then reads them).
 *
 *   x     [N, H] of x_dt (MOE_BF16 or MOE_F32).
 *   w_r   [E, H] of x_dt: row e holds expert e's H weights (a linear layer's weight).
 *   z     [N, E] fp32 out: z[t, e] = sum_h x[t, h] * w_r[e, h], accumulated in fp32.
 *   ws    workspace of moe_workspace_bytes(MOE_OP_ROUTER, N, H, 0, E, 0, x_dt) bytes (may
 *         be 0: then ws may be NULL).  bf16 operands with H % 128 == 0 and E % 4 == 0 run on
 *         the matrix cores with K split into parts whose fp32 partial sums the workspace
 *         holds; they are added in a fixed order, so z is the same on every call.
 * x, w_r, z (and a non-empty ws) must be 16-byte aligned.  E <= MOE_MAX_EXPERTS.
 */
moe_status moe_router_logits(const void* x, moe_dtype x_dt, int N, int H, const void* w_r, int E, float* z,
                             void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_route -- router top-k with optional bias and group limit, renormalised gates.
 *
 * Definition: "EP / DeepEP explanation" page, section 2 (logits z, index set I_t, gates
 * g_{t,e}); "MoE part 4" page, section 4.2 (top-k with a per-expert correction bias,
 * grouped top-k, renormalisation); "Wide EP" page, section "Group-limited routing" (pick
 * groups first, then the top-k experts inside the allowed groups).
 *
 *   z          [N, E] fp32 router logits.
 *   bias       [E] fp32 added to every token's logits before selection and gating, or NULL.
 *   n_group, topk_group
 *              0, 0 = no group limit.  Otherwise the experts form n_group contiguous
 *              groups of E / n_group; a group's score is its largest biased logit; each
 *              token keeps the topk_group best groups (equal scores: lower group id).
 *   topk_idx   [N, k] int32 out: slot j is the j-th largest allowed biased logit; equal
 *              logits go to the lower expert index; +0 and -0 compare equal.
 *   topk_gate  [N, k] fp32 out: g_{t,j} = exp(z'_j - z'_0) / sum_j' exp(z'_j' - z'_0),
 *              z' the biased logits of the selected experts (softmax over all experts,
 *              restricted to I_t and renormalised).
 * Requires 1 <= k <= min(E, 32), E <= 1024; with groups: n_group <= 64, E % n_group == 0,
 * 1 <= topk_group <= n_group and k <= topk_group * E / n_group.
 */
moe_status moe_route(const float* z, int N, int E, int k, const float* bias, int n_group,
                     int topk_group, int32_t* topk_idx, float* topk_gate, hipStream_t stream);

/*
 * moe_dispatch_layout -- expert histogram, offsets and the three index maps.
 *
 * Definition: "EP / DeepEP explanation" page, section 2 (n_e), section 3 (bucket tokens
 * by target expert, metadata built on the GPU without host sync) and section 6 (token ->
 * send position, send position -> expert-local position, return position -> token).
 * Slot s = t * k + j names the pair (token t, its j-th expert).
 *
 *   topk_idx   [N * k] int32 expert ids in [0, E).  An id outside [0, E) is not counted
 *              and its send_pos is set to -1.
 *   n_e        [E] int32 out: rows per expert.
 *   offsets    [E + 1] int32 out: exclusive prefix sum of n_e (offsets[E] = valid pairs).
 *   send_pos   [N * k] int32 out: row of slot s in the expert-ordered buffer.  Rows of one
 *              expert are ordered by ascending slot (hence ascending token).
 *              Expert-local position = send_pos[s] - offsets[topk_idx[s]].
 *   src_slot   [N * k] int32 out: src_slot[send_pos[s]] = s (the return map); entries
 *              at rows >= offsets[E] are left untouched.
 *   ws         workspace of at least moe_workspace_bytes(MOE_OP_DISPATCH_LAYOUT, N, 0,
 *              0, E, k, 0) bytes.
 * Deterministic: no atomic operation's order reaches an output.
 */
moe_status moe_dispatch_layout(const int32_t* topk_idx, int N, int k, int E, int32_t* n_e,
                               int32_t* offsets, int32_t* send_pos, int32_t* src_slot, void* ws,
                               size_t ws_bytes, hipStream_t stream);

/*
 * moe_dispatch_layout_noalloc -- moe_dispatch_layout with no workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments (minus ws), outputs and determinism.
 *
 * The per-chunk expert counts go to a fixed array of MOE_LAYOUT_SCRATCH_BYTES in device
 * memory that the library holds on each device it runs on until the process ends.  No HIP
 * allocation is made.  Sizes whose count table exceeds it, i.e.
 * moe_workspace_bytes(MOE_OP_DISPATCH_LAYOUT, N, 0, 0, E, k, 0) > MOE_LAYOUT_SCRATCH_BYTES
 * (never for E <= 256; for E = 1024 once N * k exceeds 2^20), return MOE_ERR_WORKSPACE
 * before anything is enqueued.  Every call on one device shares that device's array:
 * calls that overlap in time on one device (two streams, two threads) race and must be
 * ordered by the caller.  Nothing has to be cleared between calls.
 */
#define MOE_LAYOUT_SCRATCH_BYTES (4u << 20)
moe_status moe_dispatch_layout_noalloc(const int32_t* topk_idx, int N, int k, int E, int32_t* n_e,
                                       int32_t* offsets, int32_t* send_pos, int32_t* src_slot,
                                       hipStream_t stream);

/*
 * moe_permute -- x_perm[send_pos[t * k + j]] = x[t] (the local stand-in of dispatch).
 *
 * Definition: "EP / DeepEP explanation" page, section 3 (tokens bucketed by expert into a
 * layout the grouped GEMM can use) and section 6 (an fp8 payload's scales share the
 * token's index); "MoE part 4" page, section 4 (permute by expert).
 *
 *   x          [N, H] of x_dt (MOE_F32 or MOE_BF16).
 *   send_pos   [N * k] int32 from moe_dispatch_layout; slots with send_pos < 0 are skipped.
 *   x_perm     [N * k, H] of perm_dt out.  perm_dt == x_dt copies rows.  perm_dt ==
 *              MOE_FP8_E4M3 (x_dt must be MOE_BF16 or MOE_F32) quantizes each token once
 *              per 128-column block: s = fp32(amax / 448) (1 when amax = 0),
 *              q = e4m3(fp32(x / s)) with round-to-nearest-even and saturation at 448,
 *              and writes k copies.
 *   perm_scale [N * k, H / 128] fp32 out, the block scales of each row (fp8 only, else
 *              ignored and may be NULL).
 * Requires H * sizeof(x_dt) % 16 == 0; H % 128 == 0 for fp8.
 */
moe_status moe_permute(const void* x, moe_dtype x_dt, int N, int H, int k,
                       const int32_t* send_pos, void* x_perm, moe_dtype perm_dt, float* perm_scale,
                       hipStream_t stream);

/*
 * moe_quantize_fp8 -- the per-(row, 128-column block) e4m3 quantization of moe_permute
 * applied to every row of a matrix in place order (used to quantize expert weights).
 *
 *   x [rows, cols] of x_dt (MOE_BF16 or MOE_F32) -> q [rows, cols] uint8 codes and
 *   scale [rows, cols / 128] fp32.  Requires cols % 128 == 0.
 */
moe_status moe_quantize_fp8(const void* x, moe_dtype x_dt, int64_t rows, int cols, uint8_t* q,
                            float* scale, hipStream_t stream);

/*
 * moe_dequantize_fp8 -- the values of e4m3 codes with their block scales, as bf16.
 *
 * Definition: the block-scaled fp8 format of moe_quantize_fp8 (value = code times the fp32
 * scale of its row's 128-column block; "EP / DeepEP explanation" page, section 10, and
 * "DeepEP" page, section 7: fp8 payload with per-block scales).  Each value is the fp32
 * product of the decoded code and the scale, rounded to the nearest bf16 (even on ties); the
 * NaN codes give NaN.
 *
 *   q [rows, cols] uint8 codes, scale [rows, cols / 128] fp32 -> out [rows, cols] bf16.
 *   Requires cols % 128 == 0 and rows * cols / 8 < 2^31 (MOE_ERR_UNSUPPORTED otherwise);
 *   q and out 16-byte aligned (MOE_ERR_INVALID_ARG otherwise).  rows == 0 returns MOE_OK.
 */
moe_status moe_dequantize_fp8(const uint8_t* q, const float* scale, int64_t rows, int cols, void* out,
                              hipStream_t stream);

/*
 * moe_grouped_ffn -- every expert's SwiGLU FFN on its rows, as grouped GEMMs.
 *
 * Definition: "MoE part 4" page, section 2 (one launch for many expert GEMMs with
 * differing row counts; it does not change the layer's mathematics) and section 4.1 (an
 * expert is FC1 -> activation -> FC2).  For each expert e and its rows
 * [offsets[e], offsets[e+1]) of the expert-ordered buffer a:
 *
 *     h   = silu(a W_gate,e^T) * (a W_up,e^T),   silu(v) = v / (1 + exp(-v))
 *     out = h W_down,e^T
 *
 *   a         [rows, H] of a_dt: MOE_F32, MOE_BF16 or MOE_FP8_E4M3 (then a_scale
 *             [rows, H / 128] fp32 holds its block scales).
 *   offsets   [E + 1] int32 device array (from moe_dispatch_layout).  Rows at or beyond
 *             offsets[E] are not computed.  A shared expert is one more call with E = 1
 *             and offsets = {0, N} on x.
 *   w13       [E, 2I, H]: rows 0..I-1 of each expert are W_gate, rows I..2I-1 W_up.
 *   w2        [E, H, I]: W_down.
 *             Weights are of a_dt's kind: MOE_F32 with f32 activations, MOE_BF16 with
 *             bf16, MOE_FP8_E4M3 with fp8 (w13_scale [E, 2I, H / 128] and w2_scale
 *             [E, H, I / 128] fp32 block scales, one per output row and 128 columns).
 *   out       [rows, H] of out_dt (MOE_F32 for f32 layers, else MOE_BF16).
 *   ws        workspace of moe_workspace_bytes(MOE_OP_GROUPED_FFN, ...) bytes; it holds
 *             the intermediate h [rows, I] (fp32 for f32 layers, else bf16) and, for fp8
 *             layers, a bf16 copy of a.
 * Accumulation is fp32.  fp8 layers: the gate/up GEMM at decode sizes (at most 16 rows per
 * expert on average) sums each 128-wide K block of code products in fp32, then scales it by
 * the product of the two block scales; above that, each fp8 operand value is its code times
 * its block scale rounded to the nearest bf16 (relative error at most 2^-8 per value), and the
 * products are summed in fp32.  The down projection reads bf16 h against fp8 W_down the same
 * way.
 * Requires H % 128 == 0 and I % 128 == 0.
 */
moe_status moe_grouped_ffn(const void* a, const float* a_scale, moe_dtype a_dt,
                           const int32_t* offsets, int E, int rows, int H, int I, const void* w13,
                           const float* w13_scale, const void* w2, const float* w2_scale, void* out,
                           moe_dtype out_dt, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_expert_gate_up / moe_expert_down -- the two grouped GEMMs of moe_grouped_ffn as
 * separate calls (same definitions and argument meanings).  h is [rows, I], fp32 for f32
 * layers and bf16 otherwise.  ws needs moe_workspace_bytes(MOE_OP_EXPERT_GEMM, ...) with
 * the call's a_dt (fp8: the tile schedule and a bf16 copy of a, rows x H; MOE_ERR_WORKSPACE
 * when smaller).
 */
moe_status moe_expert_gate_up(const void* a, const float* a_scale, moe_dtype a_dt,
                              const int32_t* offsets, int E, int rows, int H, int I,
                              const void* w13, const float* w13_scale, void* h, void* ws,
                              size_t ws_bytes, hipStream_t stream);
moe_status moe_expert_down(const void* h, moe_dtype h_dt, const int32_t* offsets, int E, int rows,
                           int I, int H, const void* w2, moe_dtype w2_dt, const float* w2_scale,
                           void* out, moe_dtype out_dt, void* ws, size_t ws_bytes,
                           hipStream_t stream);

/*
 * moe_expert_gate_up_gathered -- moe_expert_gate_up with the permute folded into the
 * operand loads: row r of the expert-ordered operand is read straight from x, token
 * src_slot[r] / k, so the permuted copy is never written.
 *
 * Definition: "EP / DeepEP explanation" page, section 3 (the dispatch sends each token's
 * row to the slots of its selected experts) and "MoE part 4" page, section 2 (the grouped
 * GEMM over the expert-ordered rows); the result equals moe_permute followed by
 * moe_expert_gate_up on the same rows, bit for bit.
 *
 *   x         [N, H] bf16 tokens (x_dt must be MOE_BF16).
 *   src_slot  [rows] int32 device array from moe_dispatch_layout: row r holds slot t*k + j.
 *             A token index outside [0, N) is clamped into it (no fault; that row's result
 *             is then meaningless).
 *   k, N      slots per token and number of tokens.
 *   offsets, E, rows, H, I, w13, h, ws: as for moe_expert_gate_up.
 * Requires H % 128 == 0, I % 128 == 0 and N * H * 2 < 2^32 (MOE_ERR_UNSUPPORTED otherwise).
 */
moe_status moe_expert_gate_up_gathered(const void* x, moe_dtype x_dt, int N, const int32_t* src_slot,
                                       int k, const int32_t* offsets, int E, int rows, int H, int I,
                                       const void* w13, void* h, void* ws, size_t ws_bytes,
                                       hipStream_t stream);

/*
 * moe_expert_gate_up_gathered_shared / moe_expert_down_shared -- the routed grouped GEMMs
 * with the shared expert as one more segment of the same launch.
 *
 * Definition: "EP / DeepEP explanation" page, section 2 (the layer output adds a shared
 * branch that every token takes, with gate 1) and "MoE part 4" page, section 2 (one grouped
 * launch over all segments).  Rows [0, rows) are the routed rows, exactly as in
 * moe_expert_gate_up_gathered and moe_expert_down; rows [rows, rows + n) are the shared
 * expert's, one per token: row rows + t takes token t of x (gate/up) or row rows + t of h
 * (down), with the shared weights.  The shared rows' results equal a separate
 * moe_expert_gate_up / moe_expert_down with E = 1 on all n tokens.
 *
 *   gate/up:  x [N, H] bf16; src_slot, k, offsets, E, rows, H, I, w13 as for
 *             moe_expert_gate_up_gathered; shared_w13 [2*I, H] bf16 (W_gate rows, then
 *             W_up rows); h [rows + N, I] bf16 (shared rows last); n = N.
 *             au [rows + N, 2I] bf16, or NULL: when given, the gate and up pre-activations of
 *             every row as well (gate in columns 0..I-1, up in I..2I-1; the training forward
 *             keeps them for moe_swiglu_backward instead of moe_expert_gate_up_preact).
 *   down:     h [rows + n_shared, I] bf16; w2 [E, H, I] and shared_w2 [H, I] bf16;
 *             out [rows + n_shared, H] bf16 (the shared rows last: pass out + rows * H to
 *             moe_combine as shared_out).
 *             src_slot [rows] and topk_gate [rows] (the layout's map and the router's gates,
 *             slot t*k+j): when both are given the down epilogue multiplies routed row r by
 *             its gate topk_gate[src_slot[r]] before rounding, so moe_combine is then called
 *             with topk_gate = NULL.  This is the weighted sum of "MoE part 4" page, section 4
 *             with its multiply moved into the GEMM (section 4.1: fused MoE kernels take the
 *             routing metadata into the expert GEMM).  Slots outside [0, rows) are clamped.
 *             Both NULL: unscaled outputs.  One NULL: MOE_ERR_INVALID_ARG.
 *   ws        >= moe_workspace_bytes(MOE_OP_EXPERT_GEMM, rows + n, H, I, E + 1, 1, MOE_BF16).
 * bf16 only; requires E < MOE_MAX_EXPERTS, H % 128 == 0, I % 128 == 0 and N * H * 2 < 2^32
 * (MOE_ERR_UNSUPPORTED otherwise).  rows + n == 0 returns MOE_OK without launching.
 *
 * moe_expert_gate_up_gathered_shared_e4m3 / moe_expert_down_shared_e4m3 -- the same launches
 * with e4m3 weights (an fp8 layer above decode sizes): w13 [E, 2I, H] and shared_w13 [2I, H]
 * (or w2 [E, H, I] and shared_w2 [H, I]) uint8 codes, w13_scale [E, 2I, H / 128] and
 * shared_w13_scale [2I, H / 128] (w2_scale [E, H, I / 128], shared_w2_scale [H, I / 128])
 * fp32 block scales.  x [N, H] bf16 holds the tokens' fp8 payload as values
 * (moe_quantize_fp8 then moe_dequantize_fp8 of x: each token quantized once, its k rows and
 * its shared row gathered from the same values).  Each weight value is its code times its
 * block scale rounded to bf16; products are summed in fp32.  No au, no gates in the epilogue.
 * Same requirements and workspace; scales missing: MOE_ERR_INVALID_ARG.
 */
moe_status moe_expert_gate_up_gathered_shared(const void* x, moe_dtype x_dt, int N, const int32_t* src_slot,
                                              int k, const int32_t* offsets, int E, int rows, int H, int I,
                                              const void* w13, const void* shared_w13, void* h, void* au,
                                              void* ws, size_t ws_bytes, hipStream_t stream);
moe_status moe_expert_gate_up_gathered_shared_e4m3(const void* x, int N, const int32_t* src_slot, int k,
                                                   const int32_t* offsets, int E, int rows, int H, int I,
                                                   const uint8_t* w13, const float* w13_scale,
                                                   const uint8_t* shared_w13, const float* shared_w13_scale,
                                                   void* h, void* ws, size_t ws_bytes, hipStream_t stream);
moe_status moe_expert_down_shared_e4m3(const void* h, const int32_t* offsets, int E, int rows, int n_shared,
                                       int I, int H, const uint8_t* w2, const float* w2_scale,
                                       const uint8_t* shared_w2, const float* shared_w2_scale, void* out,
                                       void* ws, size_t ws_bytes, hipStream_t stream);
moe_status moe_expert_down_shared(const void* h, moe_dtype h_dt, const int32_t* offsets, int E, int rows,
                                  int n_shared, int I, int H, const void* w2, const void* shared_w2,
                                  const int32_t* src_slot, const float* topk_gate, void* out,
                                  moe_dtype out_dt, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_combine -- y_t = sum_{j<k} g_{t,j} * expert_out[send_pos[t*k+j]] (+ shared_out_t).
 *
 * Definition: "EP / DeepEP explanation" page, section 2 (y_t, with an optional shared
 * branch) and section 3 (the source sums the returned rows with the gates in original
 * token order); "DeepEP" page, section 7 (the combine sums in higher precision).
 *
 *   expert_out [rows, H] of eo_dt (MOE_F32 or MOE_BF16), rows >= max(send_pos) + 1.
 *   send_pos   [N * k] int32; slots with send_pos < 0 are skipped.
 *   topk_gate  [N, k] fp32, or NULL when the expert outputs already carry their gates
 *              (moe_expert_down_shared with gates): then the rows are summed with weight 1.
 *   shared_out [N, H] of eo_dt, added with gate 1, or NULL.
 *   y          [N, H] of y_dt (MOE_F32 or MOE_BF16) out.
 * The sum is fp32 in the order j = 0..k-1, then the shared row; one rounding to y_dt.
 * Requires H * sizeof(eo_dt) % 16 == 0 and H % 8 == 0.
 */
moe_status moe_combine(const void* expert_out, moe_dtype eo_dt, int N, int H, int k,
                       const int32_t* send_pos, const float* topk_gate, const void* shared_out,
                       void* y, moe_dtype y_dt, hipStream_t stream);

/*
 * moe_stream_probe -- a measurement utility, not a step of the layer: the achievable HBM
 * rate of combine's access mix.  dst[i] = sum over j < ratio of src[j * n16 + i], each
 * 16-byte word added as four 32-bit integers (wrapping).
 *
 *   src   [ratio * n16] 16-byte words, dst [n16] 16-byte words (16-byte aligned).
 *   ratio in {1, 2, 4, 8, 9, 16} (MOE_ERR_UNSUPPORTED otherwise); 9 is the DeepSeek-V3-shaped
 *         combine's mix: 8 expert rows and the shared expert's row read per row written.
 * Every access is sequential, so the rate (ratio + 1) * n16 * 16 bytes over the kernel time is
 * the ceiling for a kernel that reads ratio rows per row it writes.
 */
moe_status moe_stream_probe(const void* src, size_t n16, int ratio, void* dst, hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * Backward pass (training).  "DeepSeek MoE: EP and FSDP guide": the backward of the layer
 * mirrors its forward -- the backward of dispatch is combine (and that of combine a
 * dispatch of dy, scaled by the gates) -- and each expert keeps its own weight gradients.
 * Top-k selection is piecewise constant, so gradients reach the router through the gates
 * only.  For the bf16 layer with upstream gradient dy [N, H]:
 *
 *   moe_combine_backward        d_expert_out, d_gate
 *   moe_expert_gate_up_preact   the gate/up pre-activations au = x W13_e^T (recomputed)
 *   moe_expert_dgrad            dh = d_expert_out W_down,e
 *   moe_swiglu_backward         d_au = (da, du), and h recomputed from au
 *   moe_expert_wgrad            dW_down,e = d_expert_out_e^T h_e,  dW13_e = d_au_e^T x_e
 *   moe_expert_dgrad            d_perm = d_au W13_e
 *   moe_router_backward         dz on the selected logits, dW_r
 *   moe_router_input_grad       dx_r = sum_j dz_tj W_r[e_tj] (+ the shared expert's input gradient)
 *   moe_combine (gates = NULL, rows of d_perm, + dx_r)
 *                               dx = dx_r + sum_j d_perm[send_pos[t,j]]
 * (the shared expert: the same GEMMs with E = 1 on all N tokens and d_out = dy).
 * ------------------------------------------------------------------------------------ */

/*
 * moe_combine_backward -- gradients of moe_combine's weighted sum.
 *
 * Definition: "EP / DeepEP explanation" page, section 2 (y_t = sum_j g_tj o_tj) and the
 * chain rule: d_expert_out[send_pos[t*k+j]] = g_tj dy_t and d_gate[t*k+j] = <dy_t,
 * expert_out[send_pos[t*k+j]]> (fp32 sum).  Slots with send_pos < 0 get d_gate 0.
 *   dy, expert_out, d_expert_out: dt (MOE_BF16 or MOE_F32); dy [N, H]; the others [rows, H].
 * Requires H * sizeof(dt) % 16 == 0.
 */
moe_status moe_combine_backward(const void* dy, moe_dtype dt, int N, int H, int k, const int32_t* send_pos,
                                const float* topk_gate, const void* expert_out, void* d_expert_out, float* d_gate,
                                hipStream_t stream);

/*
 * moe_expert_gate_up_preact -- the gate/up GEMM without its activation: au[r] = a_r W13_e^T
 * ([rows, 2I] bf16: the gate pre-activations in columns 0..I-1, the up ones in I..2I-1),
 * a_r = x[src_slot[r] / k] (src_slot given) or row r of x (src_slot NULL: x [rows, H]).
 * Definition: "MoE part 4" page, section 4.1 (FC1 before the activation).  bf16 only; ws as
 * for moe_expert_gate_up; H % 128 == 0, I % 128 == 0.
 */
moe_status moe_expert_gate_up_preact(const void* x, moe_dtype x_dt, int N, const int32_t* src_slot, int k,
                                     const int32_t* offsets, int E, int rows, int H, int I, const void* w13, void* au,
                                     void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_swiglu_backward -- for h = silu(a) * u: da = dh u s(a) (1 + a (1 - s(a))) and
 * du = dh a s(a), s the logistic function (the chain rule on the SwiGLU of "MoE part 4" page,
 * section 4.1).  au [rows, 2I] and dh [rows, I] bf16 in; d_au [rows, 2I] bf16 out (da in
 * columns 0..I-1, du in I..2I-1); h [rows, I] bf16 out = silu(a) u, or NULL.  I % 8 == 0.
 */
moe_status moe_swiglu_backward(const void* au, const void* dh, int rows, int I, void* d_au, void* h,
                               hipStream_t stream);

/*
 * moe_expert_dgrad -- out[r, :] = dC[r, :] W_e for the rows r of segment e (the input
 * gradient of an expert GEMM; "MoE part 4" page, section 2: one grouped launch over ragged
 * segments).  dC [rows, K] bf16; W [E, K, N] bf16 (the forward weight as stored: w2 with
 * K = H, N = I gives dh; w13 with K = 2I, N = H gives the input gradient); out [rows, N]
 * bf16; fp32 accumulation.  ws >= moe_workspace_bytes(MOE_OP_EXPERT_DGRAD, rows, 0, 0, E,
 * 0, 0).  Requires K % 32 == 0, N % 128 == 0, E <= MOE_MAX_EXPERTS.
 */
moe_status moe_expert_dgrad(const void* dC, const int32_t* offsets, int E, int rows, int K, int N, const void* w,
                            void* out, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_expert_wgrad -- dW_e = A_e^T B_e, the weight gradient of every expert over its own
 * rows ("DeepSeek MoE: EP and FSDP guide": each expert keeps its gradients).  A [rows, M]
 * bf16; B rows [.., N] bf16: row r of the product uses row r of b, or row b_rows[r] / b_div
 * (clamped into [0, b_nrows)) when b_rows is given (x through the layout's src_slot map);
 * dW [E, M, N] of dw_dt (MOE_F32 or MOE_BF16), fp32 accumulation in row order; an expert
 * without rows gets zeros.  Requires M % 128 == 0, N % 128 == 0.
 */
moe_status moe_expert_wgrad(const void* a, int M, const void* b, int N, const int32_t* b_rows, int b_div,
                            int b_nrows, const int32_t* offsets, int E, int rows, void* dw, moe_dtype dw_dt,
                            hipStream_t stream);

/*
 * moe_router_input_grad -- the router's share of the input gradient, through z = x W_r^T.
 *
 * Definition: "EP / DeepEP explanation" page, section 2 (z = the router's logits of x) and
 * the chain rule: dx_t = sum_{j<k} dz_tj W_r[topk_idx[t,j]] (+ rest_t), fp32 sum in slot order
 * then rest, one rounding to dx_dt.  The same gather-sum as moe_combine over the E rows of
 * W_r, each row read by about N k / E slots, so its loads stay in the caches (moe_combine
 * marks its loads as read once).
 *   w_r [E, H] of w_dt (MOE_BF16 or MOE_F32); topk_idx [N, k] int32 in [0, E) (from
 *   moe_route; negative ids are skipped, ids >= E are undefined behaviour); dz [N, k] fp32
 *   (from moe_router_backward); rest [N, H] of w_dt or NULL; dx [N, H] of dx_dt out.
 * Requires H % 8 == 0 and H * sizeof(w_dt) % 16 == 0; 16-byte aligned w_r, rest and dx.
 */
moe_status moe_router_input_grad(const void* w_r, moe_dtype w_dt, int N, int E, int H, int k,
                                 const int32_t* topk_idx, const float* dz, const void* rest, void* dx,
                                 moe_dtype dx_dt, hipStream_t stream);

/*
 * moe_router_backward -- gradients through the renormalised gates into the router.
 *
 * Definition: "EP / DeepEP explanation" page, section 2 and "MoE part 4" page, section 4.2
 * (gates = softmax over the selected logits): dz[s] = g_s (d_gate_s - sum_j g_tj d_gate_tj)
 * over token t's k slots (fp32); z = x W_r^T then gives dW_r[e] = sum over the slots s
 * routed to e of dz[s] x_{s / k}, summed in the layout's row order (offsets, src_slot from
 * moe_dispatch_layout; rows = offsets[E]).  The input gradient sum_j dz_tj W_r[e_tj] is a
 * moe_combine over the rows of W_r with send_pos = topk_idx and gates dz.
 *   x [N, H] of x_dt (MOE_BF16 or MOE_F32); dz [N, k] fp32 out; dw_r [E, H] of dw_dt out.
 */
moe_status moe_router_backward(const float* topk_gate, const float* d_gate, int N, int k, const int32_t* offsets,
                               const int32_t* src_slot, int E, int rows, const void* x, moe_dtype x_dt, int H,
                               float* dz, void* dw_r, moe_dtype dw_dt, hipStream_t stream);

/*
 * moe_workspace_bytes -- bytes of workspace `op` needs for these sizes (0 if none).
 * For MOE_OP_GROUPED_FFN and MOE_OP_EXPERT_GEMM pass the GEMMs' row count as N.
 * Arguments that an op does not use are ignored.  Returns 0 for invalid sizes.
 */
size_t moe_workspace_bytes(int op, int N, int H, int I, int E, int k, int a_dt);

/* Static description of a status code. */
const char* moe_status_str(moe_status status);

/* Library version string ("major.minor.patch"). */
const char* moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
