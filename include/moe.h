/*
 * moe.h - C ABI of libmoe: one GPU's share of a Mixture-of-Experts
 * expert-parallel layer on AMD Instinct MI355X (gfx950).
 *
 * The layer is the one the expert-parallel overlap pages describe: tokens are
 * dispatched to their experts, each expert runs its FFN, and the results are
 * combined back per token (skill card page 1, "What it is"); the backward pass
 * runs combine -> expert MLP -> dispatch, with the MLP's activation gradient (D)
 * computed before its weight gradient (W) so the latter can be deferred (1F1B
 * note page 2, "MoE 1F1B overlap" and the backward chain under "how the 8 ops
 * are split"; skill card page 1, delay_wgrad_compute).  Two micro-batches run
 * on two streams so that one's dispatch/combine overlaps the other's expert
 * GEMMs (page 2, "MoE 1F1B overlap": two streams + two micro-batches).
 * The pages leave the routing function and FFN type open; this library uses
 * top-K softmax routing (or forced balance, page 1 "HybridEP benchmark":
 * "Routing: force balance") and SwiGLU experts.
 *
 * Conventions (all entry points):
 *  - Pointers are DEVICE pointers unless stated otherwise; the caller owns
 *    every buffer.  The library allocates no device memory: scratch space is
 *    the caller's `ws` of at least moe_workspace_bytes() bytes.
 *  - Every call validates its arguments on the host before any launch.  On a
 *    validation failure it returns a negative MOE_ERR_* code, launches
 *    nothing and writes nothing; moe_last_error() then describes the problem.
 *  - Every call is asynchronous on the given stream and never synchronises the
 *    device.  Buffers must stay alive until that stream's work completes (the
 *    free-input hazard the 1F1B note reports under "TP=1 bug", page 2).
 *  - Activations ("data" tensors) are in shape->dtype (MOE_BF16, MOE_F16 or
 *    MOE_F32).
 *    Logits, gates, gate gradients, logit gradients and weight gradients are
 *    always float32; indices and maps are int32.  Layouts are row-major.
 *  - Results are deterministic: the same inputs give bit-identical outputs,
 *    whatever the stream schedule.
 *  - HIP launch failures return MOE_ERR_HIP.  There is no silent fallback.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------- */
#define MOE_OK               0
#define MOE_ERR_NULL        -1   /* a required pointer is NULL                 */
#define MOE_ERR_SHAPE       -2   /* a size is outside the supported range      */
#define MOE_ERR_DTYPE       -3   /* dtype is not MOE_F32 / MOE_BF16 / MOE_F16  */
#define MOE_ERR_WORKSPACE   -4   /* workspace smaller than required            */
#define MOE_ERR_HIP         -5   /* a HIP runtime call or launch failed        */
#define MOE_ERR_UNSUPPORTED -6   /* mode / flag combination not supported      */
#define MOE_ERR_ARG         -7   /* unknown mode or flag value                 */

/* ---- data types ---------------------------------------------------------- */
#define MOE_F32   0
#define MOE_BF16  1
#define MOE_F16   2   /* IEEE binary16 (the pages' other mixed precision, fp16
                         next to bf16): same matrix-core path as bf16, with
                         float32 accumulation and round-to-nearest-even stores */

/* ---- routing modes ------------------------------------------------------- */
/* Top-K over router logits = x . W_r (+ bias); gates = softmax over the K
 * selected logits (= softmax over all E renormalised over the selected). */
#define MOE_ROUTE_TOPK              0
/* Top-K over caller-given logits (same selection and gates). */
#define MOE_ROUTE_TOPK_FROM_LOGITS  1
/* Forced balance: slot k of token t goes to expert (t*K + k) mod E; the gates
 * are caller-given inputs and are not touched. */
#define MOE_ROUTE_FORCE_BALANCE     2

/* ---- accumulate bits ------------------------------------------------------ */
#define MOE_ACCUM_DX  1   /* moe_dispatch_bwd: add into dx instead of overwrite */
#define MOE_ACCUM_DW  2   /* moe_ffn_wgrad / moe_route_bwd: add into weight grads */

/* ---- moe_overlap_step flags ------------------------------------------------ */
#define MOE_STEP_SERIALIZE   1  /* everything on s_compute, forward then backward */
#define MOE_STEP_EAGER_WGRAD 2  /* wgrad right after dgrad (not after the other
                                   micro-batch's forward GEMMs)                   */
#define MOE_STEP_SKIP_WGRAD  4  /* leave the backward micro-batch's wgrad out: the
                                   caller issues moe_ffn_wgrad later (e.g. while the
                                   next layer's forward runs, page 1
                                   delay_wgrad_compute); its inputs (xp, a, dh,
                                   dyp, offsets of `bwd`) must then stay intact   */
#define MOE_STEP_FUSED_PERMUTE 8 /* fuse the permute into the expert GEMMs: the
                                   forward dispatch writes no xp, GEMM1 and the
                                   dW_gu part of wgrad read the token rows of x
                                   through pair_of_row (page 1 names the fused
                                   permute, moe_permute_fusion); xp of both
                                   micro-batches may be NULL, and `bwd` needs x
                                   and pair_of_row                                */
#define MOE_STEP_MID_WGRAD   16 /* the routed experts' wgrad between the two dgrad
                                   GEMMs (after dy_p -> dh, before dh -> dx_p)
                                   instead of last: on one GPU, where the dispatch
                                   backward is a local gather, this lets the wgrad's
                                   partial last round of tiles share the chip with
                                   the other stream's GEMMs.  Excludes EAGER_WGRAD
                                   and SKIP_WGRAD; results are unchanged           */
#define MOE_STEP_FUSED_COMBINE_BWD 32 /* the fused permute's mirror on the backward
                                   side: the combine backward writes only dgates
                                   (no dy_p); the dgrad's first GEMM gathers the
                                   dout rows through pair_of_row and scales them by
                                   the rows' gates, and writes ag = gate * a' (a'
                                   recomputed from the stored h); the wgrad's
                                   dW_down product takes the gathered dout rows
                                   and ag.  `bwd` needs ag [T*K,F] and pair_of_row;
                                   its dyp may be NULL.  The results match the
                                   unfused path within the numeric tolerance (the
                                   gate is applied in float32 instead of through a
                                   rounded dy_p), not bit for bit               */
#define MOE_STEP_PAIR_WGRAD 64 /* moe_overlap_steps: the routed experts' weight
                                 gradients of steps j and j + 1 in one launch
                                 (moe_ffn_wgrad_pair) in step j + 1, pairs
                                 formed from the first step on where step j + 1
                                 accumulates (MOE_ACCUM_DW) into the same dW
                                 buffers; the launch
                                 overwrites or accumulates as step j asks.
                                 Step j's backward micro-batch must stay intact
                                 until then (step j + 1 may not forward into
                                 its buffers); not with the fused permute or the
                                 fused combine backward, and not under stream
                                 capture (MOE_ERR_UNSUPPORTED) */
#define MOE_STEP_FUSED_SCATTER 128 /* the unpermute fused into GEMM2: its epilogue
                                 writes y by (token, slot) pair into the
                                 micro-batch's yp buffer (moe_expert_ffn_fwd_scatter),
                                 and the combine and the combine backward read
                                 a token's slots as one run (moe_combine_pairs,
                                 moe_combine_bwd_pairs).  Bit-identical results */
#define MOE_STEP_GROUP4_WGRAD 256 /* moe_overlap_steps: as MOE_STEP_PAIR_WGRAD with
                                 groups of four steps: the routed experts' weight
                                 gradients of steps j .. j + 3 in one launch
                                 (moe_ffn_wgrad_multi) in step j + 3, where steps
                                 j + 1 .. j + 3 accumulate; the deferred
                                 micro-batches must stay intact until then.
                                 Excludes MOE_STEP_PAIR_WGRAD */

/*
 * Layer shape.  T tokens of hidden size d; E experts routed over, of which the
 * local window [e_lo, e_lo + E_l) lives on this GPU; K experts per token; F is
 * the expert FFN width.  Supported: T >= 0, T*K < 2^31, 1 <= K <= min(E, 16),
 * 1 <= E <= 512, 1 <= E_l <= 256, 0 <= e_lo, e_lo + E_l <= E,
 * d and F multiples of 64 in [64, 16384].  reserved must be 0.
 * N (rows dispatched to the local window) is at most cap = T*K; it is only
 * known on the device (offsets[E_l]), so row buffers are sized to cap.
 */
typedef struct moe_shape {
  int64_t T, d, F, E, e_lo, E_l, K;
  int32_t dtype;
  int32_t reserved;
} moe_shape;

/* Bytes of workspace any single call below needs for this shape. */
size_t moe_workspace_bytes(const moe_shape* s);
/* Bytes of workspace moe_overlap_step needs (two micro-batches in flight). */
size_t moe_step_workspace_bytes(const moe_shape* s);
/* Rows per M-tile of the grouped GEMMs; tile_offsets are counted in these. */
int moe_tile_m(void);
/* Thread-local description of the last error (empty string if none). */
const char* moe_last_error(void);
/* Library version (major*10000 + minor*100 + patch). */
int moe_version(void);

/*
 * moe_route - routing (router scores, top-K selection, gates).
 * Passages: the router is the layer's first MoE scope, captured in a graph of
 * its own with the permutation plan (skill card page 1, "HybridEP benchmark":
 * Transformer Engine graph scopes moe_router and moe_preprocess, and "Routing:
 * force balance"); routing precedes the dispatch phase in the phase chain
 * attn -> dispatch -> mlp -> combine (1F1B note page 2, "how the 8 ops are
 * split").  The routing function itself is not given on the pages; top-K
 * softmax over router logits (gates renormalised over the selected experts)
 * is the reading used.
 *   x      [T,d] dtype        (MOE_ROUTE_TOPK only)
 *   W_r    [d,E] dtype        (MOE_ROUTE_TOPK only)
 *   bias   [E] f32 or NULL    (MOE_ROUTE_TOPK only; added to the logits, so it
 *                              affects selection and gates)
 *   logits [T,E] f32          written (TOPK), read (TOPK_FROM_LOGITS), unused
 *                              (FORCE_BALANCE, may be NULL)
 *   idx    [T,K] i32 written  selected experts, descending logit, ties -> lower
 *                              expert index
 *   gates  [T,K] f32          written (TOPK modes); caller input (FORCE_BALANCE,
 *                              may be NULL)
 *   ws/ws_bytes               workspace (TOPK)
 * Logits must be finite.
 */
int moe_route(const moe_shape* s, int mode, const void* x, const void* W_r,
              const float* bias, float* logits, int32_t* idx, float* gates,
              void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_dispatch - dispatch plan and permute (the local half of the token
 * all-to-all of page 1, "What it is").  A stable counting sort of the
 * (token, slot) pairs whose expert is local, in (t, k) order:
 *   idx          [T,K] i32 in   from moe_route
 *   counts       [E_l] i32 out  rows per local expert
 *   offsets      [E_l+1] i32 out exclusive prefix sum; offsets[E_l] = N
 *   row_of_pair  [T*K] i32 out  row of pair t*K+k, or -1 if its expert is not local
 *   pair_of_row  [T*K] i32 out  inverse map on rows [0,N); -1 on rows [N, T*K)
 *   tile_offsets [E_l+1] i32 out exclusive prefix sum of ceil(counts/moe_tile_m())
 *   x            [T,d] dtype in
 *   xp           [T*K,d] dtype out  xp[row_of_pair[t*K+k]] = x[t] (exact copy);
 *                                   rows >= N untouched.  NULL: the plan only
 *                                   (for the fused-permute calls below; x may
 *                                   then be NULL too)
 */
int moe_dispatch(const moe_shape* s, const void* x, const int32_t* idx,
                 int32_t* counts, int32_t* offsets, int32_t* row_of_pair,
                 int32_t* pair_of_row, int32_t* tile_offsets, void* xp,
                 void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_dispatch_noalloc - moe_dispatch for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same plan and permute, with identical results, but
 * the plan's scratch is a fixed device array inside the library instead of a
 * caller workspace, and the call allocates nothing.  Arguments as
 * moe_dispatch, without ws.
 *   Limit: the plan scratch, 2 * E_l * ceil(T*K / 2048) * 4 bytes (rounded up
 *   to 256), must fit moe_dispatch_noalloc_max_scratch() = 4 MiB (e.g. every
 *   E_l = 128 shape with T*K <= 8M pairs); larger shapes return
 *   MOE_ERR_WORKSPACE before anything is launched.
 *   Sharing: each GPU holds one copy of the array, from the first call on that
 *   device until the process ends; every call on a GPU uses that GPU's copy,
 *   so calls that overlap on one GPU (other streams, other host threads) race
 *   and must be ordered by the caller.  Nothing in the scratch needs to start
 *   at zero: each call writes every entry it reads.
 *   The first call on a device looks the array's address up (with that device
 *   current); errors of that lookup return MOE_ERR_HIP.
 */
int moe_dispatch_noalloc(const moe_shape* s, const void* x, const int32_t* idx,
                         int32_t* counts, int32_t* offsets, int32_t* row_of_pair,
                         int32_t* pair_of_row, int32_t* tile_offsets, void* xp,
                         hipStream_t stream);
/* Bytes of the fixed scratch array moe_dispatch_noalloc uses (4 MiB). */
size_t moe_dispatch_noalloc_max_scratch(void);

/*
 * moe_expert_ffn_fwd - the expert FFN computation that the token exchange is
 * overlapped with (skill card page 1, "What it is"), the mlp phase between
 * dispatch and combine (1F1B note page 2, "how the 8 ops are split").  The
 * pages do not give the expert type; a SwiGLU FFN is the reading used.  Per
 * local expert j (rows [offsets[j], offsets[j+1])):
 *   [g,u] = xp . W_gu[j]^T,  a = silu(g) * u,  y_p = a . W_down[j]^T
 *   xp [T*K,d], W_gu [E_l,2F,d] (rows [0,F) gate, [F,2F) up), W_down [E_l,d,F]
 *   h  [T*K,2F] out (g and u, saved for the backward), a [T*K,F] out,
 *   yp [T*K,d] out.  All dtype.  a is computed from g, u before rounding.
 *   offsets, tile_offsets from moe_dispatch.  Rows >= N are untouched.
 */
int moe_expert_ffn_fwd(const moe_shape* s, const void* xp, const int32_t* offsets,
                       const int32_t* tile_offsets, const void* W_gu,
                       const void* W_down, void* h, void* a, void* yp,
                       hipStream_t stream);

/*
 * moe_expert_ffn_fwd_gather - moe_expert_ffn_fwd with the permute fused into
 * GEMM1's operand loads (page 1 lists the fused permute, moe_permute_fusion,
 * among the options): row r of the product reads token pair_of_row[r] / K of
 * x [T,d] directly, so xp is never materialised.  Results are identical to
 * moe_dispatch (with xp) followed by moe_expert_ffn_fwd.  pair_of_row from
 * moe_dispatch; x must stay below 2^31 bytes.
 */
int moe_expert_ffn_fwd_gather(const moe_shape* s, const void* x,
                              const int32_t* pair_of_row, const int32_t* offsets,
                              const int32_t* tile_offsets, const void* W_gu,
                              const void* W_down, void* h, void* a, void* yp,
                              hipStream_t stream);

/*
 * moe_combine - unpermute and gate-weighted sum (page 1, "What it is":
 * combine).  out[t] = sum over local slots k, ascending, of
 * gates[t,k] * yp[row_of_pair[t*K+k]], accumulated in float32; a token with no
 * local slot gets 0.   yp [T*K,d], gates [T,K] f32, out [T,d].
 */
int moe_combine(const moe_shape* s, const void* yp, const float* gates,
                const int32_t* row_of_pair, void* out, hipStream_t stream);

/*
 * moe_expert_ffn_fwd_scatter - moe_expert_ffn_fwd with the unpermute half of
 * the combine fused into GEMM2's epilogue (page 1 lists the fused permute,
 * moe_permute_fusion; this is its scatter side): dispatched row r of the
 * product goes to row pair_of_row[r] of yq, so
 *   yq [T*K,d]:  yq[t*K+k] = the expert output of pair (t,k) for local pairs
 * (rows of non-local pairs are not written).  The values are those of
 * moe_expert_ffn_fwd's yp, bit for bit, at other rows.  xp, or, with xp NULL,
 * x [T,d] gathered through pair_of_row as moe_expert_ffn_fwd_gather does.
 * The gate-weighted sum stays in moe_combine_pairs: every token sums K rows,
 * and a sum in GEMM2's epilogue would need float atomics whose order varies
 * between runs.
 */
int moe_expert_ffn_fwd_scatter(const moe_shape* s, const void* xp, const void* x,
                               const int32_t* pair_of_row, const int32_t* offsets,
                               const int32_t* tile_offsets, const void* W_gu,
                               const void* W_down, void* h, void* a, void* yq,
                               hipStream_t stream);

/*
 * moe_combine_pairs - moe_combine over y by pair (yq from
 * moe_expert_ffn_fwd_scatter): out[t] = sum over local slots k, ascending, of
 * gates[t,k] * yq[t*K+k], in float32, one rounding; the same result as
 * moe_combine on the dispatched-row layout, bit for bit.  row_of_pair marks the
 * local slots (>= 0).
 */
int moe_combine_pairs(const moe_shape* s, const void* yq, const float* gates,
                      const int32_t* row_of_pair, void* out, hipStream_t stream);

/*
 * moe_combine_bwd - backward of combine (page 2, backward chain: combine's
 * backward first).  For each local pair (t,k) with row r:
 *   dyp[r] = gates[t,k] * dout[t];  dgates[t,k] = <dout[t], yp[r]> (f32)
 * dgates is 0 for non-local pairs.  dout [T,d], dyp [T*K,d] (rows >= N untouched).
 * dyp may be NULL: dgates only (the fused combine backward, whose GEMMs read
 * dout themselves: moe_ffn_dgrad_gather, moe_ffn_wgrad_fused).
 */
int moe_combine_bwd(const moe_shape* s, const void* dout, const void* yp,
                    const float* gates, const int32_t* row_of_pair, void* dyp,
                    float* dgates, hipStream_t stream);

/*
 * moe_combine_bwd_pairs - moe_combine_bwd reading y by pair (yq): dgates[t,k]
 * = <dout[t], yq[t*K+k]>; dyp is still written by dispatched row
 * (dyp[row_of_pair[t*K+k]] = gates[t,k] * dout[t]), as the dgrad reads it.
 * Bit-identical to moe_combine_bwd on the dispatched-row layout.
 */
int moe_combine_bwd_pairs(const moe_shape* s, const void* dout, const void* yq,
                          const float* gates, const int32_t* row_of_pair, void* dyp,
                          float* dgates, hipStream_t stream);

/*
 * moe_ffn_dgrad - the D of the W/D split (page 2, "MoE 1F1B overlap"): the
 * expert FFN's activation gradient, per local expert j:
 *   da = dyp . W_down[j];  with g, u from h and s = sigmoid(g):
 *   dg = da*u*s*(1 + g*(1-s)),  du = da*g*s;  dh = [dg, du];  dxp = dh . W_gu[j]
 *   dh [T*K,2F] out, dxp [T*K,d] out (dtype).
 *   ws/ws_bytes: workspace (bf16: the call stores transposed copies of W_down
 *   and W_gu there, so both products read K-contiguous operands).
 */
int moe_ffn_dgrad(const moe_shape* s, const void* dyp, const void* h,
                  const int32_t* offsets, const int32_t* tile_offsets,
                  const void* W_gu, const void* W_down, void* dh, void* dxp,
                  void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_ffn_wgrad - the W of the W/D split, deferrable (page 1,
 * delay_wgrad_compute).  Reduced over each expert's rows:
 *   dW_down[j] = sum_r dyp[r] (outer) a[r]   [E_l,d,F] f32
 *   dW_gu[j]   = sum_r dh[r]  (outer) xp[r]  [E_l,2F,d] f32
 * accumulate & MOE_ACCUM_DW: add to the existing values (gradient
 * accumulation); otherwise overwrite (an expert with no rows gets 0).
 */
int moe_ffn_wgrad(const moe_shape* s, const void* xp, const void* a,
                  const void* dh, const void* dyp, const int32_t* offsets,
                  float* dW_gu, float* dW_down, int accumulate, hipStream_t stream);

/*
 * moe_ffn_wgrad_pair - the weight gradients of two micro-batches of one shape
 * in one launch: the deferred W (page 1, delay_wgrad_compute) of one
 * micro-batch issued together with the next one's.  For each expert the
 * reduction runs over micro-batch A's rows (xp, a, dh, dyp, offsets), then
 * B's (xp2, a2, dh2, dyp2, offsets2), in one float32 accumulation:
 *   dW_down[j] (+)= sum_{r in A} dyp[r] (outer) a[r] + sum_{r in B} dyp2[r] (outer) a2[r]
 *   dW_gu[j]   (+)= sum_{r in A} dh[r] (outer) xp[r] + sum_{r in B} dh2[r] (outer) xp2[r]
 * so dW is read and written once for both (with gradient accumulation, half
 * the weight-gradient traffic of two moe_ffn_wgrad calls).  The sum equals
 * two moe_ffn_wgrad calls up to float32 rounding order, not bit for bit.
 * accumulate as moe_ffn_wgrad.  Layouts and sizes as moe_ffn_wgrad, for each
 * micro-batch.  Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_ARG (unknown
 * accumulate bits).
 */
int moe_ffn_wgrad_pair(const moe_shape* s, const void* xp, const void* a, const void* dh,
                       const void* dyp, const int32_t* offsets, const void* xp2,
                       const void* a2, const void* dh2, const void* dyp2,
                       const int32_t* offsets2, float* dW_gu, float* dW_down, int accumulate,
                       hipStream_t stream);

/* One micro-batch's weight-gradient operands (device pointers, layouts as
 * moe_ffn_wgrad). */
typedef struct moe_wgrad_ops {
  const void* xp;
  const void* a;
  const void* dh;
  const void* dyp;
  const int32_t* offsets;
} moe_wgrad_ops;

/*
 * moe_ffn_wgrad_multi - moe_ffn_wgrad_pair for n micro-batches, 1 <= n <= 4:
 * ops [n] (host array) in order; for each expert the reduction runs over
 * ops[0]'s rows, then ops[1]'s, and so on, in one float32 accumulation, so
 * dW is read and written once for all n (the deferred W of page 1,
 * delay_wgrad_compute, gathered over a group of steps).  n = 1 is
 * moe_ffn_wgrad.  Errors: MOE_ERR_NULL (an operand), MOE_ERR_SHAPE,
 * MOE_ERR_ARG (n out of range, unknown accumulate bits).
 */
int moe_ffn_wgrad_multi(const moe_shape* s, int n, const moe_wgrad_ops* ops, float* dW_gu,
                        float* dW_down, int accumulate, hipStream_t stream);

/*
 * moe_ffn_wgrad_gather - moe_ffn_wgrad with the fused permute: dW_gu reads
 * row r of its xp operand as token pair_of_row[r] / K of x [T,d].  Results
 * are identical to moe_ffn_wgrad on the materialised xp.  x must stay below
 * 2^31 bytes.
 */
int moe_ffn_wgrad_gather(const moe_shape* s, const void* x, const int32_t* pair_of_row,
                         const void* a, const void* dh, const void* dyp,
                         const int32_t* offsets, float* dW_gu, float* dW_down,
                         int accumulate, hipStream_t stream);

/*
 * moe_ffn_dgrad_gather - moe_ffn_dgrad with the combine backward fused in (the
 * mirror, on the backward side, of the fused permute that page 1 lists as
 * moe_permute_fusion): dy_p is never materialised.  Row r of the first
 * product reads token pair_of_row[r] / K of dout [T,d] and is scaled by that
 * pair's gate in float32:
 *   da = gates[p] * (dout[p / K] . W_down[j]),  p = pair_of_row[r];
 * dh and dxp as moe_ffn_dgrad.  It also writes, for the fused weight gradient,
 *   ag [T*K,F]:  ag[r] = gates[p] * silu(g) * u  (g, u from the stored h).
 * gates [T*K] f32 (the pairs' gates), pair_of_row from moe_dispatch.  dout
 * must stay below 2^31 bytes.  Results are within the numeric tolerance of
 * moe_combine_bwd + moe_ffn_dgrad (the gate is not rounded into dy_p first).
 */
int moe_ffn_dgrad_gather(const moe_shape* s, const void* dout, const int32_t* pair_of_row,
                         const float* gates, const void* h, const int32_t* offsets,
                         const int32_t* tile_offsets, const void* W_gu, const void* W_down,
                         void* dh, void* dxp, void* ag, void* ws, size_t ws_bytes,
                         hipStream_t stream);

/*
 * moe_ffn_wgrad_fused - the weight gradient of the fused combine backward:
 *   dW_down[j] = sum_r dout[pair_of_row[r] / K] (outer) ag[r]     (= dy_p^T . a)
 *   dW_gu[j]   = sum_r dh[r] (outer) xp[r]
 * with ag from moe_ffn_dgrad_gather.  xp NULL: the permute is fused too, and
 * dW_gu reads row r of its operand as token pair_of_row[r] / K of x [T,d].
 * accumulate as moe_ffn_wgrad.  dout (and x) must stay below 2^31 bytes.
 */
int moe_ffn_wgrad_fused(const moe_shape* s, const void* xp, const void* x,
                        const int32_t* pair_of_row, const void* ag, const void* dh,
                        const void* dout, const int32_t* offsets, float* dW_gu, float* dW_down,
                        int accumulate, hipStream_t stream);

/*
 * moe_route_bwd - backward of the top-K softmax gates and of the router
 * product (TOPK modes; returns MOE_ERR_UNSUPPORTED for FORCE_BALANCE, whose
 * gates are inputs with gradient dgates).  Passage: the backward chain runs
 * combine -> mlp -> dispatch -> attn, each phase returning the gradient of its
 * input (1F1B note page 2, "how the 8 ops are split"); the gates' gradient
 * (dgates, from moe_combine_bwd) reaches the router logits here, and the
 * router's weight gradient is accumulated like every weight gradient there
 * (accumulate_grad=True).  The router's input-gradient term, dlogits . W_r^T,
 * is not formed here: moe_dispatch_bwd adds it to dx in the same pass as the
 * dispatched rows, so dx is rounded once.
 *   dlogits[t, idx[t,j]] = g_j * (dg_j - sum_k g_k dg_k); other logits 0.  [T,E] f32
 *   dW_r = x^T . dlogits  [d,E] f32 (skipped when x or dW_r is NULL; with
 *   accumulate & MOE_ACCUM_DW added to the existing value)
 * With bf16 data, dW_r runs on the matrix cores: dlogits is split into two
 * bf16 terms per value (hi = bf16(v), lo = bf16(v - hi), about 16 significant
 * bits together), each chunk of tokens gives a float32 partial of x^T [hi|lo],
 * and the partials are summed in a fixed order (deterministic).  fp16 and f32
 * data use float32 vector arithmetic.
 */
int moe_route_bwd(const moe_shape* s, int mode, const float* dgates,
                  const float* gates, const int32_t* idx, const void* x,
                  float* dlogits, float* dW_r, int accumulate, void* ws,
                  size_t ws_bytes, hipStream_t stream);

/*
 * moe_dispatch_bwd - backward of dispatch (page 2, backward chain:
 * dispatch's backward after the MLP's):
 *   dx[t] = [dx[t] if accumulate & MOE_ACCUM_DX] + sum over local k of dxp[row(t,k)]
 *           [+ sum_k dlogits[t, idx[t,k]] * W_r[:, idx[t,k]]  if dlogits != NULL]
 * rounded once.  The router term is the input gradient of x . W_r; only the
 * K selected logits of a token have nonzero gradient.  idx and W_r are
 * required when dlogits is given.  dx [T,d] dtype.
 */
int moe_dispatch_bwd(const moe_shape* s, const void* dxp,
                     const int32_t* row_of_pair, const int32_t* idx,
                     const float* dlogits, const void* W_r, void* dx,
                     int accumulate, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---- shared expert -------------------------------------------------------- */
/*
 * The shared expert (page 1 lists the shared-expert overlap among the
 * options): one SwiGLU FFN of width F_s that every token passes through beside
 * the routed experts; its output is added to the combine's and its input
 * gradient to the dispatch backward's.  It is an expert over all T tokens in
 * token order with gate 1, so it runs on the same grouped GEMMs.
 *   W_gu_s [2F_s,d] (rows [0,F_s) gate, [F_s,2F_s) up), W_down_s [d,F_s] (dtype)
 *   F_s a multiple of 64 in [64, 16384]; workspace moe_shared_workspace_bytes.
 */
size_t moe_shared_workspace_bytes(const moe_shape* s, int64_t F_s);
/* h_s [T,2F_s], a_s [T,F_s], y_s [T,d] out: the FFN of x [T,d]. */
int moe_shared_expert_fwd(const moe_shape* s, int64_t F_s, const void* x,
                          const void* W_gu_s, const void* W_down_s, void* h_s, void* a_s,
                          void* y_s, void* ws, size_t ws_bytes, hipStream_t stream);
/* its D for output gradient dout [T,d]: dh_s [T,2F_s], dx_s [T,d] out
 * (same formulas as moe_ffn_dgrad). */
int moe_shared_expert_dgrad(const moe_shape* s, int64_t F_s, const void* dout,
                            const void* h_s, const void* W_gu_s, const void* W_down_s,
                            void* dh_s, void* dx_s, void* ws, size_t ws_bytes,
                            hipStream_t stream);
/* its W: dW_gu_s = dh_s^T . x [2F_s,d], dW_down_s = dout^T . a_s [d,F_s] (f32);
 * accumulate & MOE_ACCUM_DW adds to the existing values. */
int moe_shared_expert_wgrad(const moe_shape* s, int64_t F_s, const void* x, const void* a_s,
                            const void* dh_s, const void* dout, float* dW_gu_s,
                            float* dW_down_s, int accumulate, void* ws, size_t ws_bytes,
                            hipStream_t stream);

/* ---- two-micro-batch step ------------------------------------------------ */
/* One micro-batch's buffers (sizes as in the calls above). */
typedef struct moe_mb {
  /* forward */
  const void* x;
  float* logits;
  int32_t* idx;
  float* gates;
  int32_t* counts;
  int32_t* offsets;
  int32_t* row_of_pair;
  int32_t* pair_of_row;
  int32_t* tile_offsets;
  void* xp;
  void* h;
  void* a;
  void* yp;     /* [T*K,d]: by dispatched row, or by pair with MOE_STEP_FUSED_SCATTER */
  void* out;
  /* backward */
  const void* dout;
  void* dyp;
  float* dgates;
  float* dlogits;
  void* dh;
  void* dxp;
  void* dx;
  /* shared expert (used when moe_step.F_s > 0) */
  void* h_s;    /* [T,2F_s] forward, saved for the backward */
  void* a_s;    /* [T,F_s]  forward, saved for the backward */
  void* y_s;    /* [T,d]    forward */
  void* dh_s;   /* [T,2F_s] backward */
  void* dx_s;   /* [T,d]    backward */
  /* fused combine backward (MOE_STEP_FUSED_COMBINE_BWD) */
  void* ag;     /* [T*K,F]  gate-scaled activation for the dW_down product */
} moe_mb;

typedef struct moe_step {
  moe_shape shape;
  int32_t route_mode;     /* MOE_ROUTE_* */
  int32_t accumulate;     /* MOE_ACCUM_DW: add weight grads into dW_* */
  const void* W_r;        /* [d,E] (TOPK) */
  const float* bias;      /* [E] or NULL */
  const void* W_gu;       /* [E_l,2F,d] */
  const void* W_down;     /* [E_l,d,F] */
  float* dW_r;            /* [d,E] or NULL */
  float* dW_gu;           /* [E_l,2F,d] */
  float* dW_down;         /* [E_l,d,F] */
  const moe_mb* fwd;      /* micro-batch forwarded in this step, or NULL */
  const moe_mb* bwd;      /* micro-batch back-propagated in this step (its
                             forward buffers hold its forward results), or NULL */
  void* ws;               /* >= moe_step_workspace_bytes(&shape), or
                             moe_step_workspace_bytes_shared(&shape, F_s) */
  size_t ws_bytes;
  /* shared expert: F_s = 0 for none */
  int64_t F_s;
  const void* W_gu_s;     /* [2F_s,d] */
  const void* W_down_s;   /* [d,F_s] */
  float* dW_gu_s;         /* [2F_s,d] (accumulate as dW_gu) */
  float* dW_down_s;       /* [d,F_s] */
} moe_step;

/* Bytes of workspace moe_overlap_step needs with a shared expert of width F_s
 * (F_s = 0: moe_step_workspace_bytes). */
size_t moe_step_workspace_bytes_shared(const moe_shape* s, int64_t F_s);

/*
 * moe_overlap_step - forward of micro-batch `fwd` and backward of micro-batch
 * `bwd` in one step (1F1B note page 2, "MoE 1F1B overlap": two streams and two
 * micro-batches, D before W).  The two micro-batches share no buffers, so each
 * runs start to end on its own stream and the GPU interleaves their kernels
 * (one micro-batch's permutes beside the other's expert GEMMs, and each GEMM's
 * last partial wave of tiles beside the other stream's work):
 *   s_copy:    A.route, A.dispatch, A.ffn_fwd, A.combine
 *   s_compute: B.combine_bwd, B.route_bwd, B.dgrad, B.dispatch_bwd,
 *              B.wgrad (deferred: last, unless MOE_STEP_EAGER_WGRAD; with
 *              MOE_STEP_MID_WGRAD the dgrad is split and the order is
 *              dgrad(dy_p -> dh), wgrad, dgrad(dh -> dx_p), dispatch_bwd)
 * With a shared expert (F_s > 0) A's shared forward runs on s_compute and B's
 * shared D on s_copy, each beside the other micro-batch's chain; A's combine
 * adds y_s, B's dispatch backward adds dx_s, and B's shared W follows B's
 * routed W (both left out with MOE_STEP_SKIP_WGRAD).
 * On return, work on s_compute depends on everything the step issued, so a
 * caller that waits for s_compute sees all results.  Results are bit-identical
 * to MOE_STEP_SERIALIZE (all calls on s_compute in forward-then-backward order).
 * s_copy may equal s_compute (then the step is serialized).
 * The step only launches kernels and records/waits on events (s_copy forks
 * from and joins back to s_compute), so it may be captured into a HIP graph
 * on s_compute and replayed; it issues no memset, copy, allocation or
 * synchronisation.
 */
int moe_overlap_step(const moe_step* st, hipStream_t s_compute, hipStream_t s_copy,
                     int flags);

/*
 * moe_overlap_steps - n consecutive steps of the 1F1B schedule (1F1B note
 * page 2, "MoE 1F1B overlap": the micro-batch forwarded in one step is
 * back-propagated in the next), pipelined across the step boundaries.
 * steps[j] describes step j as for moe_overlap_step; all steps share one shape,
 * one workspace (ws, ws_bytes), one shared-expert width F_s and the same expert
 * weights (W_gu, W_down: the micro-batches of one layer between two weight
 * updates), whose transposed copies for the dgrad are made once, at the start
 * of the call, and read by every step's dgrad on either stream; for j >= 1,
 * steps[j].bwd must hold the same buffers as steps[j-1].fwd (field by field;
 * both may be NULL), and no step may forward and back-propagate the same
 * buffers.
 * The streams' roles alternate: step j runs its forward chain on s_copy when j
 * is even and on s_compute when j is odd, and its backward chain on the other
 * stream (each chain in moe_overlap_step's order, the shared expert's forward
 * and D on the chain's own stream).  So step j's backward follows the forward
 * of the same micro-batch on its stream and starts while step j-1's backward
 * still runs on the other one.  Step j's forward waits for the end of step
 * j-2's backward (on the other stream; it has normally ended long before), so
 * a forward may reuse the buffers of any micro-batch back-propagated in an
 * earlier step.  Each stream owns one half of the workspace.  The only other
 * cross-stream waits order the weight-gradient
 * sums (dW_r, dW_gu/dW_down, the shared expert's): each step's sum into a
 * buffer waits for the latest earlier sum into it in the same call, on either
 * stream, so every sum happens in step order.
 * Flags as moe_overlap_step; MOE_STEP_SKIP_WGRAD leaves out the weight
 * gradients (routed and shared) of the LAST step's backward micro-batch only:
 * the caller issues moe_ffn_wgrad (and moe_shared_expert_wgrad) for it after
 * the call -- on s_compute, or on another stream after an event recorded on
 * s_compute, e.g. while the next layer's forward runs (page 1,
 * delay_wgrad_compute) -- and its inputs (xp or x with pair_of_row, a, dh, dyp,
 * offsets) must stay intact until then; the earlier steps' weight gradients
 * run as usual.  Results are bit-identical to n moe_overlap_step calls
 * with MOE_STEP_SERIALIZE (with SKIP_WGRAD on the last).  s_copy forks from s_compute at the start and joins
 * it at the end, so on return work on s_compute depends on everything the call
 * issued; the call may be captured into a HIP graph on s_compute.  Errors: as
 * moe_overlap_step (checked for every step before anything is launched), and
 * MOE_ERR_ARG for n < 1, a step whose bwd is not the previous step's fwd, or
 * steps with different shapes, workspaces, F_s or expert weights.
 */
int moe_overlap_steps(const moe_step* steps, int n, hipStream_t s_compute, hipStream_t s_copy,
                      int flags);

/* ---- kernel timing -------------------------------------------------------- */
/*
 * Opt-in kernel timing for measurement.  While enabled, every kernel the
 * library launches is bracketed by two timing events recorded on the stream
 * it is launched on (so the measured interval is that kernel's execution on
 * its own stream, including any slowdown from work running beside it).
 *   moe_timing_enable(max_records): start recording (up to max_records launches;
 *     further launches are not timed).  Creates the events on first use.
 *     Returns MOE_OK, MOE_ERR_SHAPE (max_records < 1) or MOE_ERR_HIP.
 *   moe_timing_disable(): stop recording (records are kept).
 *   moe_timing_reset(): drop all records.
 *   moe_timing_report(i, name, name_len, total_ms, launches): waits for the
 *     recorded events, then returns the number of distinct kernels recorded
 *     and, for 0 <= i < that number, the i-th kernel's name (copied into
 *     name[name_len]), total milliseconds and launch count.  Negative on error.
 * Timing is process-wide; record and report from one host thread.
 */
int moe_timing_enable(int max_records);
int moe_timing_disable(void);
int moe_timing_reset(void);
int moe_timing_report(int i, char* name, size_t name_len, double* total_ms, int* launches);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
