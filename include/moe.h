/*
 * moe.h - C ABI of the MI355X (gfx950) Mixture-of-Experts layer forward.
 *
 * One MoE layer forward, in four steps:
 *   1. softmax top-k routing, or sigmoid top-k routing    moe_route
 *      with a selection-only correction bias
 *   2. count-first token dispatch: per-expert histogram,  moe_dispatch
 *      exclusive scan, stable scatter into expert-contiguous
 *      capacity buckets
 *   3. grouped expert FFN, SwiGLU or ReLU-square           moe_expert_ffn
 *      (plus always-on shared experts)                     moe_shared_ffn
 *   4. weighted combine back to token order                moe_combine
 *   and all of it in one call                              moe_forward
 *
 * Sources of the operation (page title, section):
 *   - "Extend MoEPacked for Bolt ReLU-square routing and BF16 IQ2 precision"
 *     (onnxruntime PR 33963), "Measured CUDA kernel latency" and
 *     "Description": internal softmax routing or preselected FP32 expert
 *     ids/weights through k = 32, default SwiGLU experts and ReLU-square
 *     gate/down experts, isolation of malformed routes, BF16 store
 *     boundaries with FP32 final routing/reduction; and, in the commit
 *     adding projected sigmoid routing, an FP32 selection-only correction
 *     bias with mixture weights from the unbiased normalised scores, route
 *     scaling kept.
 *   - afdEP count-first dispatch validation record ("change", "setup",
 *     fault list): count routes per expert first, compute prefix sums, then
 *     place each row at its known offset in an expert-contiguous buffer of
 *     capacity C rows per expert; malformed routes (negative, out of range,
 *     duplicate) are rejected.
 *   - DeepSeek fleet megakernel on MI300X, REPORT.md (per-op table and the
 *     MoE optimisation steps): gate + top-k, slot-indexed expert gate/up with
 *     fused SiLU, expert down projection, weighted combine; two shared
 *     experts next to 64 routed experts with top-6.
 *
 * Conventions common to every entry point
 *   - All tensor arguments are DEVICE pointers (memory of the GPU current on
 *     the calling thread), row-major, 16-byte aligned, owned by the caller.
 *     The library never allocates, frees or keeps them.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every entry is
 *     asynchronous on `stream`: it validates host-visible arguments,
 *     enqueues kernels and returns; there is no host synchronisation except
 *     in moe_error.
 *   - `ws` / `ws_bytes` is a caller-held device workspace of at least
 *     moe_workspace_bytes() bytes, zeroed once with moe_workspace_init()
 *     after allocation.  Its first 256 bytes carry state between calls (the
 *     malformed-route counter), the rest is scratch.  Calls that share a
 *     workspace must be ordered (same stream or synchronised).
 *   - Routes are numbered q = t*k + j (token t, slot j).
 *   - Errors: every entry returns a moe_status and never throws.  Argument
 *     errors are detected on the host before anything is enqueued.
 *
 * Shapes (moe_problem fields): T tokens, H hidden, E routed experts, k top-k
 * (1 <= k <= min(E, 32)), I expert intermediate size, C capacity (rows per
 * expert).  R_max = min(T*k, E*C) is the size of the expert-contiguous
 * buffer.  H and I must be multiples of 128, and so must I_shared
 * (MOE_ERR_UNSUPPORTED otherwise): every expert GEMM walks K in 64-element
 * k-tiles and its output in 128-column blocks, so no ragged K or column tail
 * is handled.  The pages' workloads all satisfy it.
 *
 * Layouts:
 *   x        [T, H]          act_dtype
 *   logits   [T, E]          float32
 *   score_bias [E]           float32 correction bias of sigmoid routing
 *   ids      [T, k]          int32, slot 0 = largest selection key
 *   w        [T, k]          float32 routing weights
 *   counts   [E]             int32 raw route count per expert (sum = T*k
 *                            minus malformed routes)
 *   offsets  [E+1]           int32 exclusive scan of min(counts, C);
 *                            R = offsets[E] rows are kept
 *   row_src  [R_max]         int32 route q held by row r; -1 for r >= R
 *   route_dst[T, k]          int32 row of route q; -1 = dropped by capacity;
 *                            -2 = malformed route
 *   x_disp   [R_max, H]      act_dtype, row r = x[row_src[r] / k]
 *   w13      [E, 2I, H]      SwiGLU: rows 0..I-1 gate, I..2I-1 up
 *            [E, I, H]       ReLU-square
 *   w2       [E, H, I]
 *   s13      [E, 2I] or [E, I], s2 [E, H]: float32 per-output-row scales
 *                            of e4m3 weights (NULL otherwise)
 *   w13_sh   [n_shared, 2*I_shared, H], w2_sh [n_shared, H, I_shared]:
 *                            bf16 (f32 when act_dtype is f32) SwiGLU
 *   y_disp   [R_max, H]      act_dtype, unweighted expert output of row r
 *   y_shared [T, H]          float32 sum of the shared experts' outputs
 *   out      [T, H]          act_dtype
 */
#ifndef RDE_MOE_H
#define RDE_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t moe_status;
#define MOE_OK 0
#define MOE_ERR_ARG (-1)          /* a NULL pointer, a bad size or dtype combination */
#define MOE_ERR_UNSUPPORTED (-2)  /* a valid problem this build does not handle */
#define MOE_ERR_WORKSPACE (-3)    /* ws NULL, misaligned or smaller than required */
#define MOE_ERR_HIP (-4)          /* a HIP runtime call or kernel launch failed */

#define MOE_F32 0
#define MOE_BF16 1
#define MOE_E4M3 2   /* OCP fp8 e4m3fn weights with float32 per-row scales */

#define MOE_SWIGLU 0 /* h = silu(x W1^T) * (x W3^T), silu(a) = a / (1 + e^-a) */
#define MOE_RELU2 1  /* h = max(x W1^T, 0)^2 */

#define MOE_SOFTMAX 0 /* scores softmax(logits), selection on the logits */
#define MOE_SIGMOID 1 /* scores sigmoid(logits), selection on score + bias */

typedef struct moe_problem {
    int32_t T, H, E, k, I, C;
    int32_t n_shared;    /* always-on shared SwiGLU experts, weight 1 (0 = none) */
    int32_t I_shared;    /* their intermediate size */
    int32_t act_dtype;   /* MOE_F32 or MOE_BF16: x, x_disp, y_disp, out */
    int32_t w_dtype;     /* MOE_F32 (needs act f32), MOE_BF16, MOE_E4M3 (needs act bf16) */
    int32_t act;         /* MOE_SWIGLU or MOE_RELU2 */
    int32_t renormalize; /* 0: w = the selected scores; 1: normalised over the k selected */
    int32_t score_func;  /* MOE_SOFTMAX or MOE_SIGMOID */
    float route_scale;   /* every routed weight is multiplied by it; 0 means 1 */
} moe_problem;

/* Stage boundaries of moe_forward, for moe_meta.stage_events. */
#define MOE_STAGE_BEGIN 0    /* before the first kernel */
#define MOE_STAGE_ROUTE 1    /* after the router (or the copy of preselected routes) */
#define MOE_STAGE_COUNT 2    /* after the histogram / rank / scan kernel */
#define MOE_STAGE_SCATTER 3  /* after the row scatter */
#define MOE_STAGE_GEMM1 4    /* after the gate/up projection with its activation */
#define MOE_STAGE_GEMM2 5    /* after the down projection (routing weights applied) */
#define MOE_STAGE_SHARED 6   /* after the shared experts */
#define MOE_STAGE_COMBINE 7  /* after the final sum to token order */
#define MOE_N_STAGES 8

/* Optional metadata outputs of moe_forward (any field may be NULL; a NULL
 * field is kept in the workspace instead).  Layouts as above.
 * stage_events: NULL, or MOE_N_STAGES hipEvent_t handles (entries may be
 * NULL) that moe_forward records on `stream` at the stage boundaries above,
 * so a caller can time each kernel with events on the stream it runs on.
 * Stages that do no work record their event at the same point as the
 * previous one. */
typedef struct moe_meta {
    int32_t *ids;
    float *w;
    int32_t *counts;
    int32_t *offsets;
    int32_t *row_src;
    int32_t *route_dst;
    void *const *stage_events;
} moe_meta;

/* Workspace size in bytes for problem `p` (the same for every entry point).
 * The workspace is the caller's and is reused from call to call, so that a
 * captured launch sequence replays without allocation (PR 33963
 * "Description": existing routing workspaces are reused; the afdEP
 * count-first record, "setup": runs under CUDA graphs): per-block counts,
 * route ranks, the expert-contiguous rows, the intermediate h and the
 * token-ordered slot rows of the combine.  Returns
 * MOE_ERR_ARG for an invalid problem. */
moe_status moe_workspace_bytes(const moe_problem *p, size_t *bytes);

/* Zero the persistent state at the head of a freshly allocated workspace
 * (by a fill kernel on `stream`). */
moe_status moe_workspace_init(void *ws, size_t ws_bytes, void *stream);

/* Top-k routing (PR 33963 "Measured CUDA kernel latency": internal softmax
 * routing; the commit adding projected sigmoid routing: FP32 selection-only
 * correction bias, weights from the unbiased normalised scores, route
 * scaling).  Per token t:
 *   MOE_SOFTMAX: the selection key of expert e is logits[t,e]; its score is
 *     exp(logits[t,e] - m) / S with m = max_e logits[t,e] and
 *     S = sum_e exp(logits[t,e] - m).  score_bias must be NULL.
 *   MOE_SIGMOID: the score is s_e = 1 / (1 + exp(-logits[t,e])), rounded
 *     once to float32 (computed in double); the selection key is the float32
 *     sum s_e + score_bias[e] (score_bias NULL: no bias).
 *   ids[t, 0..k-1] = the k experts with the largest keys, in descending key
 *   order; equal keys (including -0 and +0) rank by lower index; NaN ranks
 *   below -inf.
 *   w[t, j] = route_scale * score of ids[t,j] (renormalize = 0), or
 *   route_scale * that score over the sum of the k selected scores
 *   (renormalize = 1; for softmax the numerators exp(l - m) over their sum).
 * Weights are computed in float32.  A softmax row of all -inf (or holding a
 * NaN) gets NaN weights. */
moe_status moe_route(const moe_problem *p, const float *logits, const float *score_bias,
                     int32_t *ids, float *w, void *ws, size_t ws_bytes, void *stream);

/* Count-first dispatch (afdEP count-first record: counts, prefix sums, rows
 * at known offsets).  ids may come from moe_route or be preselected by the
 * caller.  A route is malformed when its id is outside [0, E) or repeats an
 * id of an earlier slot of the same token; it is not counted or placed,
 * route_dst = -2, and the workspace's malformed-route counter grows (read it
 * with moe_error).  Of the well-formed routes of expert e, taken in
 * ascending q, the r-th goes to row offsets[e] + r when r < C and is dropped
 * (route_dst = -1) otherwise.  x_disp row r receives an exact copy of
 * x[row_src[r] / k].  All outputs are bit-exact (integer and copy work). */
moe_status moe_dispatch(const moe_problem *p, const void *x, const int32_t *ids,
                        int32_t *counts, int32_t *offsets, int32_t *row_src,
                        int32_t *route_dst, void *x_disp, void *ws,
                        size_t ws_bytes, void *stream);

/* Grouped expert FFN (PR 33963 "Description": SwiGLU default, ReLU-square
 * gate/down experts; BF16 store boundaries).  For every expert e and every
 * row r in [offsets[e], offsets[e+1]):
 *   SwiGLU:      h = silu(x_disp[r] W1_e^T) * (x_disp[r] W3_e^T)
 *   ReLU-square: h = max(x_disp[r] W1_e^T, 0)^2
 *   y_disp[r] = h W2_e^T
 * with float32 accumulation; h is rounded to bf16 (act bf16) before the
 * second projection; y_disp is rounded to act_dtype.  For e4m3 weights the
 * row scales multiply the float32 accumulators.  Rows >= offsets[E] of
 * y_disp are left untouched. */
moe_status moe_expert_ffn(const moe_problem *p, const void *x_disp,
                          const int32_t *offsets, const void *w13,
                          const void *w2, const float *s13, const float *s2,
                          void *y_disp, void *ws, size_t ws_bytes, void *stream);

/* Shared experts (fleet megakernel report: two shared experts beside the
 * routed ones, applied to every token with weight 1):
 *   y_shared[t] = sum_s SwiGLU_s(x[t])   (float32). */
moe_status moe_shared_ffn(const moe_problem *p, const void *x,
                          const void *w13_sh, const void *w2_sh,
                          float *y_shared, void *ws, size_t ws_bytes,
                          void *stream);

/* Weighted combine back to token order (PR 33963 "Description": FP32 final
 * routing/reduction):
 *   out[t] = sum_{j = 0..k-1, route_dst[t,j] >= 0} w[t,j] * y_disp[route_dst[t,j]]
 *            (+ y_shared[t] when y_shared != NULL)
 * summed in float32 in slot order, rounded once to act_dtype.  A token with
 * a malformed route (route_dst = -2) gets a NaN row; other tokens are not
 * affected. */
moe_status moe_combine(const moe_problem *p, const void *y_disp,
                       const int32_t *route_dst, const float *w,
                       const float *y_shared, void *out, void *ws,
                       size_t ws_bytes, void *stream);

/* The whole layer, in the order of the fleet megakernel report's MoE steps
 * (gate and top-k, experts, weighted combine) with the count-first dispatch
 * of the afdEP record between routing and experts, and PR 33963's contract
 * ("Description": internal routing or preselected FP32 ids/weights taken
 * unchanged, BF16 store boundaries, FP32 final reduction): route as
 * moe_route does with `logits` and `score_bias`
 * (or take ids_in / w_in, unchanged, when both are non-NULL),
 * dispatch, expert FFN with the combine weights applied in the
 * down-projection epilogue, shared experts, and the final sum to token
 * order.  Same results as the separate calls: bit-identical metadata,
 * outputs within rounding of the separate path.  Intermediates live in ws. */
moe_status moe_forward(const moe_problem *p, const void *x, const float *logits,
                       const float *score_bias, const int32_t *ids_in, const float *w_in,
                       const void *w13, const void *w2, const float *s13,
                       const float *s2, const void *w13_sh, const void *w2_sh,
                       void *out, const moe_meta *meta, void *ws,
                       size_t ws_bytes, void *stream);

/* moe_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments and results without `ws` / `ws_bytes`.  Its workspace is
 * a device array inside the library, MOE_STATIC_SCRATCH_BYTES bytes on every
 * GPU it runs on, held until the process ends.  A problem whose
 * moe_workspace_bytes() exceeds that returns MOE_ERR_WORKSPACE before
 * anything is enqueued (the decode and ReLU-square shapes and prefill
 * batches of a few hundred tokens fit).  It calls no allocating routine.
 * The first call on a device also enqueues, on `stream`, a clear of the
 * array's control words.  All calls on one GPU share its array: calls that
 * may overlap on one GPU (different streams, or threads) race and must be
 * ordered by the caller.  Malformed routes still poison their tokens' rows;
 * their count is kept in the array and not reported. */
#define MOE_STATIC_SCRATCH_BYTES (32u << 20)
moe_status moe_forward_static(const moe_problem *p, const void *x, const float *logits,
                              const float *score_bias, const int32_t *ids_in, const float *w_in,
                              const void *w13, const void *w2, const float *s13,
                              const float *s2, const void *w13_sh, const void *w2_sh,
                              void *out, const moe_meta *meta, void *stream);

/* Malformed-route report (PR 33963 "Description": isolation of malformed
 * routes, affected tokens poisoned; the afdEP record's correctness runner
 * counts rejected routes of each invalid class).
 * Synchronise `stream`, return the number of malformed routes seen since
 * the last call in *n_invalid_routes, and clear the counter. */
moe_status moe_error(void *ws, size_t ws_bytes, void *stream,
                     int32_t *n_invalid_routes);

/* Human-readable name of a status code (static string). */
const char *moe_status_string(moe_status s);

#ifdef __cplusplus
}
#endif

#endif /* RDE_MOE_H */
