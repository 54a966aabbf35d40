/*
 * moe.h -- C ABI of the MI355X (gfx950) Mixture-of-Experts layer forward.
 *
 * The layer is the one stated in "Writing a fused MoE operator in Ascend C"
 * (section "MoE computation flow"): for tokens x[T,H],
 *   1. routing   logits = x . W_r (+ b_r), ids = the top_k experts per token;
 *   2. gating    w = softmax over the top_k selected logits;
 *   3. dispatch  the tokens of each expert gathered into a contiguous block;
 *   4. experts   y_e = GELU(x_e . W1[e]) . W2[e]   (tanh-form GELU, no bias);
 *   5. combine   y[t] = sum_j w[t,j] * y_{ids[t,j]}[t].
 * The stage entry points below split the layer at the same cuts as that
 * article's step list; moe_forward runs all of them.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers (memory of the current HIP
 *     device) unless marked "host".  Layouts are dense row-major with the
 *     shapes given.  The caller allocates and owns every buffer; the library
 *     never allocates or frees device memory, never synchronises, and never
 *     copies device data to the host.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL means
 *     the default stream).  Results are ready when the stream reaches them.
 *   - dtype selects the element type of x, W_r, W1, W2, xp, yp and y:
 *     MOE_F32 (fp32 throughout) or MOE_BF16 (bf16 storage, fp32
 *     accumulation; the FFN intermediate is rounded to bf16).  Router bias
 *     and gate weights are always fp32; expert ids and indices are int32.
 *   - Alignment: tensors in dtype (x, W_r, W1, W2, xp, yp, y and their
 *     gradients) and every workspace or saved buffer must be 16-byte
 *     aligned; int32 and fp32 arrays (ids, offsets, indices, gate weights,
 *     router bias) 4-byte aligned.  (hipMalloc / torch allocations and
 *     whole rows of them are.)
 *   - Arguments are validated on the host before anything is enqueued; a
 *     call that returns an error has no device side effects.
 *   - Results are bitwise deterministic for fixed inputs and shapes (no
 *     floating-point atomics).
 *   - The library is stateless and re-entrant.  Calls on different streams
 *     must not share a workspace.
 *
 * Status codes
 *   MOE_OK                 success (work enqueued)
 *   MOE_ERR_INVALID_ARG    a required pointer is NULL or under-aligned, a
 *                          size is <= 0, top_k is outside [1, E], or
 *                          ws_bytes is smaller than the entry point needs
 *   MOE_ERR_UNSUPPORTED    dtype is not MOE_F32/MOE_BF16, H or F is not a
 *                          multiple of 8, E > 1024, top_k > 16, or a size
 *                          exceeds the int32 index range (T*top_k*max(H,F)
 *                          and H*F elements must stay below 2^31)
 *   MOE_ERR_LAUNCH         the HIP runtime reported an error for a launch
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t moe_status;
enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,
  MOE_ERR_UNSUPPORTED = 2,
  MOE_ERR_LAUNCH = 3,
};

typedef int32_t moe_dtype;
enum {
  MOE_F32 = 0,
  MOE_BF16 = 1,
};

/* Gate weights (moe_route_ex, moe_forward_ex). */
typedef int32_t moe_gating;
enum {
  /* softmax over the top_k selected logits: each row of topk_w sums to 1
     (fused article, section 1 "Routing + Gating"; the default everywhere) */
  MOE_GATE_TOPK_SOFTMAX = 0,
  /* softmax over all E logits, then the probabilities of the top_k selected
     experts, not renormalised (CANN MoE operator article, section 2.1:
     Softmax -> Top-k -> mask); the selected experts are the same */
  MOE_GATE_SOFTMAX_TOPK = 1,
};

/* Host string for a status code (static storage; never NULL). */
const char* moe_status_string(moe_status status);

/*
 * Bytes of workspace that moe_forward needs for this layer shape, written to
 * *bytes (host pointer).  This amount is also enough for every stage entry
 * point called with the same (or smaller) sizes.  The workspace holds the
 * router's partial logits, dispatch counters, the dispatched rows xp[T*k,H],
 * the FFN intermediate h[T*k,F] and the expert outputs yp[T*k,H].
 */
moe_status moe_workspace_bytes(int64_t T, int64_t H, int64_t E, int32_t top_k,
                               int64_t F, moe_dtype dtype, size_t* bytes);

/* Stages, for moe_stage_workspace_bytes. */
typedef int32_t moe_stage;
enum {
  MOE_STAGE_ROUTE = 0,
  MOE_STAGE_PERMUTE = 1,
  MOE_STAGE_EXPERT_FFN = 2,
  MOE_STAGE_COMBINE = 3,
  MOE_STAGE_FORWARD = 4,
  MOE_STAGE_EXPERT_FFN_BACKWARD = 5,
  MOE_STAGE_EXPERT_FFN_GATHER = 6,
};

/*
 * Bytes of workspace one entry point needs for a layer of this shape,
 * written to *bytes (host pointer): MOE_STAGE_ROUTE -> moe_route,
 * MOE_STAGE_PERMUTE -> moe_permute, MOE_STAGE_EXPERT_FFN -> moe_expert_ffn
 * with R = T*top_k rows, MOE_STAGE_COMBINE -> 0 (no workspace),
 * MOE_STAGE_FORWARD -> moe_forward (same as moe_workspace_bytes),
 * MOE_STAGE_EXPERT_FFN_BACKWARD -> moe_expert_ffn_backward with R = T*top_k,
 * MOE_STAGE_EXPERT_FFN_GATHER -> moe_expert_ffn_gather with R = T*top_k.
 * Returns MOE_ERR_INVALID_ARG for an unknown stage.
 */
moe_status moe_stage_workspace_bytes(moe_stage stage, int64_t T, int64_t H,
                                     int64_t E, int32_t top_k, int64_t F,
                                     moe_dtype dtype, size_t* bytes);

/*
 * Routing + gating (fused article, section 1 "Routing + Gating";
 * routing article, "Top-K routing").
 *   x[T,H], w_r[H,E] in dtype; router_bias[E] fp32 or NULL (no bias).
 *   logits[t,e] = sum_h x[t,h]*w_r[h,e] + router_bias[e], accumulated in fp32.
 *   topk_ids[T,top_k] int32: the top_k experts of each token in descending
 *     logit order; equal logits go to the lower expert index.
 *   topk_w[T,top_k] fp32: softmax over the top_k selected logits, in the
 *     same slot order (so each row sums to 1).
 *   A NaN logit ranks as -inf, so every token still gets top_k distinct
 *     experts in [0, E); a token with any NaN logit gets NaN weights in all
 *     its slots (so NaN inputs show in y instead of being dropped).
 *   ws/ws_bytes: device workspace (partial logits).
 */
moe_status moe_route(const void* x, const void* w_r, const float* router_bias,
                     int64_t T, int64_t H, int64_t E, int32_t top_k,
                     moe_dtype dtype, int32_t* topk_ids, float* topk_w,
                     void* ws, size_t ws_bytes, void* stream);

/*
 * Routing + gating with the variants of the CANN MoE operator article:
 *   router_dtype: element type of w_r.  Either dtype itself, or MOE_F32 with
 *     dtype MOE_BF16: an fp32 router for bf16 tokens (section 4.2 keeps the
 *     routing network in FP32); the products x*w_r are then formed from the
 *     fp32 weights (accumulated in fp32).  Any other pair returns
 *     MOE_ERR_UNSUPPORTED.
 *   gating: MOE_GATE_TOPK_SOFTMAX or MOE_GATE_SOFTMAX_TOPK (else
 *     MOE_ERR_INVALID_ARG).
 * Everything else as moe_route, which is moe_route_ex(..., dtype, dtype,
 * MOE_GATE_TOPK_SOFTMAX, ...).  The workspace size is the same for both
 * router types (moe_stage_workspace_bytes with MOE_STAGE_ROUTE).
 */
moe_status moe_route_ex(const void* x, const void* w_r, const float* router_bias,
                        int64_t T, int64_t H, int64_t E, int32_t top_k,
                        moe_dtype dtype, moe_dtype router_dtype, moe_gating gating,
                        int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes,
                        void* stream);

/*
 * Expert capacity (CANN MoE operator article, section 4.3, capacity_factor;
 * fused article, "MoE computation flow": dispatch into [num_experts,
 * expert_capacity] blocks): *capacity (host) = ceil(F * T * top_k / E) for
 * the factor F = factor_num / factor_den, computed exactly in integers (the
 * article's 1.2 is 6/5).  factor_num <= 0 gives 0 (no limit).  Returns
 * MOE_ERR_INVALID_ARG for a NULL capacity, T < 0, top_k < 1, E < 1 or
 * factor_den <= 0, and MOE_ERR_UNSUPPORTED when factor_num or factor_den
 * exceeds 2^20, T exceeds 2^31, E exceeds 2^20 or the result exceeds
 * INT32_MAX.  Host only; enqueues nothing.
 */
moe_status moe_expert_capacity(int64_t T, int32_t top_k, int64_t E, int64_t factor_num,
                               int64_t factor_den, int32_t* capacity);

/*
 * Dispatch (fused article, GatherTokensByExpert): group the R = T*top_k
 * (token, slot) pairs by expert, dropless, in ascending token order within
 * each expert (then ascending slot).
 *   topk_ids[T,top_k] int32 in [0,E) (as produced by moe_route).
 *   expert_offsets[E+1] int32: expert e owns dispatched rows
 *     [expert_offsets[e], expert_offsets[e+1]); expert_offsets[E] = R when
 *     every id is in [0,E).
 *   sorted_token[R] int32: source token of each dispatched row.
 *   inv_pos[T*top_k] int32: dispatched row of pair (t, j), at index t*top_k+j.
 *   xp[R,H] (dtype): xp[p,:] = x[sorted_token[p],:], a bit copy.  xp may be
 *     NULL: then only the indices are built (for moe_expert_ffn_gather,
 *     which reads the rows from x itself).
 * A pair whose id is outside [0,E) is dropped as a pair beyond the capacity
 * of moe_permute_ex is (inv_pos = -1, not counted in expert_offsets): a bad
 * id never indexes memory.
 */
moe_status moe_permute(const void* x, const int32_t* topk_ids,
                       int64_t T, int64_t H, int64_t E, int32_t top_k,
                       moe_dtype dtype, int32_t* expert_offsets,
                       int32_t* sorted_token, int32_t* inv_pos, void* xp,
                       void* ws, size_t ws_bytes, void* stream);

/*
 * Capacity-limited dispatch (same articles as moe_expert_capacity): as
 * moe_permute, but each expert keeps only its first `capacity` pairs in the
 * dispatch order (ascending token, then slot); the other pairs are dropped:
 *   inv_pos[t*top_k+j] = -1 for a dropped pair;
 *   expert_offsets[e+1] - expert_offsets[e] = min(pairs of e, capacity), so
 *     expert_offsets[E] (the kept rows) may be less than T*top_k;
 *   sorted_token and xp are written for the kept rows only.
 * capacity <= 0 means no limit (exactly moe_permute).  Same workspace as
 * moe_permute.
 */
moe_status moe_permute_ex(const void* x, const int32_t* topk_ids,
                          int64_t T, int64_t H, int64_t E, int32_t top_k,
                          moe_dtype dtype, int32_t capacity, int32_t* expert_offsets,
                          int32_t* sorted_token, int32_t* inv_pos, void* xp,
                          void* ws, size_t ws_bytes, void* stream);

/*
 * Experts (fused article, expert kernel step 3: Mmad -> GELU -> Mmad):
 * for each expert e with rows [expert_offsets[e], expert_offsets[e+1]),
 *   yp[rows] = GELU(xp[rows] . w1[e]) . w2[e]
 *   xp[R,H], w1[E,H,F], w2[E,F,H], yp[R,H] in dtype; expert_offsets[E+1]
 *   int32, non-decreasing, expert_offsets[0] = 0, expert_offsets[E] <= R
 *   (rows from expert_offsets[E] on are neither read nor written).  Other
 *   offsets are clamped, expert e taking rows [a, b) with
 *   a = min(max(off[e], 0), R) and b = min(max(off[e+1], a), R): no row
 *   outside the R rows is touched (rows two such ranges share are written
 *   twice, in no fixed order).
 *   GELU is the tanh form 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))).
 *   Experts with no rows are skipped (their weights are not read).
 *   ws holds h[R,F] (dtype).
 */
moe_status moe_expert_ffn(const void* xp, const int32_t* expert_offsets,
                          const void* w1, const void* w2, int64_t R, int64_t H,
                          int64_t E, int64_t F, moe_dtype dtype, void* yp,
                          void* ws, size_t ws_bytes, void* stream);

/*
 * Experts with the dispatch fused into the first GEMM (fused article,
 * "fusion idea": the dispatched tokens go straight into the expert compute
 * instead of through a gathered copy): as moe_expert_ffn, except that
 * dispatched row p is row sorted_token[p] of x, so xp is never written.
 * This is the expert stage exactly as moe_forward runs it.
 *   x[T,H] (dtype); sorted_token[R] int32 (as moe_permute returns it): the
 *   source token of each dispatched row.  A sorted_token entry outside
 *   [0,T) reads as a zero row (no memory outside x is read).
 *   expert_offsets, w1, w2, yp, R, H, E, F, dtype: as moe_expert_ffn.
 *   ws: h[R,F] (and, for MOE_F32, the gathered rows; the fp32 GEMM reads
 *   contiguous rows), sized by moe_stage_workspace_bytes with
 *   MOE_STAGE_EXPERT_FFN_GATHER.
 * Errors as moe_expert_ffn; T < 0 is MOE_ERR_INVALID_ARG, and T*H beyond the
 * int32 index range MOE_ERR_UNSUPPORTED.
 */
moe_status moe_expert_ffn_gather(const void* x, int64_t T, const int32_t* sorted_token,
                                 const int32_t* expert_offsets, const void* w1, const void* w2,
                                 int64_t R, int64_t H, int64_t E, int64_t F, moe_dtype dtype,
                                 void* yp, void* ws, size_t ws_bytes, void* stream);

/*
 * Combine (fused article, ScatterWithWeights): weighted accumulation of each
 * token's expert outputs,
 *   y[t,:] = sum_{j<top_k} topk_w[t,j] * yp[inv_pos[t*top_k+j],:]
 * summed in fp32 in slot order, then stored in dtype (round to nearest even).
 * A slot whose inv_pos is outside [0, T*top_k) adds nothing (-1: a pair
 * dropped by the dispatch); yp is never read outside its T*top_k rows.
 *   yp[T*top_k,H], y[T,H] in dtype; inv_pos int32; topk_w fp32.
 */
moe_status moe_combine(const void* yp, const int32_t* inv_pos,
                       const float* topk_w, int64_t T, int64_t H,
                       int32_t top_k, moe_dtype dtype, void* y, void* stream);

/*
 * The whole layer forward (fused article, section 3 "full call"): route,
 * dispatch, experts and combine, enqueued back to back on `stream`.  For a
 * bf16 layer with top_k = 1 the combine runs inside the second expert GEMM
 * (fused article, "fusion idea": each token's single row, weighted, is
 * written straight to y); y is the same bits either way.
 *   y[T,H] (dtype) output.
 *   topk_ids_out[T,top_k] / topk_w_out[T,top_k]: optional (may be NULL)
 *     copies of the routing decision and gate weights.
 *   ws_bytes must be at least moe_workspace_bytes() for the same shape.
 */
moe_status moe_forward(const void* x, const void* w_r, const float* router_bias,
                       const void* w1, const void* w2, int64_t T, int64_t H,
                       int64_t E, int32_t top_k, int64_t F, moe_dtype dtype,
                       void* y, int32_t* topk_ids_out, float* topk_w_out,
                       void* ws, size_t ws_bytes, void* stream);

/*
 * The whole layer forward with the variants: router_dtype and gating as in
 * moe_route_ex, capacity as in moe_permute_ex (<= 0: dropless).  A token
 * whose slots are all dropped gets y[t,:] = 0.  moe_forward is
 * moe_forward_ex(..., dtype, dtype, MOE_GATE_TOPK_SOFTMAX, 0, ...); the
 * workspace is moe_workspace_bytes() for the same shape.
 */
moe_status moe_forward_ex(const void* x, const void* w_r, const float* router_bias,
                          const void* w1, const void* w2, int64_t T, int64_t H,
                          int64_t E, int32_t top_k, int64_t F, moe_dtype dtype,
                          moe_dtype router_dtype, moe_gating gating, int32_t capacity,
                          void* y, int32_t* topk_ids_out, float* topk_w_out,
                          void* ws, size_t ws_bytes, void* stream);

/*
 * The layer forward for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  As
 * moe_forward (default gating, dropless, router weights in dtype), but with
 * no workspace argument: the workspace is a fixed 32 MiB device array inside
 * the library (one copy per GPU, held until the process ends), so nothing is
 * allocated by the library or the caller beyond x, the weights and the
 * outputs.  For the layer to fit, its moe_forward workspace less the split
 * GEMM partials (routing outputs, dispatch indices, the expert outputs
 * yp[T*top_k,H] and the larger of h[T*top_k,F] and the router's partial
 * logits) must be at most 32 MiB, else MOE_ERR_UNSUPPORTED: decode-sized
 * batches (e.g. 64 tokens of a 7168-wide layer with 8 of 256 experts).  The
 * expert GEMMs do not split tiles along K here, so y may differ from
 * moe_forward's in rounding (ids and gate weights are identical).  Every call
 * on a GPU uses that GPU's one array: calls that overlap on one GPU (other
 * streams, other threads) race and must be serialised by the caller.
 */
moe_status moe_forward_noalloc(const void* x, const void* w_r, const float* router_bias,
                               const void* w1, const void* w2, int64_t T, int64_t H, int64_t E,
                               int32_t top_k, int64_t F, moe_dtype dtype, void* y,
                               int32_t* topk_ids_out, float* topk_w_out, void* stream);

/* ------------------------------------------------------------------------
 * Training: a forward that keeps what the backward needs, and the backward.
 *
 * The pages describe training with this layer (CANN MoE article: section 3,
 * the backward pass's gradient aggregation; section 4.2, the router kept in
 * fp32; section 5, whole training steps) but print no gradient formulas.
 * The backward computes the exact derivative of the forward above for an
 * output gradient dy: no gradient flows through the top-k choice or the
 * capacity drop (both are piecewise constant in the logits), so the logits
 * receive gradient only through the gate weights of the selected experts;
 * a dropped (token, slot) pair's weight gets none.  GELU' is that of the tanh
 * form.  Accumulation is fp32; bf16 results are rounded to nearest even.
 * ------------------------------------------------------------------------ */

/*
 * *bytes = size of the state moe_forward_train keeps for moe_backward
 * (dispatch indices, fp32 logits [T,E], the first expert GEMM's
 * pre-activation z [T*top_k,F] and GELU(z), the expert outputs
 * [T*top_k,H]).  Its layout is private to the library.
 */
moe_status moe_saved_bytes(int64_t T, int64_t H, int64_t E, int32_t top_k, int64_t F,
                           moe_dtype dtype, size_t* bytes);

/* *bytes = workspace moe_backward needs for this shape. */
moe_status moe_backward_workspace_bytes(int64_t T, int64_t H, int64_t E, int32_t top_k,
                                        int64_t F, moe_dtype dtype, size_t* bytes);

/*
 * Backward of moe_expert_ffn over the dispatched rows (the expert stage of
 * moe_backward, for callers that run their own dispatch): for every expert e
 * with rows [expert_offsets[e], expert_offsets[e+1]),
 *   dz = (dyp W2[e]^T) * GELU'(z),   dW2[e] = h^T dyp,
 *   dxp = dz W1[e]^T,                 dW1[e] = xp^T dz.
 *   dyp[R,H]: gradient with respect to the expert outputs yp; xp[R,H]: the
 *     dispatched token rows; z[R,F], h[R,F]: the first GEMM's pre-activation
 *     and GELU(z) (as moe_forward_train keeps them); all in dtype.
 *   dxp[R,H], dw1[E,H,F], dw2[E,F,H] (dtype) outputs.  dxp may be the same
 *     buffer as dyp.  Experts with no rows get zero weight gradients; with
 *     R == 0 only those are written (dyp, xp, z, h, dxp may be NULL).
 *   ws holds dz[R,F] (moe_stage_workspace_bytes, MOE_STAGE_EXPERT_FFN_BACKWARD).
 */
moe_status moe_expert_ffn_backward(const void* dyp, const void* xp,
                                   const int32_t* expert_offsets, const void* z, const void* h,
                                   const void* w1, const void* w2, int64_t R, int64_t H,
                                   int64_t E, int64_t F, moe_dtype dtype, void* dxp, void* dw1,
                                   void* dw2, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_forward_ex that also fills `saved` (device, caller-owned, at least
 * moe_saved_bytes()) for moe_backward.  topk_ids / topk_w are required here
 * (the backward takes them back).  y, ids and w equal moe_forward_ex's for
 * the same inputs.  ws as for moe_forward_ex.  With T == 0 nothing is
 * enqueued and x, y, topk_ids, topk_w (empty) may be NULL.
 */
moe_status moe_forward_train(const void* x, const void* w_r, const float* router_bias,
                             const void* w1, const void* w2, int64_t T, int64_t H, int64_t E,
                             int32_t top_k, int64_t F, moe_dtype dtype, moe_dtype router_dtype,
                             moe_gating gating, int32_t capacity, void* y, int32_t* topk_ids,
                             float* topk_w, void* saved, size_t saved_bytes, void* ws,
                             size_t ws_bytes, void* stream);

/*
 * Backward of the layer for dy[T,H] (dtype), after moe_forward_train with the
 * same inputs, shape, types and gating (its topk_ids, topk_w and `saved`,
 * unchanged; the capacity is already in `saved`).  Outputs (device, caller
 * owned, fully overwritten):
 *   dx[T,H] (dtype), dw_r[H,E] (router_dtype), dw1[E,H,F], dw2[E,F,H] (dtype);
 *   db_r[E] fp32, optional (NULL: not computed; the router bias's gradient);
 *   dtopk_w[T,top_k] fp32, optional (NULL: kept in the workspace): the
 *   gradient with respect to the gate weights (0 for dropped pairs).
 * An expert that received no rows gets zero weight gradients.
 * topk_ids must be the training forward's (k distinct experts per token;
 * the gradient assumes no expert repeats within a token).  Should a slot's
 * id lie outside [0,E) anyway, that slot is left out of the router gradient
 * (its weight and weight gradient take no part in the softmax Jacobian, and
 * no logit, row of W_r or column of dW_r is addressed for it); dtopk_w, dW1
 * and dW2 follow the dispatch kept in `saved`.
 * ws_bytes must be at least moe_backward_workspace_bytes().  Errors as for
 * the forward; enqueued on `stream`, nothing allocated or synchronised.
 * With T == 0 the weight gradients are zero-filled and dy, x, topk_ids,
 * topk_w, dx (empty) may be NULL.
 */
moe_status moe_backward(const void* dy, const void* x, const void* w_r, const void* w1,
                        const void* w2, int64_t T, int64_t H, int64_t E, int32_t top_k,
                        int64_t F, moe_dtype dtype, moe_dtype router_dtype, moe_gating gating,
                        const int32_t* topk_ids, const float* topk_w, const void* saved,
                        size_t saved_bytes, void* dx, void* dw_r, float* db_r, void* dw1,
                        void* dw2, float* dtopk_w, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
