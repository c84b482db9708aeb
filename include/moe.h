/*
 * moe.h -- C interface of the MI355X (gfx950) top-k sparse mixture-of-experts
 * feed-forward layer (Mixtral: 8 experts, top-2).
 *
 * The layer ("Mixtral 8x7B -- The Evolving Transformer", section 05 MOE ROUTER
 * + MOE, formula y = sum_k w_k E_{i_k}(x); section 04 SWIGLU for the expert):
 * a bias-free linear router scores E experts per token, the top_k largest
 * scores are kept (Mixtral: 2 of 8), a softmax over the kept scores gives
 * their weights, the token runs through each kept SwiGLU expert
 * down(silu(x W1) * (x W3)) and the expert outputs are summed with those
 * weights.  Section 05's MoERouter takes k as a parameter, and the
 * KerasFormers Mixtral page (API table: num_experts, num_experts_per_tok)
 * names the same two parameters; every expert stays resident in device
 * memory.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Shapes   T tokens, d = d_model, f = d_ff, E = n_experts, k = top_k.
 *          The caller flattens (batch, seq) into T rows; the layer routes
 *          R = k T (token, slot) assignments.
 * Layout   dense row-major, no transposes, y = x W:
 *            x [T, d]      w_gate [d, E]
 *            w1 [E, d, f]  (gate)     w3 [E, d, f]  (up)     w2 [E, f, d]  (down)
 *            y [T, d]
 *          (The page's SwiGLU listing calls gate / up / down w1 / w2 / w3;
 *          this interface calls them w1 / w3 / w2.)
 * Dtypes   x, w_gate, w1, w3, w2, y, xp all have shape->dtype (MOE_F32 or
 *          MOE_BF16).  Routing indices are int32, routing weights fp32 and
 *          expert outputs o fp32, in both modes.  Arithmetic is fp32
 *          throughout; with MOE_BF16 the SwiGLU activation between the gate/up
 *          and down products and the output y are rounded to bf16
 *          (round-to-nearest-even).  Router logits are never rounded.
 * Memory   every array argument is a device pointer owned by the caller,
 *          16-byte aligned.  The library allocates and frees nothing; the
 *          scratch it needs comes from the caller's workspace.
 * Aliasing an output must not overlap an input, another output or the
 *          workspace, and the workspace must not overlap an input
 *          (MOE_ERR_ALIAS; the byte ranges checked are the ones the call
 *          reads or writes).  Inputs may overlap one another.  The one
 *          exception is moe_block_forward, whose out may be exactly h or
 *          exactly the residual.
 * Streams  `stream` is a hipStream_t (NULL = the null stream).  Calls only
 *          enqueue work on it and return; results are valid once the
 *          stream has been synchronised.  There is no host/device
 *          synchronisation and no device-to-host copy inside any call.
 * Errors   arguments are checked before anything is enqueued; a failed
 *          check returns a non-zero moe_status_t and enqueues nothing.
 *          MOE_ERR_HIP reports a launch failure (hipGetLastError); faults
 *          inside kernels surface at the caller's next synchronisation.
 *          No call prints, throws or exits.
 * Determinism  no float atomics; every reduction has a fixed order, so two
 *          calls on the same inputs give bit-identical outputs.
 * Concurrency  calls are re-entrant; calls that share a workspace must be
 *          ordered on one stream.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The library is built with hidden visibility; these declarations are its
 * only exported symbols. */
#pragma GCC visibility push(default)

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype_t;

typedef enum {
    MOE_OK = 0,
    MOE_ERR_NULL = 1,        /* a required pointer is NULL                       */
    MOE_ERR_SHAPE = 2,       /* T < 0, d or f not a positive multiple of 8, ...   */
    MOE_ERR_DTYPE = 3,       /* dtype is neither MOE_F32 nor MOE_BF16              */
    MOE_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned                  */
    MOE_ERR_ALIAS = 5,       /* an output overlaps an input                       */
    MOE_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than moe_workspace_bytes */
    MOE_ERR_UNSUPPORTED = 7, /* E outside [2, 64], top_k outside [1, min(4, E)],
                                 or an int8-weight call off bf16 / T <= 32          */
    MOE_ERR_HIP = 8,         /* a HIP launch failed                               */
    MOE_ERR_SCRATCH = 9      /* moe_forward_noalloc: the shape needs more than
                                 MOE_SCRATCH_BYTES of workspace                     */
} moe_status_t;

typedef struct {
    int32_t T;          /* tokens (rows of x); T = 0 returns MOE_OK at once */
    int32_t d_model;    /* d: multiple of 8, >= 8                            */
    int32_t d_ff;       /* f: multiple of 8, >= 8                            */
    int32_t n_experts;  /* E: 2 .. 64                                        */
    int32_t top_k;      /* k: 1 .. min(4, E); k T <= 2^29                    */
    int32_t dtype;      /* moe_dtype_t                                       */
} moe_shape_t;

/* Human-readable name of a status code (static string, never NULL). */
const char *moe_status_str(int status);

/* Bytes of device workspace that moe_forward and moe_experts need for this
 * shape (0 for an invalid shape).  The size depends on every field. */
size_t moe_workspace_bytes(const moe_shape_t *shape);

/* Router: section 05's MoERouter (bias-free Linear d -> E, softmax, top-k,
 * renormalise over the kept experts), in the equivalent form
 *   l[t,e] = sum_j x[t,j] w_gate[j,e]                 (fp32, never rounded)
 *   topk_idx[t,s] = argmax of l over the experts not in topk_idx[t,0..s-1],
 *                   equal logits resolved toward the lower expert index
 *   topk_w[t,s] = e_s / (e_0 + ... + e_{k-1}),  e_s = exp(l[idx_s] - l[idx_0])
 *                   (the softmax of the kept logits; for k = 2 this is
 *                   1/(1+q), q/(1+q) with q = exp(l[idx1] - l[idx0]))
 * Outputs topk_idx int32 [T, k] and topk_w fp32 [T, k], slots in decreasing
 * logit order. */
int moe_route(const moe_shape_t *shape, const void *x, const void *w_gate,
              int32_t *topk_idx, float *topk_w, void *stream);

/* Router in the page's own order of steps: section 05's MoERouter applies
 * a softmax over all E logits, keeps the top_k probabilities and divides
 * them by their sum:
 *   l[t,e]     = sum_j x[t,j] w_gate[j,e]                        (fp32)
 *   probs[t,e] = exp(l[t,e] - m_t) / sum_e' exp(l[t,e'] - m_t),  m_t = max_e l[t,e]
 *                (the sum runs in expert order)
 *   topk_idx[t,s] = argmax of probs over the experts not yet picked, equal
 *                   probabilities resolved toward the lower expert index
 *   topk_w[t,s]   = probs[t,idx_s] / (probs[t,idx_0] + ... + probs[t,idx_{k-1}])
 * The picks and weights equal moe_route's mathematically (exp is increasing
 * and the common factor cancels); only fp32 rounding differs, by a few
 * ulps in the weights, and two logits within an exp rounding of each other
 * may tie here where moe_route orders them.  probs_opt (fp32 [T, E], may be
 * NULL) receives the probabilities.  Outputs must not overlap one another,
 * x or w_gate (MOE_ERR_ALIAS). */
int moe_route_probs(const moe_shape_t *shape, const void *x, const void *w_gate,
                    float *probs_opt, int32_t *topk_idx, float *topk_w, void *stream);

/* Dispatch: the per-expert batching of tokens that section 05 names as the
 * production form of its mask loop.  The R = k T (token, slot) assignments
 * in topk_idx [T, k] are grouped by expert, keeping token order and then
 * slot order within each expert (a stable counting sort):
 *   counts[e]    number of assignments to expert e               int32 [E]
 *   offsets[e]   sum of counts[0..e-1]; offsets[E] = R            int32 [E+1]
 *   pos[t,s]     row of assignment (t,s) in the grouped order     int32 [T, k]
 *   xp[pos[t,s], :] = x[t, :]                                      [R, d]
 * topk_idx entries must lie in [0, E) and a token's k entries must differ
 * (the router's output always does); other entries are not detected on the
 * device and give undefined results.  xp must have room for R rows. */
int moe_dispatch(const moe_shape_t *shape, const void *x, const int32_t *topk_idx,
                 int32_t *counts, int32_t *offsets, int32_t *pos, void *xp,
                 void *stream);

/* Expert gate/up: the first half of section 04's SwiGLU block, for every
 * expert e over its rows r in [offsets[e], offsets[e+1]) of xp:
 *   h[r, :] = silu(xp[r] w1[e]) * (xp[r] w3[e]),  silu(v) = v / (1 + exp(-v))
 * fp32 accumulation; h [R, f] has the layer dtype (rounded to bf16 for
 * MOE_BF16).  counts / offsets are moe_dispatch's outputs, left in device
 * memory (never read back to the host).  h must not overlap xp. */
int moe_expert_gateup(const moe_shape_t *shape, const void *xp, const int32_t *counts,
                      const int32_t *offsets, const void *w1, const void *w3, void *h,
                      void *stream);

/* moe_expert_gateup with the layer's workspace (ws / ws_bytes: at least
 * moe_workspace_bytes(shape)), running exactly the kernels the layer runs
 * for this step.  At bf16 decode sizes (T <= 32) the layer cuts the
 * (expert, 128-column) units of the last round of workgroups in two halves
 * along d_model and adds the halves' fp32 partial sums (kept in the
 * workspace) before the SiLU; elsewhere this is moe_expert_gateup.  Same
 * result as moe_expert_gateup up to the order of that one addition.  The
 * workspace region written must not overlap xp, h, counts or offsets
 * (MOE_ERR_ALIAS). */
int moe_expert_gateup_ws(const moe_shape_t *shape, const void *xp, const int32_t *counts,
                         const int32_t *offsets, const void *w1, const void *w3, void *h,
                         void *ws, size_t ws_bytes, void *stream);

/* Expert down: the second half of section 04's SwiGLU block,
 *   o[r, :] = h[r] w2[e]   for r in [offsets[e], offsets[e+1]),
 * fp32 accumulation, o fp32 [R, d].  o must not overlap h. */
int moe_expert_down(const moe_shape_t *shape, const void *h, const int32_t *counts,
                    const int32_t *offsets, const void *w2, float *o, void *stream);

/* Experts: moe_expert_gateup then moe_expert_down, with h kept in the
 * workspace:  o[r] = (silu(xp[r] w1[e]) * (xp[r] w3[e])) w2[e].
 * o is fp32 [R, d].  ws / ws_bytes: workspace of at least
 * moe_workspace_bytes(shape). */
int moe_experts(const moe_shape_t *shape, const void *xp, const int32_t *counts,
                const int32_t *offsets, const void *w1, const void *w3,
                const void *w2, float *o, void *ws, size_t ws_bytes, void *stream);

/* Combine: section 05's weighted sum over the k slots in slot order, fp32
 * math:
 *   y[t, :] = topk_w[t,0] * o[pos[t,0], :] + ... + topk_w[t,k-1] * o[pos[t,k-1], :]
 * rounded to y's dtype.  o is [R, d], pos and topk_w [T, k].  Every row of
 * y is written. */
int moe_combine(const moe_shape_t *shape, const float *o, const int32_t *pos,
                const float *topk_w, void *y, void *stream);

/* The whole layer: route, dispatch, experts, combine, enqueued back to back
 * on `stream`.  topk_idx_opt / topk_w_opt (int32 [T,k], fp32 [T,k]) receive
 * the routing when non-NULL.  y must not overlap x.
 * ws / ws_bytes: workspace of at least moe_workspace_bytes(shape).
 * At bf16 decode sizes (T <= 32) both expert products may cut the units of
 * their last round of workgroups in two halves along the reduction, as
 * moe_expert_gateup_ws describes; at bf16 prefill sizes the down product
 * may split its reduction in parts that the combine adds.  Either way the
 * result differs from the unsplit stages only in the order of those
 * additions. */
int moe_forward(const moe_shape_t *shape, const void *x, const void *w_gate,
                const void *w1, const void *w3, const void *w2, void *y,
                int32_t *topk_idx_opt, float *topk_w_opt,
                void *ws, size_t ws_bytes, void *stream);

/* ---- The layer without a caller workspace ---------------------------------
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 * moe_forward_noalloc is moe_forward (same kernels, same launch sequence,
 * bit-identical outputs) with its workspace taken from a fixed array in the
 * library's own device memory instead of a caller buffer.
 *   - The array holds MOE_SCRATCH_BYTES (64 MiB: a decode step of the 8x7B
 *     and larger expert shapes needs about 23-26 MiB).  A shape with
 *     moe_workspace_bytes(shape) > MOE_SCRATCH_BYTES returns
 *     MOE_ERR_SCRATCH and enqueues nothing.
 *   - Each GPU the library runs on holds its own copy of the array until
 *     the process ends.  The call's first use on a device looks the
 *     array's device address up (hipGetSymbolAddress); no call allocates,
 *     frees or memsets anything.
 *   - Nothing in the array has to start at zero: every call writes each
 *     workspace entry it reads.
 *   - All calls on one GPU share that GPU's array, so calls that overlap
 *     in time on one GPU (two streams, two threads) race and give undefined
 *     results; order them on one stream.
 * Arguments, outputs and errors as moe_forward (no ws / ws_bytes); y and
 * the routing outputs must not overlap the inputs or each other. */
#define MOE_SCRATCH_BYTES ((size_t)64 << 20)
int moe_forward_noalloc(const moe_shape_t *shape, const void *x, const void *w_gate,
                        const void *w1, const void *w3, const void *w2, void *y,
                        int32_t *topk_idx_opt, float *topk_w_opt, void *stream);

/* ---- Block boundary ----------------------------------------------------
 * The block of "Mixtral 8x7B -- The Evolving Transformer", section 06
 * BLOCK, runs the layer on rms_2 (section 03 RMSNORM) of the residual
 * stream and adds its output back onto the stream.  These calls fuse both into the layer:
 *   rstd[t]  = 1 / sqrt( (1/d) sum_j h[t,j]^2 + eps )        (fp32)
 *   xn[t,j]  = h[t,j] * rstd[t] * rms_weight[j], rounded to the layer dtype
 *   out[t]   = residual[t] + layer(xn)[t], rounded once to the layer dtype
 * rms_weight is [d] in the layer dtype; eps must be finite and >= 0
 * (MOE_ERR_SHAPE otherwise). */

/* Router on the normalised rows: writes xn [T, d] (layer dtype) and the
 * routing as moe_route does, routing on xn as rounded.  xn must not overlap
 * h. */
int moe_rmsnorm_route(const moe_shape_t *shape, const void *h, const void *rms_weight,
                      float eps, const void *w_gate, void *xn, int32_t *topk_idx,
                      float *topk_w, void *stream);

/* The whole block boundary: out = residual + layer(RMSNorm(h)).  residual
 * may be NULL (out = layer(RMSNorm(h))) and is usually h itself.  out may
 * be exactly h or exactly residual (an in-place update of the stream); any
 * other overlap with them is MOE_ERR_ALIAS.  topk_idx_opt / topk_w_opt as
 * in moe_forward.  ws / ws_bytes: workspace of at least
 * moe_workspace_bytes(shape) (it holds xn). */
int moe_block_forward(const moe_shape_t *shape, const void *h, const void *rms_weight,
                      float eps, const void *residual, const void *w_gate, const void *w1,
                      const void *w3, const void *w2, void *out, int32_t *topk_idx_opt,
                      float *topk_w_opt, void *ws, size_t ws_bytes, void *stream);

/* ---- Weight-only int8 expert weights (decode) ----------------------------
 * The KerasFormers Mixtral page's loading example offers int8 weight
 * quantization with low-memory loading for this model but gives no
 * scheme. These calls use symmetric int8 with one fp32 scale per output
 * channel of each expert matrix: W[j,n] ~ s[n] q[j,n]. Decode streams the
 * selected experts' weights, so the codes halve the bytes of the step.
 * Activations, router and outputs keep the layer dtype, which must be
 * MOE_BF16. The layer calls take T <= 32 (decode sizes); other shapes
 * return MOE_ERR_UNSUPPORTED. They also need d_model * d_ff < 2^31 (one
 * expert matrix of codes is addressed with 32-bit offsets), else
 * MOE_ERR_SHAPE. Codes become bf16 exactly, and each product
 * accumulates in fp32 on the bf16 matrix cores. The scale multiplies the
 * finished sum of each output column.
 *
 * Codes of a matrix W [K, N] are stored with pairs of rows interleaved in
 * groups of 8 columns, so that one 16-byte load holds 8 columns of two
 * consecutive rows: the code of W[j, n] is byte
 *   ((j / 2) * (N / 8) + n / 8) * 16 + (j % 2) * 8 + n % 8
 * of the matrix, i.e. the array is int8 [K/2][N/8][2][8]. q1, q3 hold E
 * such matrices of d x f, q2 E of f x d. Scales are s1, s3 fp32 [E, f] and
 * s2 fp32 [E, d]. */

/* Quantize n_mat matrices W [n_mat, K, N] (dtype MOE_F32 or MOE_BF16)
 * into codes q (n_mat K N bytes, in the row-pair layout above) and scales
 * fp32 [n_mat, N]. Per column n of each matrix:
 *   s[n]   = max_j |W[j,n]| / 127                       (fp32 division)
 *   q[j,n] = rint(W[j,n] / s[n]) clamped to [-127, 127] (fp32 division,
 *            round half to even)
 * A zero column gets s = 0 and q = 0. K must be even and positive, N a
 * positive multiple of 8, and n_mat at most 65535. Outputs must not overlap W or each other. The
 * call is a one-time preparation and runs on `stream` like every other
 * call. */
int moe_quantize_int8(int n_mat, int K, int N, int dtype, const void *w, int8_t *q,
                      float *scale, void *stream);

/* moe_expert_gateup on int8 codes:
 *   h[r, :] = silu(s1[e] * (xp[r] q1[e])) * (s3[e] * (xp[r] q3[e])), bf16 [R, f]. */
int moe_expert_gateup_w8(const moe_shape_t *shape, const void *xp, const int32_t *counts,
                         const int32_t *offsets, const int8_t *q1, const float *s1,
                         const int8_t *q3, const float *s3, void *h, void *stream);

/* moe_expert_gateup_w8 with the layer's workspace (ws / ws_bytes: at least
 * moe_workspace_bytes(shape)), running exactly the kernels moe_forward_w8
 * runs for this step.  When the (expert, 256-column) slabs leave the last
 * round of workgroups part-filled, the slabs past the whole rounds run as
 * column halves and as quarters (a column half over one half of d_model),
 * and a small kernel adds each quarter pair's fp32 partial sums (kept in
 * the workspace) before the SiLU.  Same result as moe_expert_gateup_w8 up
 * to the order of the additions.  The workspace region written must not
 * overlap xp, h, counts or offsets (MOE_ERR_ALIAS). */
int moe_expert_gateup_w8_ws(const moe_shape_t *shape, const void *xp, const int32_t *counts,
                            const int32_t *offsets, const int8_t *q1, const float *s1,
                            const int8_t *q3, const float *s3, void *h, void *ws,
                            size_t ws_bytes, void *stream);

/* moe_expert_down on int8 codes:
 *   o[r, :] = s2[e] * (h[r] q2[e]), fp32 [R, d]. */
int moe_expert_down_w8(const moe_shape_t *shape, const void *h, const int32_t *counts,
                       const int32_t *offsets, const int8_t *q2, const float *s2, float *o,
                       void *stream);

/* The whole layer with int8 expert weights: route and dispatch as in
 * moe_forward. Gate/up reads its rows straight from x. Down runs in two K
 * slices, and the combine adds the slices in order before it weights the
 * slots. y [T, d] bf16. ws / ws_bytes: at least moe_workspace_bytes(shape).
 * y must not overlap x. */
int moe_forward_w8(const moe_shape_t *shape, const void *x, const void *w_gate,
                   const int8_t *q1, const float *s1, const int8_t *q3, const float *s3,
                   const int8_t *q2, const float *s2, void *y, int32_t *topk_idx_opt,
                   float *topk_w_opt, void *ws, size_t ws_bytes, void *stream);

/* ---- Backward ------------------------------------------------------------
 * The pages train the router and the experts together ("Mixtral 8x7B --
 * The Evolving Transformer", section 05) and name no loss, capacity or
 * auxiliary term. moe_backward therefore returns the gradients of
 * L = sum(dy * y), with y the layer's forward output and dy [T, d] given in
 * the layer dtype. The top-k picks are a discrete choice and stay fixed;
 * the router's gradient flows through the softmax over the picked logits:
 *   dw_s = dy . o_s,  dl[e] = w_s (dw_s - sum_r w_r dw_r) at the picked e
 *   do_s = w_s dy,    da = do_s W2[e]^T
 *   dg = da * u * silu'(g),  du = da * silu(g)
 *   dx = sum_s (dg W1[e]^T + du W3[e]^T) + dl w_gate^T     (layer dtype)
 *   dw1[e] = sum over e's rows of x^T dg,  dw3[e] likewise with du,
 *   dw2[e] = sum over e's rows of h^T do,  dw_gate = x^T dl  (all fp32)
 * The call recomputes the forward pieces it needs (routing, g, u,
 * h = silu(g) u, o), so nothing has to be kept between calls. With
 * MOE_BF16, h, do, dg and du are rounded to bf16 before the products that
 * use them. Every product accumulates in fp32 on the matrix cores, and
 * every sum has a fixed order (no atomics).
 *
 * Outputs: dx [T, d] (layer dtype); dw_gate [d, E], dw1 and dw3 [E, d, f],
 * dw2 [E, f, d], all fp32 and overwritten. An expert no token picked gets
 * zero gradients. T = 0 writes zero weight gradients (x, dy and dx may
 * then be NULL). Outputs must not
 * overlap the inputs, each other or the workspace. ws / ws_bytes: at least
 * moe_backward_workspace_bytes(shape), which is 0 for an invalid shape. */
size_t moe_backward_workspace_bytes(const moe_shape_t *shape);
int moe_backward(const moe_shape_t *shape, const void *x, const void *w_gate, const void *w1,
                 const void *w3, const void *w2, const void *dy, void *dx, float *dw_gate,
                 float *dw1, float *dw3, float *dw2, void *ws, size_t ws_bytes, void *stream);

#pragma GCC visibility pop

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
