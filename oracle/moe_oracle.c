/*
 * CPU oracle for the top-2 sparse mixture-of-experts feed-forward layer.
 *
 * TEST INFRASTRUCTURE.  This file is the slow, plain reference that the HIP
 * library is checked against.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load it.  It shares no code, header, table or
 * helper with the GPU library, and the GPU library never calls it.
 *
 * What it computes, per token t and independently of every other token
 * ("Mixtral 8x7B -- The Evolving Transformer", section 05 MOE ROUTER + MOE,
 * its formula y = sum_k w_k E_{i_k}(x) and the MoERouter / MoE modules;
 * section 04 SWIGLU for the expert body):
 *
 *   1. router logits   l[e] = sum_j x[t,j] * Wg[j,e]          (bias-free Linear)
 *   2. top-k           i0 = argmax_e l[e], i1 = argmax_{e != i0} l[e], ...
 *                      (k = 2 for Mixtral; 1 <= k <= 4 here), exact ties
 *                      resolved toward the lower expert index
 *   3. weights         softmax over the k selected logits; for k = 2:
 *                      q = exp(l[i1] - l[i0]);  w0 = 1/(1+q),  w1 = q/(1+q)
 *                      (equal to softmax over all experts, keep the top k,
 *                      divide by their sum -- the page's order of steps)
 *   4. experts         for each slot s, e = i_s:
 *                      g = x W1[e], u = x W3[e]           (gate, up)
 *                      a = silu(g) * u,  silu(v) = v / (1 + exp(-v))
 *                      o_s = a W2[e]                      (down)
 *   5. combine         y[t] = w0 * o_0 + w1 * o_1 + ...   (slot order)
 *
 * Matrix names follow the layer's C interface: W1 = gate, W3 = up,
 * W2 = down.  (The page's SwiGLU listing calls the same three matrices
 * w1 = gate, w2 = up, w3 = down.)  Layouts are dense row-major with no
 * transposes: x [T,d], Wg [d,E], W1/W3 [E,d,f], W2 [E,f,d], y [T,d].
 *
 * Precision.  Inputs arrive as fp32 or as bf16 bit patterns; both are
 * widened exactly to double.  Every sum, product and exp is fp64, sums run
 * in ascending index order, and nothing is rounded except where stated:
 * the top-2 decision is taken on the logits rounded to fp32, the precision
 * in which the GPU library takes it, so that both sides decide the same
 * integer the same way.  The weights use the unrounded fp64 logits.
 *
 * Threads split the tokens; each token's arithmetic is the same sequential
 * loop whichever thread runs it.
 *
 * Block boundary (the same page, section 06 BLOCK, with the norm of
 * section 03 RMSNORM: the layer's input is rms_2 of the residual stream,
 * and the layer's output is added back onto it):
 *
 *   r[t]    = 1 / sqrt( (1/d) sum_j h[t,j]^2 + eps )
 *   xn[t,j] = h[t,j] * r[t] * g[j], rounded once to the layer dtype
 *             (round to nearest, ties to even), the precision in which the
 *             layer consumes its input
 *   out[t]  = res[t] + y[t],  y = the layer applied to xn
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_BF16 = 1 };

/* Widen element i of an fp32 or bf16 array to double (exact in both cases:
 * a bf16 value is the upper half of an fp32 bit pattern). */
static double load_elem(const void *p, int dtype, size_t i) {
    float v;
    if (dtype == ORC_F32) {
        v = ((const float *)p)[i];
    } else {
        uint32_t bits = (uint32_t)((const uint16_t *)p)[i] << 16;
        memcpy(&v, &bits, sizeof v);
    }
    return (double)v;
}

/* Step 1: l[e] = sum_j x[j] * Wg[j, e], j ascending. */
static void router_logits(int d, int E, const void *x, size_t x_off,
                          const void *wg, int dtype, double *l) {
    for (int e = 0; e < E; ++e) l[e] = 0.0;
    for (int j = 0; j < d; ++j) {
        double xj = load_elem(x, dtype, x_off + (size_t)j);
        for (int e = 0; e < E; ++e)
            l[e] += xj * load_elem(wg, dtype, (size_t)j * E + e);
    }
}

/* Steps 2-3 on one token's logits, for top-k (1 <= k <= 4; the page's
 * MoERouter takes k as a parameter, Mixtral uses 2).  The k experts are
 * picked greedily: each pick is the largest fp32-rounded logit among the
 * experts not yet picked, and strict '>' keeps the first (lowest) index
 * among equal values.  The weights are the softmax over the picked logits,
 * taken relative to the first: e_0 = 1, e_s = exp(l[i_s] - l[i_0]),
 * w_s = e_s / (e_0 + ... + e_{k-1}).  For k = 2 this is w_0 = 1/(1+q),
 * w_1 = q/(1+q) with q = exp(l[i_1] - l[i_0]). */
enum { ORC_MAX_K = 4 };
static void topk_softmax(int E, int k, const double *l, int32_t *idx, double *w) {
    for (int s = 0; s < k; ++s) {
        int best = -1;
        for (int e = 0; e < E; ++e) {
            int taken = 0;
            for (int r = 0; r < s; ++r) taken |= idx[r] == e;
            if (taken) continue;
            if (best < 0 || (float)l[e] > (float)l[best]) best = e;
        }
        idx[s] = best;
    }
    double ex[ORC_MAX_K], sum = 0.0;
    for (int s = 0; s < k; ++s) {
        ex[s] = s == 0 ? 1.0 : exp(l[idx[s]] - l[idx[0]]);
        sum += ex[s];
    }
    for (int s = 0; s < k; ++s) w[s] = ex[s] / sum;
}

/* Step 4a for one input row xr[d] and expert e: the SwiGLU hidden
 * activation a = silu(x W1[e]) * (x W3[e]) into g[f]; u is scratch [f]. */
static void swiglu_hidden(int d, int f, const double *xr, int e, const void *w1,
                          const void *w3, int dtype, double *g, double *u) {
    size_t in_base = (size_t)e * d * f;   /* W1[e], W3[e] : [d, f] */
    for (int n = 0; n < f; ++n) { g[n] = 0.0; u[n] = 0.0; }
    for (int j = 0; j < d; ++j) {
        double xj = xr[j];
        size_t row = in_base + (size_t)j * f;
        for (int n = 0; n < f; ++n) {
            g[n] += xj * load_elem(w1, dtype, row + n);
            u[n] += xj * load_elem(w3, dtype, row + n);
        }
    }
    for (int n = 0; n < f; ++n)
        g[n] = g[n] / (1.0 + exp(-g[n])) * u[n];   /* a = silu(g) * u */
}

/* Step 4b: o[d] = a[f] W2[e]. */
static void swiglu_down(int d, int f, const double *a, int e, const void *w2, int dtype,
                        double *o) {
    size_t out_base = (size_t)e * f * d;  /* W2[e] : [f, d] */
    for (int m = 0; m < d; ++m) o[m] = 0.0;
    for (int n = 0; n < f; ++n) {
        double an = a[n];
        size_t row = out_base + (size_t)n * d;
        for (int m = 0; m < d; ++m) o[m] += an * load_elem(w2, dtype, row + m);
    }
}

/* Step 4 for one input row xr[d] and expert e.  g, u are scratch [f];
 * the result goes to o[d]. */
static void swiglu_expert(int d, int f, const double *xr, int e,
                          const void *w1, const void *w3, const void *w2,
                          int dtype, double *g, double *u, double *o) {
    swiglu_hidden(d, f, xr, e, w1, w3, dtype, g, u);
    swiglu_down(d, f, g, e, w2, dtype, o);
}

/* ------------------------------------------------------------------ */
/* Threading: split [0, n) into contiguous chunks, one per thread.     */

typedef void (*range_fn)(void *ctx, int lo, int hi);
typedef struct { range_fn fn; void *ctx; int lo, hi; } chunk_t;

static void *run_chunk(void *p) {
    chunk_t *c = (chunk_t *)p;
    c->fn(c->ctx, c->lo, c->hi);
    return NULL;
}

static void parallel_for(int n, int threads, range_fn fn, void *ctx) {
    if (threads < 1) threads = 1;
    if (threads > n) threads = n > 0 ? n : 1;
    pthread_t tid[256];
    chunk_t ch[256];
    if (threads > 256) threads = 256;
    int done = 0;
    for (int i = 0; i < threads; ++i) {
        int lo = (int)((long long)n * i / threads);
        int hi = (int)((long long)n * (i + 1) / threads);
        ch[i] = (chunk_t){fn, ctx, lo, hi};
        if (i == threads - 1 || pthread_create(&tid[i], NULL, run_chunk, &ch[i]) != 0) {
            run_chunk(&ch[i]);
            tid[i] = 0;
        }
        done = i + 1;
    }
    for (int i = 0; i < done; ++i)
        if (tid[i]) pthread_join(tid[i], NULL);
}

/* ------------------------------------------------------------------ */
/* Entry points (called through ctypes by the Python side).            */

typedef struct {
    int T, d, f, E, k, dtype;
    const void *x, *wg, *w1, *w3, *w2;
    int32_t *idx;
    double *w, *logits, *y;
} layer_ctx;

static void route_range(void *p, int lo, int hi) {
    layer_ctx *c = (layer_ctx *)p;
    double l[256];
    for (int t = lo; t < hi; ++t) {
        router_logits(c->d, c->E, c->x, (size_t)t * c->d, c->wg, c->dtype, l);
        if (c->logits)
            for (int e = 0; e < c->E; ++e) c->logits[(size_t)t * c->E + e] = l[e];
        topk_softmax(c->E, c->k, l, c->idx + (size_t)c->k * t, c->w + (size_t)c->k * t);
    }
}

/* Router for T tokens: idx [T,2] int32 (slot 0 = larger logit), w [T,2]
 * fp64, logits [T,E] fp64 (may be NULL).  Returns 0, or -1 on bad sizes. */
int oracle_route(int T, int d, int E, int k, const void *x, const void *wg, int dtype,
                 int32_t *idx, double *w, double *logits, int threads) {
    if (T < 0 || d < 1 || E < 1 || E > 256 || k < 1 || k > ORC_MAX_K || k > E) return -1;
    layer_ctx c = {T, d, 0, E, k, dtype, x, wg, NULL, NULL, NULL, idx, w, logits, NULL};
    parallel_for(T, threads, route_range, &c);
    return 0;
}

/* The router in the page's own order of steps (section 05, MoERouter:
 * softmax over all E logits, top-k of the probabilities, divide the kept
 * probabilities by their sum), for one token:
 *   p[e]  = exp(l[e] - m) / sum_e' exp(l[e'] - m),  m = max_e l[e]
 *           (subtracting m changes nothing mathematically and keeps exp finite)
 *   picks = greedy largest p among the experts not yet picked, decided on p
 *           rounded to fp32 (the GPU's precision), ties to the lower index
 *   w_s   = p[i_s] / (p[i_0] + ... + p[i_{k-1}])
 * Mathematically the picks and weights equal topk_softmax's; only rounding
 * differs. */
static void softmax_topk(int E, int k, const double *l, double *p, int32_t *idx, double *w) {
    double m = l[0];
    for (int e = 1; e < E; ++e) if (l[e] > m) m = l[e];
    double z = 0.0;
    for (int e = 0; e < E; ++e) { p[e] = exp(l[e] - m); z += p[e]; }
    for (int e = 0; e < E; ++e) p[e] /= z;
    for (int s = 0; s < k; ++s) {
        int pick = -1;
        for (int e = 0; e < E; ++e) {
            int used = 0;
            for (int r = 0; r < s; ++r) used |= idx[r] == e;
            if (!used && (pick < 0 || (float)p[e] > (float)p[pick])) pick = e;
        }
        idx[s] = pick;
    }
    double kept = 0.0;
    for (int s = 0; s < k; ++s) kept += p[idx[s]];
    for (int s = 0; s < k; ++s) w[s] = p[idx[s]] / kept;
}

typedef struct {
    int T, d, E, k, dtype;
    const void *x, *wg;
    double *probs;
    int32_t *idx;
    double *w;
} probs_ctx;

static void route_probs_range(void *p, int lo, int hi) {
    probs_ctx *c = (probs_ctx *)p;
    double l[256];
    for (int t = lo; t < hi; ++t) {
        router_logits(c->d, c->E, c->x, (size_t)t * c->d, c->wg, c->dtype, l);
        softmax_topk(c->E, c->k, l, c->probs + (size_t)t * c->E, c->idx + (size_t)c->k * t,
                     c->w + (size_t)c->k * t);
    }
}

/* Page-form router for T tokens: probs [T,E], idx [T,k], w [T,k] (fp64 but
 * idx).  Returns 0, or -1 on bad sizes. */
int oracle_route_probs(int T, int d, int E, int k, const void *x, const void *wg, int dtype,
                       double *probs, int32_t *idx, double *w, int threads) {
    if (T < 0 || d < 1 || E < 1 || E > 256 || k < 1 || k > ORC_MAX_K || k > E) return -1;
    probs_ctx c = {T, d, E, k, dtype, x, wg, probs, idx, w};
    parallel_for(T, threads, route_probs_range, &c);
    return 0;
}

typedef struct {
    int n, d, f, dtype;
    const void *rows;          /* [n, d] */
    const int32_t *expert;     /* [n]    */
    const void *w1, *w3, *w2;
    double *out;               /* [n, d] */
} rows_ctx;

static void expert_rows_range(void *p, int lo, int hi) {
    rows_ctx *c = (rows_ctx *)p;
    double *xr = malloc(sizeof(double) * c->d);
    double *g = malloc(sizeof(double) * c->f);
    double *u = malloc(sizeof(double) * c->f);
    if (!xr || !g || !u) { free(xr); free(g); free(u); return; }
    for (int r = lo; r < hi; ++r) {
        for (int j = 0; j < c->d; ++j)
            xr[j] = load_elem(c->rows, c->dtype, (size_t)r * c->d + j);
        swiglu_expert(c->d, c->f, xr, c->expert[r], c->w1, c->w3, c->w2,
                      c->dtype, g, u, c->out + (size_t)r * c->d);
    }
    free(xr); free(g); free(u);
}

/* Step 4 alone: out[r] = expert(expert[r]) applied to rows[r], fp64.
 * Returns 0, or -1 on bad sizes / expert ids out of [0, E). */
int oracle_expert_rows(int n, int d, int f, int E, const void *rows,
                       const int32_t *expert, const void *w1, const void *w3,
                       const void *w2, int dtype, double *out, int threads) {
    if (n < 0 || d < 1 || f < 1) return -1;
    for (int r = 0; r < n; ++r)
        if (expert[r] < 0 || expert[r] >= E) return -1;
    rows_ctx c = {n, d, f, dtype, rows, expert, w1, w3, w2, out};
    parallel_for(n, threads, expert_rows_range, &c);
    return 0;
}

typedef struct {
    int n, d, f, dtype, mode;  /* mode 0: hidden a [n,f] from rows [n,d];
                                  mode 1: down o [n,d] from rows [n,f] */
    const void *rows;
    const int32_t *expert;
    const void *w1, *w3, *w2;
    double *out;
} stage_ctx;

static void stage_range(void *p, int lo, int hi) {
    stage_ctx *c = (stage_ctx *)p;
    int in_w = c->mode == 0 ? c->d : c->f;
    double *xr = malloc(sizeof(double) * in_w);
    double *u = malloc(sizeof(double) * c->f);
    if (!xr || !u) { free(xr); free(u); return; }
    for (int r = lo; r < hi; ++r) {
        for (int j = 0; j < in_w; ++j)
            xr[j] = load_elem(c->rows, c->dtype, (size_t)r * in_w + j);
        if (c->mode == 0)
            swiglu_hidden(c->d, c->f, xr, c->expert[r], c->w1, c->w3, c->dtype,
                          c->out + (size_t)r * c->f, u);
        else
            swiglu_down(c->d, c->f, xr, c->expert[r], c->w2, c->dtype,
                        c->out + (size_t)r * c->d);
    }
    free(xr); free(u);
}

/* Step 4a alone: out[r] (fp64 [n,f]) = silu(rows[r] W1[e]) * (rows[r] W3[e]),
 * e = expert[r].  Returns 0, or -1 on bad sizes / expert ids. */
int oracle_expert_hidden(int n, int d, int f, int E, const void *rows,
                         const int32_t *expert, const void *w1, const void *w3,
                         int dtype, double *out, int threads) {
    if (n < 0 || d < 1 || f < 1) return -1;
    for (int r = 0; r < n; ++r)
        if (expert[r] < 0 || expert[r] >= E) return -1;
    stage_ctx c = {n, d, f, dtype, 0, rows, expert, w1, w3, NULL, out};
    parallel_for(n, threads, stage_range, &c);
    return 0;
}

/* Step 4b alone: out[r] (fp64 [n,d]) = hid[r] W2[e], hid [n,f] in the
 * input dtype, e = expert[r].  Returns 0, or -1 on bad sizes / expert ids. */
int oracle_expert_down(int n, int d, int f, int E, const void *hid,
                       const int32_t *expert, const void *w2, int dtype,
                       double *out, int threads) {
    if (n < 0 || d < 1 || f < 1) return -1;
    for (int r = 0; r < n; ++r)
        if (expert[r] < 0 || expert[r] >= E) return -1;
    stage_ctx c = {n, d, f, dtype, 1, hid, expert, NULL, NULL, w2, out};
    parallel_for(n, threads, stage_range, &c);
    return 0;
}

static void forward_range(void *p, int lo, int hi) {
    layer_ctx *c = (layer_ctx *)p;
    double l[256];
    double *xr = malloc(sizeof(double) * c->d);
    double *os = malloc(sizeof(double) * c->d * ORC_MAX_K);
    double *g = malloc(sizeof(double) * c->f);
    double *u = malloc(sizeof(double) * c->f);
    if (!xr || !os || !g || !u) goto out;
    for (int t = lo; t < hi; ++t) {
        size_t xo = (size_t)t * c->d;
        int32_t *it = c->idx + (size_t)c->k * t;
        double *wt = c->w + (size_t)c->k * t;
        router_logits(c->d, c->E, c->x, xo, c->wg, c->dtype, l);
        if (c->logits)
            for (int e = 0; e < c->E; ++e) c->logits[(size_t)t * c->E + e] = l[e];
        topk_softmax(c->E, c->k, l, it, wt);
        for (int j = 0; j < c->d; ++j) xr[j] = load_elem(c->x, c->dtype, xo + j);
        for (int s = 0; s < c->k; ++s)
            swiglu_expert(c->d, c->f, xr, it[s], c->w1, c->w3, c->w2, c->dtype, g, u,
                          os + (size_t)s * c->d);
        for (int m = 0; m < c->d; ++m) {                     /* step 5, slot order */
            double acc = 0.0;
            for (int s = 0; s < c->k; ++s) acc += wt[s] * os[(size_t)s * c->d + m];
            c->y[xo + m] = acc;
        }
    }
out:
    free(xr); free(os); free(g); free(u);
}
int oracle_forward(int T, int d, int f, int E, int k, const void *x, const void *wg,
                   const void *w1, const void *w3, const void *w2, int dtype,
                   double *y, int32_t *idx, double *w, double *logits, int threads) {
    if (T < 0 || d < 1 || f < 1 || E < 1 || E > 256 || k < 1 || k > ORC_MAX_K || k > E)
        return -1;
    layer_ctx c = {T, d, f, E, k, dtype, x, wg, w1, w3, w2, idx, w, logits, y};
    parallel_for(T, threads, forward_range, &c);
    return 0;
}

/* ------------------------------------------------------------------------
 * Backward.  The pages train the router and the experts together and name
 * no loss, capacity or auxiliary term, so the backward is the gradient of
 * the forward above as written, for a given upstream gradient dy [T,d]
 * (L = sum_t dy[t] . y[t]).  The top-k picks are a discrete choice: they
 * stay fixed, and the gradient reaches the router only through the softmax
 * over the picked logits.  Per token t and slot s (e = i_s):
 *
 *   dw_s   = dy . o_s                             (o_s the expert's output)
 *   dl_e   = w_s (dw_s - sum_r w_r dw_r)          (softmax Jacobian; 0 for
 *                                                  experts not picked)
 *   do_s   = w_s dy
 *   da     = do_s W2[e]^T,   da_n = sum_m do_m W2[e][n][m]
 *   dg     = da * u * silu'(g),  silu'(g) = sig(g) (1 + g (1 - sig(g)))
 *   du     = da * silu(g)
 *   dx    += dg W1[e]^T + du W3[e]^T             (slots in order)
 *   dW1[e] += x^T dg,  dW3[e] += x^T du,  dW2[e] += a^T do_s
 *   dx    += dl Wg^T,    dWg += x^T dl
 *
 * Weight gradients sum over tokens in token order (then slot order).  */

typedef struct {
    int T, d, f, E, k, dtype;
    const void *x, *wg, *w1, *w3, *w2;
    const double *dy;                 /* [T, d] */
    int32_t *idx;                     /* [T, k] */
    double *w;                        /* [T, k] */
    double *dx;                       /* [T, d] */
    double *dl;                       /* [T, E] */
    double *a, *dg, *du, *dov;        /* per assignment: [R, f] x3, [R, d] */
} bwd_ctx;

static void bwd_token_range(void *p, int lo, int hi) {
    bwd_ctx *c = (bwd_ctx *)p;
    const int d = c->d, f = c->f, E = c->E, k = c->k;
    double l[256], dws[ORC_MAX_K];
    double *xr = malloc(sizeof(double) * d);
    double *g = malloc(sizeof(double) * f);
    double *u = malloc(sizeof(double) * f);
    double *o = malloc(sizeof(double) * d);
    double *da = malloc(sizeof(double) * f);
    if (!xr || !g || !u || !o || !da) goto out;
    for (int t = lo; t < hi; ++t) {
        const size_t xo = (size_t)t * d;
        int32_t *it = c->idx + (size_t)k * t;
        double *wt = c->w + (size_t)k * t;
        const double *dyt = c->dy + xo;
        double *dxt = c->dx + xo;
        router_logits(d, E, c->x, xo, c->wg, c->dtype, l);
        topk_softmax(E, k, l, it, wt);
        for (int j = 0; j < d; ++j) { xr[j] = load_elem(c->x, c->dtype, xo + j); dxt[j] = 0.0; }
        for (int s = 0; s < k; ++s) {
            const int e = it[s];
            const size_t r = (size_t)k * t + s;
            double *ar = c->a + r * f, *dgr = c->dg + r * f, *dur = c->du + r * f;
            double *dor = c->dov + r * d;
            /* forward pieces: g, u, a, o */
            const size_t in_base = (size_t)e * d * f;
            for (int n = 0; n < f; ++n) { g[n] = 0.0; u[n] = 0.0; }
            for (int j = 0; j < d; ++j) {
                const size_t row = in_base + (size_t)j * f;
                for (int n = 0; n < f; ++n) {
                    g[n] += xr[j] * load_elem(c->w1, c->dtype, row + n);
                    u[n] += xr[j] * load_elem(c->w3, c->dtype, row + n);
                }
            }
            for (int n = 0; n < f; ++n) ar[n] = u[n] * g[n] * (1.0 / (1.0 + exp(-g[n])));
            const size_t out_base = (size_t)e * f * d;
            for (int m = 0; m < d; ++m) o[m] = 0.0;
            for (int n = 0; n < f; ++n) {
                const size_t row = out_base + (size_t)n * d;
                for (int m = 0; m < d; ++m) o[m] += ar[n] * load_elem(c->w2, c->dtype, row + m);
            }
            /* dw_s, do_s */
            double acc = 0.0;
            for (int m = 0; m < d; ++m) acc += dyt[m] * o[m];
            dws[s] = acc;
            for (int m = 0; m < d; ++m) dor[m] = wt[s] * dyt[m];
            /* da = do W2[e]^T */
            for (int n = 0; n < f; ++n) {
                const size_t row = out_base + (size_t)n * d;
                double v = 0.0;
                for (int m = 0; m < d; ++m) v += dor[m] * load_elem(c->w2, c->dtype, row + m);
                da[n] = v;
            }
            /* dg, du */
            for (int n = 0; n < f; ++n) {
                const double sg = 1.0 / (1.0 + exp(-g[n]));
                dgr[n] = da[n] * u[n] * sg * (1.0 + g[n] * (1.0 - sg));
                dur[n] = da[n] * g[n] * sg;
            }
            /* dx += dg W1[e]^T + du W3[e]^T */
            for (int j = 0; j < d; ++j) {
                const size_t row = in_base + (size_t)j * f;
                double v = 0.0;
                for (int n = 0; n < f; ++n)
                    v += dgr[n] * load_elem(c->w1, c->dtype, row + n) +
                         dur[n] * load_elem(c->w3, c->dtype, row + n);
                dxt[j] += v;
            }
        }
        /* router: softmax Jacobian over the picked logits */
        double mean = 0.0;
        for (int s = 0; s < k; ++s) mean += wt[s] * dws[s];
        double *dlt = c->dl + (size_t)t * E;
        for (int e = 0; e < E; ++e) dlt[e] = 0.0;
        for (int s = 0; s < k; ++s) dlt[it[s]] = wt[s] * (dws[s] - mean);
        for (int j = 0; j < d; ++j) {
            double v = 0.0;
            for (int e = 0; e < E; ++e) v += dlt[e] * load_elem(c->wg, c->dtype, (size_t)j * E + e);
            dxt[j] += v;
        }
    }
out:
    free(xr); free(g); free(u); free(o); free(da);
}

typedef struct {
    const bwd_ctx *c;
    double *dwg, *dw1, *dw3, *dw2;
} bwd_w_ctx;

/* Weight gradients, one (expert, input row) of each matrix per item:
 * items [0, E*d) are rows j of dW1[e] / dW3[e], items [E*d, E*d + E*f) rows
 * n of dW2[e], items past that rows j of dWg.  Each sums over tokens in
 * order, then slots. */
static void bwd_weight_range(void *p, int lo, int hi) {
    const bwd_w_ctx *wc = (const bwd_w_ctx *)p;
    const bwd_ctx *c = wc->c;
    const int d = c->d, f = c->f, E = c->E, k = c->k, T = c->T;
    for (int item = lo; item < hi; ++item) {
        if (item < E * d) {
            const int e = item / d, j = item % d;
            double *r1 = wc->dw1 + ((size_t)e * d + j) * f, *r3 = wc->dw3 + ((size_t)e * d + j) * f;
            for (int n = 0; n < f; ++n) { r1[n] = 0.0; r3[n] = 0.0; }
            for (int t = 0; t < T; ++t)
                for (int s = 0; s < k; ++s) {
                    if (c->idx[(size_t)k * t + s] != e) continue;
                    const double xj = load_elem(c->x, c->dtype, (size_t)t * d + j);
                    const size_t r = (size_t)k * t + s;
                    for (int n = 0; n < f; ++n) {
                        r1[n] += xj * c->dg[r * f + n];
                        r3[n] += xj * c->du[r * f + n];
                    }
                }
        } else if (item < E * d + E * f) {
            const int it2 = item - E * d, e = it2 / f, n = it2 % f;
            double *r2 = wc->dw2 + ((size_t)e * f + n) * d;
            for (int m = 0; m < d; ++m) r2[m] = 0.0;
            for (int t = 0; t < T; ++t)
                for (int s = 0; s < k; ++s) {
                    if (c->idx[(size_t)k * t + s] != e) continue;
                    const size_t r = (size_t)k * t + s;
                    const double an = c->a[r * f + n];
                    for (int m = 0; m < d; ++m) r2[m] += an * c->dov[r * d + m];
                }
        } else {
            const int j = item - E * d - E * f;
            double *rg = wc->dwg + (size_t)j * E;
            for (int e = 0; e < E; ++e) rg[e] = 0.0;
            for (int t = 0; t < T; ++t) {
                const double xj = load_elem(c->x, c->dtype, (size_t)t * d + j);
                for (int e = 0; e < E; ++e) rg[e] += xj * c->dl[(size_t)t * E + e];
            }
        }
    }
}

/* Gradients of L = sum(dy * y) for the layer: dx [T,d], dwg [d,E], dw1 and
 * dw3 [E,d,f], dw2 [E,f,d] (all fp64), plus the routing (idx, w).  Returns
 * 0, -1 on bad sizes, -2 when out of memory. */
int oracle_backward(int T, int d, int f, int E, int k, const void *x, const void *wg,
                    const void *w1, const void *w3, const void *w2, int dtype, const double *dy,
                    double *dx, double *dwg, double *dw1, double *dw3, double *dw2,
                    int32_t *idx, double *w, int threads) {
    if (T < 0 || d < 1 || f < 1 || E < 1 || E > 256 || k < 1 || k > ORC_MAX_K || k > E)
        return -1;
    const size_t R = (size_t)T * k;
    double *dl = calloc((size_t)T * E + 1, sizeof(double));
    double *a = malloc(sizeof(double) * (R * f + 1));
    double *dg = malloc(sizeof(double) * (R * f + 1));
    double *du = malloc(sizeof(double) * (R * f + 1));
    double *dov = malloc(sizeof(double) * (R * d + 1));
    int rc = 0;
    if (!dl || !a || !dg || !du || !dov) { rc = -2; goto out; }
    bwd_ctx c = {T, d, f, E, k, dtype, x, wg, w1, w3, w2, dy, idx, w, dx, dl, a, dg, du, dov};
    parallel_for(T, threads, bwd_token_range, &c);
    bwd_w_ctx wc = {&c, dwg, dw1, dw3, dw2};
    parallel_for(E * d + E * f + d, threads, bwd_weight_range, &wc);
out:
    free(dl); free(a); free(dg); free(du); free(dov);
    return rc;
}

/* ------------------------------------------------------------------------
 * Weight-only int8 expert weights.
 *
 * The pages name weight-only int8 loading for this model (the KerasFormers
 * Mixtral page's loading example: quantization="int8" with low-memory
 * loading) but give no scheme.  The plainest one is used: symmetric, one
 * scale per output channel of each expert matrix.  For a matrix W [K, N]
 * (K = input, N = output channel) and each column n:
 *
 *   a[n]    = max_j |W[j,n]|
 *   s[n]    = a[n] / 127            (fp32 division; s = 0 for a zero column)
 *   q[j,n]  = rint(W[j,n] / s[n])   (fp32 division, round half to even,
 *                                    clamped to [-127, 127]; q = 0 when s = 0)
 *
 * The division and the rounding are the decision that produces an integer,
 * so they are taken in fp32, the precision the GPU library takes them in.
 * The layer then uses W~[j,n] = s[n] * q[j,n] in place of W: with the scale
 * taken out of each sum, g[n] = s1[n] * sum_j x[j] q1[j,n] and likewise for
 * u and the down projection, all in fp64.  */

static void quantize_column(int K, int N, const void *w, int dtype, size_t base, int n,
                            int8_t *q, float *scale) {
    float a = 0.0f;
    for (int j = 0; j < K; ++j) {
        const float v = fabsf((float)load_elem(w, dtype, base + (size_t)j * N + n));
        if (v > a) a = v;
    }
    const float sc = a / 127.0f;
    *scale = sc;
    for (int j = 0; j < K; ++j) {
        int8_t code = 0;
        if (sc > 0.0f) {
            float r = rintf((float)load_elem(w, dtype, base + (size_t)j * N + n) / sc);
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            code = (int8_t)r;
        }
        q[base + (size_t)j * N + n] = code;
    }
}

typedef struct {
    int K, N, dtype;
    const void *w;
    int8_t *q;
    float *scale;
} quant_ctx;

static void quantize_range(void *p, int lo, int hi) {
    quant_ctx *c = (quant_ctx *)p;
    for (int col = lo; col < hi; ++col) {        /* col = e * N + n */
        const int e = col / c->N, n = col % c->N;
        quantize_column(c->K, c->N, c->w, c->dtype, (size_t)e * c->K * c->N, n, c->q,
                        c->scale + col);
    }
}

/* E matrices W [E, K, N] -> q int8 [E, K, N], scale fp32 [E, N]. */
int oracle_quantize_int8(int E, int K, int N, const void *w, int dtype, int8_t *q,
                         float *scale, int threads) {
    if (E < 1 || K < 1 || N < 1) return -1;
    quant_ctx c = {K, N, dtype, w, q, scale};
    parallel_for(E * N, threads, quantize_range, &c);
    return 0;
}

typedef struct {
    int T, d, f, E, k, dtype;
    const void *x, *wg;
    const int8_t *q1, *q3, *q2;
    const float *s1, *s3, *s2;
    int32_t *idx;
    double *w, *y;
} w8_ctx;

/* a = silu(x W~1[e]) * (x W~3[e]) into g[f]; u is scratch [f]. */
static void w8_hidden(const w8_ctx *c, const double *xr, int e, double *g, double *u) {
    const int d = c->d, f = c->f;
    const size_t base = (size_t)e * d * f;
    for (int n = 0; n < f; ++n) { g[n] = 0.0; u[n] = 0.0; }
    for (int j = 0; j < d; ++j) {
        const double xj = xr[j];
        const size_t row = base + (size_t)j * f;
        for (int n = 0; n < f; ++n) {
            g[n] += xj * (double)c->q1[row + n];
            u[n] += xj * (double)c->q3[row + n];
        }
    }
    for (int n = 0; n < f; ++n) {
        const double gn = (double)c->s1[(size_t)e * f + n] * g[n];
        const double un = (double)c->s3[(size_t)e * f + n] * u[n];
        g[n] = gn / (1.0 + exp(-gn)) * un;
    }
}

/* o[d] = a[f] W~2[e]. */
static void w8_down(const w8_ctx *c, const double *a, int e, double *o) {
    const int d = c->d, f = c->f;
    const size_t base = (size_t)e * f * d;
    for (int m = 0; m < d; ++m) o[m] = 0.0;
    for (int n = 0; n < f; ++n) {
        const double an = a[n];
        const size_t row = base + (size_t)n * d;
        for (int m = 0; m < d; ++m) o[m] += an * (double)c->q2[row + m];
    }
    for (int m = 0; m < d; ++m) o[m] *= (double)c->s2[(size_t)e * d + m];
}

static void w8_forward_range(void *p, int lo, int hi) {
    w8_ctx *c = (w8_ctx *)p;
    double l[256];
    double *xr = malloc(sizeof(double) * c->d);
    double *os = malloc(sizeof(double) * c->d * ORC_MAX_K);
    double *g = malloc(sizeof(double) * c->f);
    double *u = malloc(sizeof(double) * c->f);
    if (!xr || !os || !g || !u) goto out;
    for (int t = lo; t < hi; ++t) {
        const size_t xo = (size_t)t * c->d;
        int32_t *it = c->idx + (size_t)c->k * t;
        double *wt = c->w + (size_t)c->k * t;
        router_logits(c->d, c->E, c->x, xo, c->wg, c->dtype, l);
        topk_softmax(c->E, c->k, l, it, wt);
        for (int j = 0; j < c->d; ++j) xr[j] = load_elem(c->x, c->dtype, xo + j);
        for (int s = 0; s < c->k; ++s) {
            w8_hidden(c, xr, it[s], g, u);
            w8_down(c, g, it[s], os + (size_t)s * c->d);
        }
        for (int m = 0; m < c->d; ++m) {                     /* slot order */
            double acc = 0.0;
            for (int s = 0; s < c->k; ++s) acc += os[(size_t)s * c->d + m] * wt[s];
            c->y[xo + m] = acc;
        }
    }
out:
    free(xr); free(os); free(g); free(u);
}

typedef struct {
    const w8_ctx *c;
    int mode;                  /* 0: hidden a [n,f] from rows [n,d]; 1: down o [n,d] from [n,f] */
    const void *rows;          /* layer dtype */
    const int32_t *expert;
    double *out;
} w8_stage_ctx;

static void w8_stage_range(void *p, int lo, int hi) {
    const w8_stage_ctx *sc = (const w8_stage_ctx *)p;
    const w8_ctx *c = sc->c;
    const int in_w = sc->mode == 0 ? c->d : c->f;
    double *xr = malloc(sizeof(double) * in_w);
    double *u = malloc(sizeof(double) * c->f);
    if (!xr || !u) { free(xr); free(u); return; }
    for (int r = lo; r < hi; ++r) {
        for (int j = 0; j < in_w; ++j)
            xr[j] = load_elem(sc->rows, c->dtype, (size_t)r * in_w + j);
        if (sc->mode == 0)
            w8_hidden(c, xr, sc->expert[r], sc->out + (size_t)r * c->f, u);
        else
            w8_down(c, xr, sc->expert[r], sc->out + (size_t)r * c->d);
    }
    free(xr); free(u);
}

/* The int8 gate/up stage alone: out [n,f] = silu(s1 (rows q1[e])) * (s3 (rows q3[e])),
 * e = expert[r] (mode 0); or the down stage: out [n,d] = s2 (rows q2[e]) (mode 1).
 * rows are in `dtype`.  Returns 0, or -1 on bad sizes / expert ids. */
int oracle_expert_stage_w8(int mode, int n, int d, int f, int E, const void *rows,
                           const int32_t *expert, int dtype, const int8_t *q1, const float *s1,
                           const int8_t *q3, const float *s3, const int8_t *q2,
                           const float *s2, double *out, int threads) {
    if (n < 0 || d < 1 || f < 1 || (mode != 0 && mode != 1)) return -1;
    for (int r = 0; r < n; ++r)
        if (expert[r] < 0 || expert[r] >= E) return -1;
    w8_ctx c = {0, d, f, E, 1, dtype, NULL, NULL, q1, q3, q2, s1, s3, s2, NULL, NULL, NULL};
    w8_stage_ctx sc = {&c, mode, rows, expert, out};
    parallel_for(n, threads, w8_stage_range, &sc);
    return 0;
}

/* The layer with int8 expert weights (router and x in `dtype`): y [T,d]
 * fp64, idx [T,k], w [T,k]. */
int oracle_forward_w8(int T, int d, int f, int E, int k, const void *x, const void *wg,
                      int dtype, const int8_t *q1, const float *s1, const int8_t *q3,
                      const float *s3, const int8_t *q2, const float *s2, double *y,
                      int32_t *idx, double *w, int threads) {
    if (T < 0 || d < 1 || f < 1 || E < 1 || E > 256 || k < 1 || k > ORC_MAX_K || k > E)
        return -1;
    w8_ctx c = {T, d, f, E, k, dtype, x, wg, q1, q3, q2, s1, s3, s2, idx, w, y};
    parallel_for(T, threads, w8_forward_range, &c);
    return 0;
}

/* ------------------------------------------------------------------------
 * Block boundary: RMSNorm before the layer.  */

/* v rounded to the nearest bf16 value (8 significant bits), ties to even,
 * taken directly from the double (no intermediate rounding to fp32). */
static double round_bf16(double v) {
    if (v == 0.0 || !isfinite(v)) return v;
    int ex;
    const double m = frexp(v, &ex);            /* |m| in [0.5, 1) */
    const double r = nearbyint(ldexp(m, 8));   /* 8 significant bits, RNE */
    return ldexp(r, ex - 8);
}

static void store_elem(void *p, int dtype, size_t i, double v) {
    if (dtype == ORC_F32) {
        ((float *)p)[i] = (float)v;            /* C conversion: round to nearest even */
    } else {
        const float f = (float)round_bf16(v);  /* exact: 8 significant bits */
        uint32_t bits;
        memcpy(&bits, &f, sizeof bits);
        ((uint16_t *)p)[i] = (uint16_t)(bits >> 16);
    }
}

struct norm_ctx {
    int d, dtype;
    const void *h, *g;
    double eps;
    void *xn;
    double *rstd;
};

static void norm_range(void *p, int lo, int hi) {
    const struct norm_ctx *c = (const struct norm_ctx *)p;
    for (int t = lo; t < hi; ++t) {
        const size_t row = (size_t)t * c->d;
        double ss = 0.0;
        for (int j = 0; j < c->d; ++j) {
            const double v = load_elem(c->h, c->dtype, row + j);
            ss += v * v;
        }
        const double r = 1.0 / sqrt(ss / (double)c->d + c->eps);
        c->rstd[t] = r;
        for (int j = 0; j < c->d; ++j)
            store_elem(c->xn, c->dtype, row + j,
                       load_elem(c->h, c->dtype, row + j) * r * load_elem(c->g, c->dtype, j));
    }
}

/* xn [T,d] in the layer dtype and rstd [T] (fp64) from h [T,d] and the
 * norm's per-channel weight g [d]. */
int oracle_rmsnorm(int T, int d, const void *h, const void *g, double eps, int dtype,
                   void *xn, double *rstd, int threads) {
    if (T < 0 || d <= 0 || !(eps >= 0.0)) return 1;
    struct norm_ctx c = {d, dtype, h, g, eps, xn, rstd};
    parallel_for(T, threads, norm_range, &c);
    return 0;
}

