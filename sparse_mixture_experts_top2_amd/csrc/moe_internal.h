// Internal declarations shared by the HIP translation units of libmoe:
// workspace planning, device helpers and the kernel launchers that the
// C interface (abi.hip) sequences.  Not installed; include/moe.h is the
// public surface.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kMaxExperts = 64;
constexpr int kMaxTopK = 4;     // experts per token
// Token counts up to this use the weight-streaming (decode) expert kernels;
// an expert then has at most 32 rows (a token never picks one expert twice,
// whatever top_k is).
constexpr int kDecodeMaxT = 32;
// K slices of the int8-weight down projection at decode sizes; the combine
// adds the slices in order.  The workspace's o region holds this many
// copies of o when T <= kDecodeMaxT (kMaxDownSplit copies above it).
constexpr int kDownParts = 2;
// Most K parts the prefill down product is cut into (see launch_down_split_bf16).
constexpr int kMaxDownSplit = 2;
// Decode gate/up: most (expert, 128-column) units cut in K halves to fill the
// last round of workgroups, and the fp32 partial sums they need (2 halves x
// 2 matrices x 32 rows x 128 columns each).
constexpr int kDecodeTailMaxUnits = 256;
constexpr size_t kDecodeTailBytes = (size_t)kDecodeTailMaxUnits * 2 * 2 * 32 * 128 * 4;

// Whether the decode kernels request their first weights before reading
// the routing (which they need only for the activation rows): when the
// routed rows are at least twice the experts, an expert holds no rows with
// probability about exp(-2) or less under near-uniform routing, and each
// such expert's workgroups waste one K step of their weights.
inline int decode_early_weights(int rows, int E) { return rows >= 2 * E ? 1 : 0; }

// parts: one int32, the K part count the prefill down kernel chose.
// gpart: at bf16 decode sizes, the decode gate/up's K-half partial sums.
struct Layout {
    size_t idx, w, counts, offsets, pos, src, xn, xp, h, o, parts, gpart, total;
};

// Byte offsets of every workspace region for this shape (256-byte aligned).
Layout plan_workspace(const moe_shape_t &s);

// Workspace of the backward (backward.hip): routing, grouped rows xp, the
// recomputed g, u (fp32) and h, the expert outputs o (later the per-row
// input gradients), dO, dG, dU (layer dtype) and the router gradient dl.
// o holds kMaxDownSplit partial sums (the split products' K parts); nparts
// two int32, the part counts the o and dXp products chose.
// At bf16 sizes the weight-gradient GEMMs take, xpT, hT, dOT, dGT and dUT
// hold K-contiguous copies of xp, h, dO, dG and dU whose columns are the
// grouped rows padded per expert to a multiple of 64 (q_dw_ldk columns);
// otherwise those regions are empty.
struct BackwardLayout {
    size_t idx, w, counts, offsets, pos, xp, g, u, h, o, dout, dg, du, dl, dwgp, nparts;
    size_t xpT, hT, dOT, dGT, dUT, total;
    int ldk;   // row length of the K-contiguous copies (0: not used)
};
BackwardLayout plan_backward(const moe_shape_t &s);
hipError_t launch_backward(const moe_shape_t &s, const void *x, const void *wg, const void *w1,
                           const void *w3, const void *w2, const void *dy, void *dx, float *dwg,
                           float *dw1, float *dw3, float *dw2, const BackwardLayout &L,
                           char *base, hipStream_t stream);

inline size_t elem_bytes(int dtype) { return dtype == MOE_BF16 ? 2 : 4; }
// Routed rows: top_k per token.
inline int routed_rows(const moe_shape_t &s) { return s.top_k * s.T; }

// ---------------------------------------------------------------------------
// Kernel launchers.  Each enqueues on `stream` and returns hipGetLastError().

hipError_t launch_route(const moe_shape_t &s, const void *x, const void *w_gate,
                        int32_t *idx, float *w, hipStream_t stream);
// Router on the RMSNorm of x (weight g, eps); writes the normalised rows to
// xn (layer dtype).  g == NULL: plain launch_route.
hipError_t launch_route_norm(const moe_shape_t &s, const void *x, const void *g, float eps,
                             const void *w_gate, void *xn, int32_t *idx, float *w,
                             hipStream_t stream);

// Router in the page's order of steps: softmax over all E logits, top-k
// of the probabilities, kept probabilities renormalised; probs [T, E] is
// written when not NULL.
hipError_t launch_route_probs(const moe_shape_t &s, const void *x, const void *w_gate,
                              float *probs, int32_t *idx, float *w, hipStream_t stream);

hipError_t launch_dispatch(const moe_shape_t &s, const void *x, const int32_t *idx,
                           int32_t *counts, int32_t *offsets, int32_t *pos, void *xp,
                           hipStream_t stream);
// The ranking half of the dispatch alone (counts, offsets, pos), plus, when
// src is not NULL, src[r] = the token of grouped row r, for kernels that
// gather their rows from x instead of reading xp.
hipError_t launch_rank(const moe_shape_t &s, const int32_t *idx, int32_t *counts,
                       int32_t *offsets, int32_t *pos, int32_t *src, hipStream_t stream);
// The same ranking, computed inside the decode gate/up kernel (T <= kDecodeMaxT:
// at most kDecodeMaxT * kMaxTopK assignments) instead of by its own launch:
// every workgroup ranks the routing picks idx for itself (one wavefront, from
// L2), and workgroup 0 also stores counts, offsets, pos and src for the
// kernels after it.
struct DecodeRank {
    const int32_t *idx;   // [T * top_k] routing picks
    int n_assign, top_k;
    int32_t *counts, *offsets, *pos, *src;
};

// DecodeRank's ranking by one wavefront (at most 128 assignments, E <= 64):
// lane x counts expert x's picks in each 64-pick batch (ballots), an
// inclusive scan over the lanes gives the offsets, and each pick's grouped
// row is its expert's offset + the expert's picks in earlier batches + those
// on lower lanes of its own batch -- the stable order of dispatch_rank_kernel.
// s_counts / s_offsets / s_src get the result (the caller's barrier makes it
// visible); with to_global the outputs of DecodeRank are written too.
__device__ __forceinline__ void decode_rank_wave(const DecodeRank &rk, int E, int lane,
                                                 int32_t *s_counts, int32_t *s_offsets,
                                                 int32_t *s_src, bool to_global) {
    const uint64_t lower = (1ull << lane) - 1ull;
    int ev[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int a = 64 * b + lane;
        ev[b] = a < rk.n_assign ? (int)min((unsigned)rk.idx[a], (unsigned)(E - 1)) : -1;
    }
    int c0 = 0, c1 = 0;
    uint64_t mine0 = 0, mine1 = 0;
    for (int x = 0; x < E; ++x) {
        const uint64_t m0 = __ballot(ev[0] == x), m1 = __ballot(ev[1] == x);
        if (lane == x) {
            c0 = __popcll(m0);
            c1 = __popcll(m1);
        }
        if (ev[0] == x) mine0 = m0;
        if (ev[1] == x) mine1 = m1;
    }
    const int tot = c0 + c1;
    int inc = tot;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int u = __shfl_up(inc, off, 64);
        if (lane >= off) inc += u;
    }
    const int excl = inc - tot;
    if (lane < E) {
        s_counts[lane] = tot;
        s_offsets[lane] = excl;
        if (to_global) {
            rk.counts[lane] = tot;
            rk.offsets[lane] = excl;
        }
    }
    if (lane == E - 1) {
        s_offsets[E] = inc;
        if (to_global) rk.offsets[E] = inc;
    }
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int e = ev[b] < 0 ? 0 : ev[b];
        const int first = __shfl(excl, e, 64) + (b == 1 ? __shfl(c0, e, 64) : 0);
        if (ev[b] >= 0) {
            const int a = 64 * b + lane;
            const int p = first + __popcll((b == 0 ? mine0 : mine1) & lower);
            s_src[p] = a / rk.top_k;
            if (to_global) {
                rk.pos[a] = p;
                rk.src[p] = a / rk.top_k;
            }
        }
    }
}

// Grouped SwiGLU over expert-sorted rows, in two launches:
//   gate/up: h = silu(xp w1[e]) * (xp w3[e])    (h in the layer dtype)
//   down:    o = h w2[e]                          (o fp32)
hipError_t launch_gateup(const moe_shape_t &s, const void *xp, const int32_t *counts,
                         const int32_t *offsets, const void *w1, const void *w3, void *h,
                         hipStream_t stream);
// gpart as for launch_gateup_bf16 (bf16 decode sizes only; may be NULL).
hipError_t launch_down(const moe_shape_t &s, const void *h, const int32_t *counts,
                       const int32_t *offsets, const void *w2, float *o, hipStream_t stream,
                       float *gpart = nullptr);

// y = w0 o[pos0] + w1 o[pos1] + ... (+ res when res is not NULL), rounded
// once.  With parts > 1, o holds that many partial sums, each kT x d, one
// after the other; every row is their sum in order before it is weighted.
// parts_dev (device int32, may be NULL): the part count is read there
// instead of taken from `parts`.
hipError_t launch_combine(const moe_shape_t &s, const float *o, const int32_t *pos,
                          const float *w, void *y, hipStream_t stream,
                          const void *res = nullptr, int parts = 1,
                          const int *parts_dev = nullptr);

// Weight-only int8 (experts_w8.hip).  W [n_mat, K, N] (dtype) -> codes
// q [n_mat, K, N] and per-column scales [n_mat, N].
hipError_t launch_quantize_int8(int n_mat, int K, int N, int dtype, const void *w, int8_t *q,
                                float *scale, hipStream_t stream);
// Gate/up and down on int8 codes, T <= kDecodeMaxT only (bf16 activations).
// Down writes `parts` K-slice partial sums, each kT x d, one after another.
// Gate/up with rank (and src): it ranks the picks itself, as
// launch_gateup_bf16 does.  part (fp32, kDecodeTailBytes, may be NULL):
// room for the partial sums of the slabs cut to fill the last round.
hipError_t launch_gateup_w8(const moe_shape_t &s, const uint16_t *xp, const int32_t *counts,
                            const int32_t *offsets, const int8_t *q1, const float *s1,
                            const int8_t *q3, const float *s3, uint16_t *h, hipStream_t stream,
                            const int32_t *src = nullptr, const DecodeRank *rank = nullptr,
                            float *part = nullptr);
hipError_t launch_down_w8(const moe_shape_t &s, const uint16_t *h, const int32_t *counts,
                          const int32_t *offsets, const int8_t *q2, const float *s2, float *o,
                          int parts, hipStream_t stream);

// Per-dtype expert launchers (experts_f32.hip, experts_bf16.hip).  The bf16
// ones pick the weight-streaming kernels for T <= kDecodeMaxT.
hipError_t launch_gateup_f32(const moe_shape_t &s, const float *xp, const int32_t *counts,
                             const int32_t *offsets, const float *w1, const float *w3,
                             float *h, hipStream_t stream);
hipError_t launch_down_f32(const moe_shape_t &s, const float *h, const int32_t *counts,
                           const int32_t *offsets, const float *w2, float *o,
                           hipStream_t stream);
// With src not NULL (only for T <= kDecodeMaxT), row r of the activations
// is read from xp + src[r] * d_model, i.e. xp is x itself.  gpart (fp32,
// kDecodeTailBytes, may be NULL): room for the K halves' partial sums of
// the units the decode kernel cuts to fill its last round of workgroups.
// rank not NULL (decode sizes, with src): counts, offsets and src are
// outputs, made by the kernel from rank->idx (see DecodeRank).
hipError_t launch_gateup_bf16(const moe_shape_t &s, const uint16_t *xp, const int32_t *counts,
                              const int32_t *offsets, const uint16_t *w1, const uint16_t *w3,
                              uint16_t *h, hipStream_t stream, const int32_t *src = nullptr,
                              float *gpart = nullptr, const DecodeRank *rank = nullptr);
// The prefill gate/up kernel storing g and u (fp32 [kT, f]) beside h, for
// the backward.  hipErrorNotSupported when the shape does not take the
// direct-to-LDS kernel (T <= kDecodeMaxT, d % 64 or f % 128 not zero).
hipError_t launch_gateup_bf16_gu(const moe_shape_t &s, const uint16_t *xp,
                                 const int32_t *counts, const int32_t *offsets,
                                 const uint16_t *w1, const uint16_t *w3, uint16_t *h, float *g,
                                 float *u, hipStream_t stream);
// Backward products on the prefill pipeline with a K-contiguous B (a
// transposed expert matrix B[e] = B + e * N * K1, line n at n * K1), over
// grouped rows (counts / offsets).  The store form: C = A B[e]^T (+ A2
// B2[e]^T when A2 / B2 are not NULL, the second K1 of a 2 * K1 reduction),
// with the reduction cut into 1..kMaxDownSplit parts chosen on the device
// from the expert counts, part p stored at C + p * part_stride and the
// count stored to *parts_out.  The dswiglu form: da = A B[e]^T turned into
// dg, du (bf16) with g, u (fp32).  All arrays have row stride K1 (A, A2) or
// N (C, g, u, dg, du).  hipErrorNotSupported unless K1 % 64 == 0 and
// N % 256 == 0.
hipError_t launch_bt_store_split_bf16(int rows, int E, const uint16_t *A, const uint16_t *B,
                                      const uint16_t *A2, const uint16_t *B2, int K1, int N,
                                      const int32_t *counts, const int32_t *offsets, float *C,
                                      size_t part_stride, int *parts_out, hipStream_t stream);
hipError_t launch_bt_dswiglu_bf16(int rows, int E, const uint16_t *A, const uint16_t *B, int K1,
                                  int N, const int32_t *counts, const int32_t *offsets,
                                  const float *g, const float *u, uint16_t *dg, uint16_t *du,
                                  hipStream_t stream);
// Prefill down product with the reduction over K cut into `parts` runs of
// whole 64-wide stages: part p stores the sum over its run at o + p *
// part_stride (fp32 [rows, N] each).  parts = 0 lets the kernel choose 1 to
// kMaxDownSplit from the expert counts and the device's CU count, and store
// its choice to *parts_out (device memory) for the combine.
// hipErrorNotSupported unless K % 64 == 0, K / 64 >= kMaxDownSplit and
// N % 256 == 0.
hipError_t launch_down_split_bf16(int rows, int E, const uint16_t *h, const int32_t *counts,
                                  const int32_t *offsets, const uint16_t *w2, int K, int N,
                                  int parts, size_t part_stride, float *o, int *parts_out,
                                  hipStream_t stream);
// The software-pipelined prefill GEMMs (gemm_bf16.h and its gemm_*.hip units), over grouped rows
// (counts / offsets, `rows` = kT rows of xp / h).  Gate/up: h = silu(xp
// w1[e]) * (xp w3[e]) (bf16), with g, u not NULL also g = xp w1[e], u = xp
// w3[e] (fp32).  Down: o = h w2[e] (fp32); parts = 1 with parts_out NULL is
// the plain product, otherwise the split form of launch_down_split_bf16
// (cu_per_xcd: the device's CUs per XCD, for parts = 0).
// hipErrorNotSupported unless K % 64 == 0, N a multiple of 128 (gate/up)
// or 256 (down), rows * K * 2 < 2^32 and K * N * 2 < 2^32.
bool q_gateup_supported(int rows, int K, int N);
bool q_down_supported(int rows, int K, int N);
hipError_t q_launch_gateup(int rows, int E, const uint16_t *xp, const int32_t *counts,
                           const int32_t *offsets, const uint16_t *w1, const uint16_t *w3, int K,
                           int N, uint16_t *h, float *g, float *u, hipStream_t stream);
hipError_t q_launch_down(int rows, int E, const uint16_t *h, const int32_t *counts,
                         const int32_t *offsets, const uint16_t *w2, int K, int N, float *o,
                         int parts, size_t part_stride, int cu_per_xcd, int *parts_out,
                         hipStream_t stream);
// The backward's products on the same pipeline.  bt_dswiglu: z = dyp
// w2[e]^T (dyp the routed rows' dy, unscaled; w2[e] [N, K1] read along
// K1), da = w_row z turned into dg, du (bf16) with g, u (fp32), all
// [rows, N]; and dw_part [rows, N / 256] = each row's sum of h z over each
// 256-column tile (h bf16 [rows, N]), the routing-weight gradient's parts.
// bt_store_split: C = A B[e]^T + A2 B2[e]^T (B[e], B2[e] [N, K1]), the
// 2 K1 reduction cut into parts chosen from the counts (count to
// *parts_out, part p at C + p * part_stride).  hipErrorNotSupported
// unless K1 % 64 == 0, N % 256 == 0 and the operands fit 32-bit offsets
// (q_bt_dswiglu_supported).
bool q_bt_dswiglu_supported(int rows, int K1, int N);
hipError_t q_launch_bt_dswiglu(int rows, int E, const uint16_t *dyp, const uint16_t *w2, int K1,
                               int N, const int32_t *counts, const int32_t *offsets,
                               const float *g, const float *u, uint16_t *dg, uint16_t *du,
                               const float *w_row, const uint16_t *h, float *dw_part,
                               hipStream_t stream);
hipError_t q_launch_bt_store_split(int rows, int E, const uint16_t *A, const uint16_t *B,
                                   const uint16_t *A2, const uint16_t *B2, int K1, int N,
                                   const int32_t *counts, const int32_t *offsets, float *C,
                                   size_t part_stride, int *parts_out, hipStream_t stream);
// Weight gradients from K-contiguous copies whose columns hold each
// expert's rows padded to a multiple of 64 with zeros (row length
// q_dw_ldk).  transpose_pad: dst [C, ldk] from src [rows, C] (grouped
// rows).  dw (nmat = 2): C[e] = At_e^T B0t_e, C2[e] = At_e^T B1t_e; (nmat =
// 1): C[e] = At_e^T B0t_e; At [M, ldk], B [N, ldk], C [E, M, N] fp32.
int q_dw_ldk(int rows, int E);
bool q_dw_supported(int rows, int E, int d, int f);
hipError_t q_launch_transpose_pad(const uint16_t *src, int rows, int C, const int32_t *counts,
                                  const int32_t *offsets, int E, uint16_t *dst, int ldk,
                                  hipStream_t stream);
hipError_t q_launch_dw(int nmat, const uint16_t *At, const uint16_t *B0t, const uint16_t *B1t,
                       float *C, float *C2, const int32_t *counts, int E, int M, int N, int ldk,
                       hipStream_t stream);
// gpart: as for launch_gateup_bf16 (decode sizes; the down product's last
// round cut the same way).
hipError_t launch_down_bf16(const moe_shape_t &s, const uint16_t *h, const int32_t *counts,
                            const int32_t *offsets, const uint16_t *w2, float *o,
                            hipStream_t stream, float *gpart = nullptr);

// ---------------------------------------------------------------------------
// Device helpers.

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16 with round-to-nearest-even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float v) {
    uint32_t u = __float_as_uint(v);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + expf(-g)); }

// Row-group lookup for grouped GEMMs.  Expert e owns ceil(counts[e]/bm)
// row tiles, laid out expert after expert.  Maps the flat tile number `mt`
// to (expert, first row, end row); returns false past the last tile.
__device__ __forceinline__ bool find_row_tile(const int32_t *counts, const int32_t *offsets,
                                              int E, int bm, int mt, int &e_out,
                                              int &row0, int &row_end) {
    int acc = 0;
    for (int e = 0; e < E; ++e) {
        int c = counts[e];
        int nt = (c + bm - 1) / bm;
        if (mt < acc + nt) {
            e_out = e;
            row0 = offsets[e] + (mt - acc) * bm;
            row_end = offsets[e] + c;
            return true;
        }
        acc += nt;
    }
    return false;
}

}  // namespace moe
