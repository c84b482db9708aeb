// Backward of the layer: gradients of L = sum(dy * y) with respect to x,
// the router and the three expert matrices.  The pages train router and
// experts jointly ("Mixtral 8x7B -- The Evolving Transformer", section 05,
// and the remark that they are trained together) and specify no loss,
// capacity or auxiliary term, so this is the gradient of the forward as
// written, with the top-k picks held fixed (a discrete choice):
//
//   dw_s = dy . o_s,   dl_e = w_s (dw_s - sum_r w_r dw_r) at the picked e
//   do_s = w_s dy,     da = do_s W2[e]^T
//   dg = da * u * silu'(g),   du = da * silu(g)
//   dx = sum_s (dg W1[e]^T + du W3[e]^T) + dl Wg^T
//   dW1[e] = X_e^T dG_e,  dW3[e] = X_e^T dU_e,  dW2[e] = H_e^T dO_e,
//   dWg = x^T dl
//
// The call recomputes what it needs of the forward (routing, grouped rows,
// g, u, h = silu(g) u and the expert outputs o) rather than keeping state
// between calls.  All products run on the matrix cores through one grouped
// GEMM template (bf16: 32x32x16 MFMA, fp32: 32x32x2 MFMA) that takes each
// operand either K-contiguous (read as is) or M/N-contiguous (transposed in
// registers on its way into LDS), grouped either by rows (every expert's
// rows times its own matrix) or by K (every expert's matrix reduced over
// its rows), with fused epilogues for the SwiGLU forward and derivative.
// Every sum has a fixed order; there are no atomics.
#include <algorithm>

#include "moe_internal.h"

namespace moe {
namespace {

__device__ __forceinline__ float to_f32(uint16_t v) { return bf16_to_f32(v); }
__device__ __forceinline__ float to_f32(float v) { return v; }
template <typename T>
__device__ __forceinline__ T from_f32(float v);
template <>
__device__ __forceinline__ uint16_t from_f32<uint16_t>(float v) {
    return (uint16_t)f32_to_bf16(v);
}
template <>
__device__ __forceinline__ float from_f32<float>(float v) { return v; }

__device__ __forceinline__ float sigmoid_f32(float g) { return 1.0f / (1.0f + expf(-g)); }

constexpr int GBM = 128, GBN = 128, GBK = 32;   // tile and K step
enum { OP_KC = 0, OP_MNC = 1 };                 // operand K-contiguous or M/N-contiguous
enum { GROUP_ROWS = 0, GROUP_K = 1 };
enum { EPI_STORE = 0, EPI_ADD = 1, EPI_UP = 2, EPI_DSWIGLU = 3 };

// Operands of one grouped GEMM, strides in elements.
//   A element (m, k): KC  -> A + m * lda + k;   MNC -> A + k * lda + m
//   B element (k, n): KC  -> B_e + n * ldb + k; MNC -> B_e + k * ldb + n
//   with B_e = B + e * b_estride.
//   GROUP_ROWS: m runs over the routed rows (global), grouped by expert;
//     the tile's expert selects B.  C + m * ldc + n.
//   GROUP_K: m, n run over the whole M x N output of expert e, and k over
//     the expert's rows [offsets[e], offsets[e] + counts[e]).
//     C + e * c_estride + m * ldc + n.
// Epilogues (C fp32 unless stated):
//   EPI_STORE   C = acc
//   EPI_ADD     C += acc
//   EPI_UP      C = u = acc; C2 (layer dtype) = silu(G) * u       (G at C's index)
//   EPI_DSWIGLU with da = acc, g = G, u = U at C's index:
//               C (layer dtype) = da * u * silu'(g), C2 (layer dtype) = da * silu(g)
struct GemmArgs {
    const void *A;
    long long lda;
    const void *B;
    long long ldb, b_estride;
    void *C;
    long long ldc, c_estride;
    void *C2;
    const float *G, *U;
    const int32_t *counts, *offsets;
    int E, M, N, K;
};

// r[i] holds row i of an 8 x 8 bf16 block (8 values along M/N, two per
// dword, the lower index in the low half); out[c] receives column c: 8
// values along K, row 0 in the low half of dword 0.
__device__ __forceinline__ void transpose_b16(const uint4 (&r)[8], uint4 (&out)[8]) {
    const uint32_t *w = reinterpret_cast<const uint32_t *>(r);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const int p = c >> 1;
        uint32_t q[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t lo = w[4 * (2 * j) + p], hi = w[4 * (2 * j + 1) + p];
            q[j] = (c & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
        }
        out[c] = make_uint4(q[0], q[1], q[2], q[3]);
    }
}

// The same for a 4 x 4 block of fp32.
__device__ __forceinline__ void transpose_b32(const uint4 (&r)[4], uint4 (&out)[4]) {
    out[0] = make_uint4(r[0].x, r[1].x, r[2].x, r[3].x);
    out[1] = make_uint4(r[0].y, r[1].y, r[2].y, r[3].y);
    out[2] = make_uint4(r[0].z, r[1].z, r[2].z, r[3].z);
    out[3] = make_uint4(r[0].w, r[1].w, r[2].w, r[3].w);
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));

// 128 x 32 tile of one operand, staged through registers into LDS.
//   KC, and MNC of fp32: 128 lines of 32 K values (pitch PITCH); an MNC
//     tile is transposed in registers (V x V blocks) on the way.
//   MNC of bf16 (TR): the tile's own layout, 32 K rows of 128 values
//     (pitch TPITCH), copied with plain 16-byte vectors by every thread;
//     MFMA fragments are read back with the LDS transpose read.
template <typename T, int LAYOUT>
struct TileLoad {
    static constexpr int V = 16 / (int)sizeof(T);          // elements per 16 bytes
    static constexpr bool TR = LAYOUT == OP_MNC && V == 8;
    static constexpr int PITCH = GBK + V;                   // LDS line pitch (KC / transposed)
    static constexpr int TPITCH = 128 + 16;                 // LDS K-row pitch (TR): the 4 rows a
                                                            // transpose read covers start 8 banks apart
    // KC: 128 lines x (32 / V) vectors; MNC: (32 / V) x (128 / V) blocks of V x V.
    static constexpr int NKC = 128 * GBK / V / 256;         // vectors per thread (KC, TR)
    static constexpr int NBLK = (GBK / V) * (128 / V);      // blocks (MNC)
    uint4 r[(LAYOUT == OP_KC || TR) ? NKC : V];

    // base points at element (line 0 of the tile, k = 0) for KC (lines are
    // ld apart; line index clamped to line_lim - 1), or at element (k = 0,
    // mn = 0) of the whole operand for MNC (k rows are ld apart; k valid in
    // [k_lo, k_hi), mn valid below mn_lim).
    __device__ __forceinline__ void load(const T *base, long long ld, int line0, int line_lim,
                                         int k0, int k_hi, int k_lo, int mn0, int mn_lim) {
        const int tid = threadIdx.x;
        if constexpr (LAYOUT == OP_KC) {
#pragma unroll
            for (int i = 0; i < NKC; ++i) {
                const int v = tid + 256 * i;
                const int line = v / (GBK / V), kv = v % (GBK / V);
                const int k = k0 + kv * V;
                const T *p = base + (long long)min(line0 + line, line_lim - 1) * ld + k;
                r[i] = k < k_hi ? *reinterpret_cast<const uint4 *>(p) : make_uint4(0, 0, 0, 0);
            }
        } else if constexpr (TR) {
#pragma unroll
            for (int i = 0; i < NKC; ++i) {
                const int v = tid + 256 * i;
                const int kr = v / (128 / V), c = (v % (128 / V)) * V;
                const int k = k0 + kr, mn = mn0 + c;
                const bool ok = k >= k_lo && k < k_hi && mn < mn_lim;
                r[i] = ok ? *reinterpret_cast<const uint4 *>(base + (long long)k * ld + mn)
                          : make_uint4(0, 0, 0, 0);
            }
        } else {
            if (tid < NBLK) {
                const int kb = tid % (GBK / V), mb = tid / (GBK / V);
                const int mn = mn0 + mb * V;
#pragma unroll
                for (int i = 0; i < V; ++i) {
                    const int k = k0 + kb * V + i;
                    const bool ok = k >= k_lo && k < k_hi && mn < mn_lim;
                    r[i] = ok ? *reinterpret_cast<const uint4 *>(base + (long long)k * ld + mn)
                              : make_uint4(0, 0, 0, 0);
                }
            }
        }
    }
    // The 32x32x16 bf16 operand of tile lines mb .. mb+31 at K offset kk:
    // lane l holds line mb + l % 32, K values kk + 8 (l / 32) .. + 7.
    __device__ __forceinline__ bf16x8_t frag(const T *s, int mb, int kk) const {
        const int lane = threadIdx.x & 63;
        if constexpr (TR) {
            // Transpose read: within each 16-lane group G, lane 4 jq + q
            // addresses K row r + jq, columns c .. c + 3, and lane j
            // receives the 4 K values of column c0 + j.
            const int G = lane >> 4, jq = (lane & 15) >> 2, q = lane & 3;
            const int c = mb + 16 * (G & 1) + 4 * q;
            const int r = kk + 8 * (G >> 1) + jq;
            typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
            const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4 *)(s + r * TPITCH + c));
            const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4 *)(s + (r + 4) * TPITCH + c));
            return __builtin_bit_cast(bf16x8_t,
                                      __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        } else {
            return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(
                s + (mb + (lane & 31)) * PITCH + kk + (lane >> 5) * 8));
        }
    }
    __device__ __forceinline__ void store(T *s) {
        const int tid = threadIdx.x;
        if constexpr (LAYOUT == OP_KC) {
#pragma unroll
            for (int i = 0; i < NKC; ++i) {
                const int v = tid + 256 * i;
                const int line = v / (GBK / V), kv = v % (GBK / V);
                *reinterpret_cast<uint4 *>(s + line * PITCH + kv * V) = r[i];
            }
        } else if constexpr (TR) {
#pragma unroll
            for (int i = 0; i < NKC; ++i) {
                const int v = tid + 256 * i;
                const int kr = v / (128 / V), c = (v % (128 / V)) * V;
                *reinterpret_cast<uint4 *>(s + kr * TPITCH + c) = r[i];
            }
        } else {
            if (tid < NBLK) {
                const int kb = tid % (GBK / V), mb = tid / (GBK / V);
                uint4 t[V];
                if constexpr (V == 8) transpose_b16(r, t);
                else transpose_b32(r, t);
#pragma unroll
                for (int c = 0; c < V; ++c)
                    *reinterpret_cast<uint4 *>(s + (mb * V + c) * PITCH + kb * V) = t[c];
            }
        }
    }
};

// One 128 x 128 output tile per workgroup, 4 wavefronts (2 x 2) of 64 x 64,
// K step 32, LDS double-buffered through registers.
template <typename T, int AL, int BL, int GROUP, int EPI>
__global__ __launch_bounds__(256) void bwd_gemm_kernel(GemmArgs p) {
    using LA = TileLoad<T, AL>;
    using LB = TileLoad<T, BL>;
    constexpr int PITCH = LA::PITCH;
    __shared__ __attribute__((aligned(16))) T sA[2][GBM * PITCH];
    __shared__ __attribute__((aligned(16))) T sB[2][GBN * PITCH];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    int e, m0, m_end, n0, k_lo, k_hi;
    if constexpr (GROUP == GROUP_ROWS) {
        const int n_tiles = (p.N + GBN - 1) / GBN;
        const int mt = blockIdx.x / n_tiles, nt = blockIdx.x % n_tiles;
        if (!find_row_tile(p.counts, p.offsets, p.E, GBM, mt, e, m0, m_end)) return;
        n0 = nt * GBN;
        k_lo = 0;
        k_hi = p.K;
    } else {
        const int m_tiles = (p.M + GBM - 1) / GBM, n_tiles = (p.N + GBN - 1) / GBN;
        e = blockIdx.x / (m_tiles * n_tiles);
        const int rem = blockIdx.x % (m_tiles * n_tiles);
        m0 = (rem / n_tiles) * GBM;
        n0 = (rem % n_tiles) * GBN;
        m_end = p.M;
        k_lo = p.offsets[e];
        k_hi = k_lo + p.counts[e];
    }
    const T *A = static_cast<const T *>(p.A);
    const T *B = static_cast<const T *>(p.B) + (GROUP == GROUP_ROWS ? (long long)e * p.b_estride : 0);

    LA la;
    LB lb;
    auto gload = [&](int k0) {
        if constexpr (AL == OP_KC)
            la.load(A, p.lda, m0, GROUP == GROUP_ROWS ? p.M : m_end, k0, k_hi, k_lo, 0, 0);
        else
            la.load(A, p.lda, 0, 0, k0, k_hi, k_lo, m0, GROUP == GROUP_ROWS ? p.M : m_end);
        if constexpr (BL == OP_KC)
            lb.load(B, p.ldb, n0, p.N, k0, k_hi, k_lo, 0, 0);
        else
            lb.load(B, p.ldb, 0, 0, k0, k_hi, k_lo, n0, p.N);
    };

    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

    const int nk = (k_hi - k_lo + GBK - 1) / GBK;
    if (nk > 0) {
        gload(k_lo);
        la.store(sA[0]);
        lb.store(sB[0]);
        __syncthreads();
    }
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) gload(k_lo + (kt + 1) * GBK);
        const T *As = sA[cur], *Bs = sB[cur];
        if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int kk = 0; kk < GBK; kk += 16) {
                bf16x8_t af[2], bfr[2];
#pragma unroll
                for (int i = 0; i < 2; ++i) af[i] = la.frag(As, wm * 64 + i * 32, kk);
#pragma unroll
                for (int j = 0; j < 2; ++j) bfr[j] = lb.frag(Bs, wn * 64 + j * 32, kk);
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j],
                                                                             acc[i][j], 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int kk = 0; kk < GBK; kk += 2) {
                const int koff = kk + (lane >> 5);
                float af[2], bfr[2];
#pragma unroll
                for (int i = 0; i < 2; ++i) af[i] = As[(wm * 64 + i * 32 + (lane & 31)) * PITCH + koff];
#pragma unroll
                for (int j = 0; j < 2; ++j) bfr[j] = Bs[(wn * 64 + j * 32 + (lane & 31)) * PITCH + koff];
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[i], bfr[j], acc[i][j],
                                                                         0, 0, 0);
            }
        }
        if (kt + 1 < nk) {
            la.store(sA[cur ^ 1]);
            lb.store(sB[cur ^ 1]);
        }
        __syncthreads();
    }

    // Epilogue.  32x32 accumulator layout: value q of lane l is row
    // 8*(q/4) + 4*(l/32) + q%4, column l%32 of the block.
    const long long cbase = GROUP == GROUP_K ? (long long)e * p.c_estride : 0;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = n0 + wn * 64 + j * 32 + (lane & 31);
            if (col >= p.N) continue;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int row = m0 + wm * 64 + i * 32 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
                if (row >= m_end) continue;
                const long long ci = cbase + (long long)row * p.ldc + col;
                const float v = acc[i][j][q];
                if constexpr (EPI == EPI_STORE) {
                    static_cast<float *>(p.C)[ci] = v;
                } else if constexpr (EPI == EPI_ADD) {
                    static_cast<float *>(p.C)[ci] += v;
                } else if constexpr (EPI == EPI_UP) {
                    const float g = p.G[ci];
                    static_cast<float *>(p.C)[ci] = v;
                    static_cast<T *>(p.C2)[ci] = from_f32<T>(g * sigmoid_f32(g) * v);
                } else {
                    const float g = p.G[ci], u = p.U[ci], sg = sigmoid_f32(g);
                    static_cast<T *>(p.C)[ci] = from_f32<T>(v * u * sg * (1.0f + g * (1.0f - sg)));
                    static_cast<T *>(p.C2)[ci] = from_f32<T>(v * g * sg);
                }
            }
        }
}

// The routed rows' dy for the dSwiGLU product (bf16): one wavefront per
// token t copies dy[t] to dyp[pos[t, s]] for every slot s and stores the
// slot's routing weight in w_row[pos[t, s]].
__global__ __launch_bounds__(256) void bwd_gather_dy_kernel(const uint4 *__restrict__ dy,
                                                            const int32_t *__restrict__ pos,
                                                            const float *__restrict__ w, int n_tok,
                                                            int k, int row_vecs,
                                                            uint4 *__restrict__ dyp,
                                                            float *__restrict__ w_row) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= n_tok) return;
    for (int s = 0; s < k; ++s) {
        const int r = pos[k * t + s];
        if (lane == 0) w_row[r] = w[k * t + s];
        for (int j = lane; j < row_vecs; j += 64)
            dyp[(size_t)r * row_vecs + j] = dy[(size_t)t * row_vecs + j];
    }
}

// One workgroup per token t: for each slot s with row r = pos[t, s],
//   dw_s = sum_i dy[t, i] o[r, i]     (fixed-order block reduction)
//   dO[r, i] = w[t, s] dy[t, i]       (layer dtype)
// then dl[t, :] = 0 except dl[t, idx_s] = w_s (dw_s - sum_r w_r dw_r).
// With dw_part (o not computed): dw_s = sum over the nct column tiles c of
// dw_part[r, c], the parts of h . (dy W2^T) = dy . o that the dSwiGLU
// product leaves, added in tile order by the first wavefront's lanes
// (lane l the tiles l, l + 64, ...) and then across its lanes (xor 32 ..
// 1): a fixed order.
template <typename T>
__global__ __launch_bounds__(256) void bwd_route_grad_kernel(
    const T *__restrict__ dy, const float *__restrict__ o, const int32_t *__restrict__ idx,
    const float *__restrict__ w, const int32_t *__restrict__ pos, int d, int E, int k,
    T *__restrict__ dO, float *__restrict__ dl, const int *__restrict__ o_parts,
    size_t part_stride, const float *__restrict__ dw_part, int nct) {
    __shared__ float part[4][kMaxTopK];
    const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bool two = o_parts && *o_parts == 2;   // o = part 0 + part 1
    float dws[kMaxTopK];
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s) {
        if (s >= k) break;
        const int r = pos[k * t + s];
        const float ws = w[k * t + s];
        float acc = 0.0f;
        if (dw_part) {
            if (wave == 0)
                for (int c = lane; c < nct; c += 64) acc += dw_part[(size_t)r * nct + c];
            for (int i = tid; i < d; i += 256)
                dO[(size_t)r * d + i] = from_f32<T>(ws * to_f32(dy[(size_t)t * d + i]));
        } else {
            for (int i = tid; i < d; i += 256) {
                const float g = to_f32(dy[(size_t)t * d + i]);
                float ov = o[(size_t)r * d + i];
                if (two) ov += o[part_stride + (size_t)r * d + i];
                acc += g * ov;
                dO[(size_t)r * d + i] = from_f32<T>(ws * g);
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
        if (lane == 0) part[wave][s] = acc;
    }
    __syncthreads();
    if (tid != 0) return;
    float mean = 0.0f;
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s) {
        if (s >= k) break;
        dws[s] = (part[0][s] + part[1][s]) + (part[2][s] + part[3][s]);
        mean += w[k * t + s] * dws[s];
    }
    for (int e = 0; e < E; ++e) dl[(size_t)t * E + e] = 0.0f;
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s) {
        if (s >= k) break;
        dl[(size_t)t * E + idx[k * t + s]] = w[k * t + s] * (dws[s] - mean);
    }
}

// dx[t, i] = sum_s dXp[pos[t, s], i] (slot order) + sum_e dl[t, e] Wg[i, e],
// rounded once to the layer dtype.  One workgroup per token.
template <typename T>
__global__ __launch_bounds__(256) void bwd_dx_kernel(const float *__restrict__ dxp,
                                                     const int32_t *__restrict__ pos,
                                                     const float *__restrict__ dl,
                                                     const T *__restrict__ wg, int d, int E,
                                                     int k, T *__restrict__ dx,
                                                     const int *__restrict__ dxp_parts,
                                                     size_t part_stride) {
    __shared__ float dlt[kMaxExperts];
    const int t = blockIdx.x, tid = threadIdx.x;
    const bool two = dxp_parts && *dxp_parts == 2;   // dXp = part 0 + part 1
    if (tid < E) dlt[tid] = dl[(size_t)t * E + tid];
    __syncthreads();
    int rows[kMaxTopK];
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s) rows[s] = s < k ? pos[k * t + s] : 0;
    auto row_value = [&](int r, int i) {
        float v = dxp[(size_t)r * d + i];
        if (two) v += dxp[part_stride + (size_t)r * d + i];
        return v;
    };
    for (int i = tid; i < d; i += 256) {
        float v = row_value(rows[0], i);
#pragma unroll
        for (int s = 1; s < kMaxTopK; ++s)
            if (s < k) v += row_value(rows[s], i);
        float r = 0.0f;
        for (int e = 0; e < E; ++e) r += dlt[e] * to_f32(wg[(size_t)i * E + e]);
        dx[(size_t)t * d + i] = from_f32<T>(v + r);
    }
}

// dWg[i, e] = sum_t x[t, i] dl[t, e], in two passes.  Pass 1: workgroup
// (b, c) takes 2 * DWG_THREADS columns i (two adjacent ones per thread, so a
// wavefront reads 128 consecutive elements of a token row in one load) and
// chunk c of the tokens; each thread sums its chunk in token order into
// part[c][i][e].  The chunk's dl rows are staged in LDS a block at a time,
// padded with zeros to EMAX columns, and every lane reads the same LDS word
// (a broadcast).  Pass 2 adds the chunks in the order c = 0, 1, ..., so the
// result does not depend on scheduling.
constexpr int DWG_THREADS = 256;
constexpr int DWG_COLS = 2 * DWG_THREADS;  // columns per workgroup
constexpr int DWG_SB = 64;                 // tokens per staged block of dl
constexpr int DWG_PARTS = 512;             // chunks x EMAX at most (partial buffer size)

inline int dwg_emax(int E) { return E <= 8 ? 8 : E <= 16 ? 16 : E <= 32 ? 32 : 64; }
// Token chunks: about 32 tokens each, at most DWG_PARTS / EMAX of them.
inline int dwg_chunks(int T_, int E) {
    return std::max(1, std::min((T_ + 31) / 32, DWG_PARTS / dwg_emax(E)));
}

// Two adjacent elements (the first at an even index of a row of even length).
__device__ __forceinline__ void load_pair(const uint16_t *p, float &a, float &b) {
    const uint32_t v = *reinterpret_cast<const uint32_t *>(p);
    a = __uint_as_float(v << 16);
    b = __uint_as_float(v & 0xffff0000u);
}
__device__ __forceinline__ void load_pair(const float *p, float &a, float &b) {
    const float2 v = *reinterpret_cast<const float2 *>(p);
    a = v.x;
    b = v.y;
}

// At most 4 wavefronts per SIMD: the scheduler then keeps the eight loads of
// a step in flight instead of trading them for occupancy.
template <typename T, int EMAX>
__global__ __launch_bounds__(DWG_THREADS) __attribute__((amdgpu_waves_per_eu(1, 4)))
void bwd_dwg_part_kernel(
    const T *__restrict__ x, const float *__restrict__ dl, int T_, int d, int E, int chunks,
    float *__restrict__ part) {
    __shared__ float dls[DWG_SB][EMAX];
    const int i = 2 * (blockIdx.x * DWG_THREADS + threadIdx.x);
    const int xi = min(i, d - 2);       // columns past d load a valid pair, never stored
    const int c = blockIdx.y;
    const int t_beg = (int)((int64_t)T_ * c / chunks), t_end = (int)((int64_t)T_ * (c + 1) / chunks);
    float acc[2][EMAX];
#pragma unroll
    for (int e = 0; e < EMAX; ++e) acc[0][e] = acc[1][e] = 0.0f;
    for (int t0 = t_beg; t0 < t_end; t0 += DWG_SB) {
        const int n = min(DWG_SB, t_end - t0);
        __syncthreads();
        for (int j = threadIdx.x; j < DWG_SB * EMAX; j += DWG_THREADS) {
            const int tt = j / EMAX, e = j % EMAX;
            dls[tt][e] = (tt < n && e < E) ? dl[(size_t)(t0 + tt) * E + e] : 0.0f;
        }
        __syncthreads();
        const T *xr = x + (size_t)t0 * d + xi;
        int tt = 0;
        for (; tt + 8 <= n; tt += 8) {     // eight token rows in flight
            float xa[8], xb[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) load_pair(xr + (size_t)(tt + u) * d, xa[u], xb[u]);
            // issue the eight loads before any use (the scheduler would
            // otherwise wait on each one in turn)
            __builtin_amdgcn_sched_group_barrier(0x020, 8, 0);
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
                for (int e = 0; e < EMAX; ++e) {
                    const float v = dls[tt + u][e];
                    acc[0][e] += xa[u] * v;
                    acc[1][e] += xb[u] * v;
                }
        }
        for (; tt < n; ++tt) {
            float xa, xb;
            load_pair(xr + (size_t)tt * d, xa, xb);
#pragma unroll
            for (int e = 0; e < EMAX; ++e) {
                const float v = dls[tt][e];
                acc[0][e] += xa * v;
                acc[1][e] += xb * v;
            }
        }
    }
    if (i >= d) return;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        float *out = part + ((size_t)c * d + i + h) * E;
#pragma unroll
        for (int e = 0; e < EMAX; ++e)
            if (e < E) out[e] = acc[h][e];
    }
}

__global__ __launch_bounds__(256) void bwd_dwg_sum_kernel(const float *__restrict__ part,
                                                          int chunks, size_t n,
                                                          float *__restrict__ dwg) {
    const size_t j = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (j >= n) return;
    float s = 0.0f;
    for (int c = 0; c < chunks; ++c) s += part[(size_t)c * n + j];
    dwg[j] = s;
}

template <typename T>
hipError_t launch_dwg(const T *x, const float *dl, int T_, int d, int E, float *part,
                      float *dwg, hipStream_t stream) {
    const int chunks = dwg_chunks(T_, E);
    const dim3 grid((d + DWG_COLS - 1) / DWG_COLS, chunks), block(DWG_THREADS);
    switch (dwg_emax(E)) {
    case 8:
        hipLaunchKernelGGL((bwd_dwg_part_kernel<T, 8>), grid, block, 0, stream, x, dl, T_, d, E,
                           chunks, part);
        break;
    case 16:
        hipLaunchKernelGGL((bwd_dwg_part_kernel<T, 16>), grid, block, 0, stream, x, dl, T_, d, E,
                           chunks, part);
        break;
    case 32:
        hipLaunchKernelGGL((bwd_dwg_part_kernel<T, 32>), grid, block, 0, stream, x, dl, T_, d, E,
                           chunks, part);
        break;
    default:
        hipLaunchKernelGGL((bwd_dwg_part_kernel<T, 64>), grid, block, 0, stream, x, dl, T_, d, E,
                           chunks, part);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t n = (size_t)d * E;
    hipLaunchKernelGGL(bwd_dwg_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                       part, chunks, n, dwg);
    return hipGetLastError();
}

template <typename T, int AL, int BL, int GROUP, int EPI>
hipError_t gemm(const GemmArgs &a, int tiles, hipStream_t stream) {
    if (tiles <= 0) return hipSuccess;
    hipLaunchKernelGGL((bwd_gemm_kernel<T, AL, BL, GROUP, EPI>), dim3(tiles), dim3(256), 0,
                       stream, a);
    return hipGetLastError();
}

inline int row_tiles_bound(int rows, int E) { return (rows + GBM - 1) / GBM + E; }
inline int tiles_of(int n) { return (n + GBN - 1) / GBN; }

template <typename T>
hipError_t run_backward_t(const moe_shape_t &s, const T *x, const T *wg, const T *w1,
                          const T *w3, const T *w2, const T *dy, T *dx, float *dwg, float *dw1,
                          float *dw3, float *dw2, const BackwardLayout &L, char *base,
                          hipStream_t str) {
    const int Tn = s.T, d = s.d_model, f = s.d_ff, E = s.n_experts, k = s.top_k;
    const int R = routed_rows(s);
    int32_t *idx = reinterpret_cast<int32_t *>(base + L.idx);
    float *w = reinterpret_cast<float *>(base + L.w);
    int32_t *counts = reinterpret_cast<int32_t *>(base + L.counts);
    int32_t *offsets = reinterpret_cast<int32_t *>(base + L.offsets);
    int32_t *pos = reinterpret_cast<int32_t *>(base + L.pos);
    T *xp = reinterpret_cast<T *>(base + L.xp);
    float *G = reinterpret_cast<float *>(base + L.g);
    float *U = reinterpret_cast<float *>(base + L.u);
    T *H = reinterpret_cast<T *>(base + L.h);
    float *O = reinterpret_cast<float *>(base + L.o);      // later dXp
    T *dO = reinterpret_cast<T *>(base + L.dout);
    T *dG = reinterpret_cast<T *>(base + L.dg);
    T *dU = reinterpret_cast<T *>(base + L.du);
    float *dl = reinterpret_cast<float *>(base + L.dl);
    float *dwgp = reinterpret_cast<float *>(base + L.dwgp);
    int *nparts = reinterpret_cast<int *>(base + L.nparts);   // o, dXp
    const size_t pstride = (size_t)R * d;                       // floats between parts

    hipError_t e = launch_route(s, x, wg, idx, w, str);
    if (e == hipSuccess) e = launch_dispatch(s, x, idx, counts, offsets, pos, xp, str);
    const int rt = row_tiles_bound(R, E);
    GemmArgs a{};
    a.counts = counts;
    a.offsets = offsets;
    a.E = E;
    // g = xp W1[e] and u = xp W3[e] (fp32), h = silu(g) u.  bf16 layers of
    // prefill size take the forward's direct-to-LDS gate/up kernel in its
    // variant that also stores g and u; other shapes the generic GEMM.
    bool fused = false;
    if constexpr (sizeof(T) == 2) {
        if (e == hipSuccess) {
            const hipError_t fe = launch_gateup_bf16_gu(s, xp, counts, offsets, w1, w3, H, G, U,
                                                        str);
            fused = fe == hipSuccess;
            if (fe != hipErrorNotSupported && fe != hipSuccess) e = fe;
        }
    }
    if (!fused) {
        a.A = xp; a.lda = d; a.b_estride = (long long)d * f; a.ldb = f; a.ldc = f;
        a.M = R; a.N = f; a.K = d;
        a.B = w1; a.C = G;
        if (e == hipSuccess)
            e = gemm<T, OP_KC, OP_MNC, GROUP_ROWS, EPI_STORE>(a, rt * tiles_of(f), str);
        a.B = w3; a.C = U; a.C2 = H; a.G = G;
        if (e == hipSuccess)
            e = gemm<T, OP_KC, OP_MNC, GROUP_ROWS, EPI_UP>(a, rt * tiles_of(f), str);
    }
    // bf16 layers whose sizes fit the pipelined tile body need no o: the
    // dSwiGLU product takes the routed rows' dy unscaled, z = dy W2[e]^T,
    // and the routing-weight gradient dy . o = h . z comes from its epilogue
    // in per-column-tile parts (w_row and the parts live in the o region,
    // which dXp takes over later).
    bool zpath = false;
    if constexpr (sizeof(T) == 2)
        zpath = q_bt_dswiglu_supported(R, d, f) && (size_t)(1 + f / 256) <= (size_t)kMaxDownSplit * d;
    const int nct = f / 256;
    float *w_row = O;
    float *dw_part = O + ((R + 63) / 64) * 64;
    bool da_done = false, dxp_done = false;
    if constexpr (sizeof(T) == 2) {
        if (zpath && e == hipSuccess && Tn > 0) {
            hipLaunchKernelGGL(bwd_gather_dy_kernel, dim3((Tn + 3) / 4), dim3(256), 0, str,
                               reinterpret_cast<const uint4 *>(dy), pos, w, Tn, k, d / 8,
                               reinterpret_cast<uint4 *>(dO), w_row);
            e = hipGetLastError();
            if (e == hipSuccess)
                e = q_launch_bt_dswiglu(R, E, dO, w2, d, f, counts, offsets, G, U, dG, dU, w_row,
                                        H, dw_part, str);
            if (e == hipSuccess) {
                hipLaunchKernelGGL(bwd_route_grad_kernel<T>, dim3(Tn), dim3(256), 0, str, dy, O,
                                   idx, w, pos, d, E, k, dO, dl, nullptr, (size_t)0, dw_part,
                                   nct);
                e = hipGetLastError();
            }
            da_done = true;
        }
    }
    // o = h W2[e]: the forward's down kernels for bf16 (at prefill sizes the
    // variant that cuts the reduction in parts; route_grad adds them), the
    // generic GEMM for fp32
    const int *o_parts = nullptr;
    if constexpr (sizeof(T) == 2) {
        if (e == hipSuccess && !zpath) {
            const hipError_t de = launch_down_split_bf16(R, E, H, counts, offsets, w2, f, d, 0,
                                                         pstride, O, nparts, str);
            if (de == hipSuccess) o_parts = nparts;
            else if (de == hipErrorNotSupported) e = launch_down_bf16(s, H, counts, offsets, w2, O, str);
            else e = de;
        }
    } else {
        a = GemmArgs{};
        a.counts = counts; a.offsets = offsets; a.E = E;
        a.A = H; a.lda = f; a.B = w2; a.ldb = d; a.b_estride = (long long)f * d;
        a.C = O; a.ldc = d; a.M = R; a.N = d; a.K = f;
        if (e == hipSuccess)
            e = gemm<T, OP_KC, OP_MNC, GROUP_ROWS, EPI_STORE>(a, rt * tiles_of(d), str);
    }
    // routing-weight gradients, dO and dl
    if (e == hipSuccess && Tn > 0 && !zpath) {
        hipLaunchKernelGGL(bwd_route_grad_kernel<T>, dim3(Tn), dim3(256), 0, str, dy, O, idx, w,
                           pos, d, E, k, dO, dl, o_parts, pstride, nullptr, 0);
        e = hipGetLastError();
    }
    // da = dO W2[e]^T, with dg, du in the epilogue.  The weight matrices are
    // read K-contiguous here (a row of W2[e] is a column of W2[e]^T); bf16
    // layers of other sizes take the direct-to-LDS variant for such
    // operands where it fits, other shapes the generic GEMM.
    if constexpr (sizeof(T) == 2) {
        if (e == hipSuccess && !da_done) {
            const hipError_t fe = launch_bt_dswiglu_bf16(R, E, dO, w2, d, f, counts, offsets,
                                                         G, U, dG, dU, str);
            da_done = fe == hipSuccess;
            if (fe != hipErrorNotSupported && fe != hipSuccess) e = fe;
        }
    }
    a = GemmArgs{};
    a.counts = counts; a.offsets = offsets; a.E = E;
    a.A = dO; a.lda = d; a.B = w2; a.ldb = d; a.b_estride = (long long)f * d;
    a.C = dG; a.C2 = dU; a.G = G; a.U = U; a.ldc = f; a.M = R; a.N = f; a.K = d;
    if (e == hipSuccess && !da_done)
        e = gemm<T, OP_KC, OP_KC, GROUP_ROWS, EPI_DSWIGLU>(a, rt * tiles_of(f), str);
    // dXp = dG W1[e]^T + dU W3[e]^T   (into the o region): one pass over a
    // reduction of 2 f on the pipeline above (cut in parts that the dx
    // kernel adds), else two generic GEMMs
    const int *dxp_parts = nullptr;
    if constexpr (sizeof(T) == 2) {
        if (e == hipSuccess) {
            const hipError_t fe = launch_bt_store_split_bf16(R, E, dG, w1, dU, w3, f, d, counts,
                                                             offsets, O, pstride, nparts + 1, str);
            dxp_done = fe == hipSuccess;
            if (dxp_done) dxp_parts = nparts + 1;
            if (fe != hipErrorNotSupported && fe != hipSuccess) e = fe;
        }
    }
    a = GemmArgs{};
    a.counts = counts; a.offsets = offsets; a.E = E;
    a.A = dG; a.lda = f; a.B = w1; a.ldb = f; a.b_estride = (long long)d * f;
    a.C = O; a.ldc = d; a.M = R; a.N = d; a.K = f;
    if (e == hipSuccess && !dxp_done)
        e = gemm<T, OP_KC, OP_KC, GROUP_ROWS, EPI_STORE>(a, rt * tiles_of(d), str);
    a.A = dU; a.B = w3;
    if (e == hipSuccess && !dxp_done)
        e = gemm<T, OP_KC, OP_KC, GROUP_ROWS, EPI_ADD>(a, rt * tiles_of(d), str);
    // dx
    if (e == hipSuccess && Tn > 0) {
        hipLaunchKernelGGL(bwd_dx_kernel<T>, dim3(Tn), dim3(256), 0, str, O, pos, dl, wg, d, E, k,
                           dx, dxp_parts, pstride);
        e = hipGetLastError();
    }
    // weight gradients: dW1[e] = xp_e^T dG_e, dW3[e] = xp_e^T dU_e, dW2[e] = h_e^T dO_e.
    // bf16 layers whose sizes fit: K-contiguous padded copies of the five
    // operands, then the pipelined GEMMs reduce over each expert's rows
    // (dW1 and dW3 in one pass sharing the xp tiles).
    if constexpr (sizeof(T) == 2) {
        if (L.ldk > 0 && R > 0) {
            const int ldk = L.ldk;
            uint16_t *xpT = reinterpret_cast<uint16_t *>(base + L.xpT);
            uint16_t *hT = reinterpret_cast<uint16_t *>(base + L.hT);
            uint16_t *dOT = reinterpret_cast<uint16_t *>(base + L.dOT);
            uint16_t *dGT = reinterpret_cast<uint16_t *>(base + L.dGT);
            uint16_t *dUT = reinterpret_cast<uint16_t *>(base + L.dUT);
            auto tp = [&](const T *src, int C, uint16_t *dst) {
                if (e == hipSuccess)
                    e = q_launch_transpose_pad(reinterpret_cast<const uint16_t *>(src), R, C,
                                               counts, offsets, E, dst, ldk, str);
            };
            tp(xp, d, xpT);
            tp(dG, f, dGT);
            tp(dU, f, dUT);
            tp(H, f, hT);
            tp(dO, d, dOT);
            if (e == hipSuccess)
                e = q_launch_dw(2, xpT, dGT, dUT, dw1, dw3, counts, E, d, f, ldk, str);
            if (e == hipSuccess)
                e = q_launch_dw(1, hT, dOT, nullptr, dw2, nullptr, counts, E, f, d, ldk, str);
            if (e == hipSuccess) e = launch_dwg<T>(x, dl, Tn, d, E, dwgp, dwg, str);
            return e;
        }
    }
    a = GemmArgs{};
    a.counts = counts; a.offsets = offsets; a.E = E;
    a.A = xp; a.lda = d; a.B = dG; a.ldb = f; a.C = dw1; a.ldc = f;
    a.c_estride = (long long)d * f; a.M = d; a.N = f;
    const int wt13 = E * tiles_of(d) * tiles_of(f);
    if (e == hipSuccess) e = gemm<T, OP_MNC, OP_MNC, GROUP_K, EPI_STORE>(a, wt13, str);
    a.B = dU; a.C = dw3;
    if (e == hipSuccess) e = gemm<T, OP_MNC, OP_MNC, GROUP_K, EPI_STORE>(a, wt13, str);
    a.A = H; a.lda = f; a.B = dO; a.ldb = d; a.C = dw2; a.ldc = d;
    a.c_estride = (long long)f * d; a.M = f; a.N = d;
    if (e == hipSuccess)
        e = gemm<T, OP_MNC, OP_MNC, GROUP_K, EPI_STORE>(a, E * tiles_of(f) * tiles_of(d), str);
    // router gradient
    if (e == hipSuccess) e = launch_dwg<T>(x, dl, Tn, d, E, dwgp, dwg, str);
    return e;
}

}  // namespace

BackwardLayout plan_backward(const moe_shape_t &s) {
    auto a256 = [](size_t v) { return (v + 255) & ~(size_t)255; };
    BackwardLayout L{};
    const size_t T = (size_t)s.T, d = (size_t)s.d_model, f = (size_t)s.d_ff;
    const size_t E = (size_t)s.n_experts, eb = elem_bytes(s.dtype);
    const size_t R = (size_t)s.top_k * T;
    size_t off = 0;
    L.idx = off;     off += a256(R * 4);
    L.w = off;       off += a256(R * 4);
    L.counts = off;  off += a256(E * 4);
    L.offsets = off; off += a256((E + 1) * 4);
    L.pos = off;     off += a256(R * 4);
    L.xp = off;      off += a256(R * d * eb);
    L.g = off;       off += a256(R * f * 4);
    L.u = off;       off += a256(R * f * 4);
    L.h = off;       off += a256(R * f * eb);
    L.o = off;       off += a256((size_t)kMaxDownSplit * R * d * 4);
    L.dout = off;    off += a256(R * d * eb);
    L.dg = off;      off += a256(R * f * eb);
    L.du = off;      off += a256(R * f * eb);
    L.dl = off;      off += a256(T * E * 4);
    L.dwgp = off;    off += a256((size_t)DWG_PARTS * d * 4);   // chunks x E <= DWG_PARTS
    L.nparts = off;  off += a256(2 * sizeof(int32_t));
    L.ldk = 0;
    L.xpT = L.hT = L.dOT = L.dGT = L.dUT = off;
    if (s.dtype == MOE_BF16 && q_dw_supported((int)R, (int)E, (int)d, (int)f)) {
        L.ldk = q_dw_ldk((int)R, (int)E);
        const size_t ldk = (size_t)L.ldk;
        L.xpT = off;     off += a256(d * ldk * 2);
        L.hT = off;      off += a256(f * ldk * 2);
        L.dOT = off;     off += a256(d * ldk * 2);
        L.dGT = off;     off += a256(f * ldk * 2);
        L.dUT = off;     off += a256(f * ldk * 2);
    }
    L.total = off;
    return L;
}

hipError_t launch_backward(const moe_shape_t &s, const void *x, const void *wg, const void *w1,
                           const void *w3, const void *w2, const void *dy, void *dx, float *dwg,
                           float *dw1, float *dw3, float *dw2, const BackwardLayout &L,
                           char *base, hipStream_t stream) {
    if (s.dtype == MOE_BF16)
        return run_backward_t<uint16_t>(
            s, static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(wg),
            static_cast<const uint16_t *>(w1), static_cast<const uint16_t *>(w3),
            static_cast<const uint16_t *>(w2), static_cast<const uint16_t *>(dy),
            static_cast<uint16_t *>(dx), dwg, dw1, dw3, dw2, L, base, stream);
    return run_backward_t<float>(
        s, static_cast<const float *>(x), static_cast<const float *>(wg),
        static_cast<const float *>(w1), static_cast<const float *>(w3),
        static_cast<const float *>(w2), static_cast<const float *>(dy), static_cast<float *>(dx),
        dwg, dw1, dw3, dw2, L, base, stream);
}

}  // namespace moe
