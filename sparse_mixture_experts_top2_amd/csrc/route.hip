// Router: logits = x w_gate (fp32), top-k (k <= 4; Mixtral uses 2) with
// lowest-index ties, softmax over the k kept logits.  "Mixtral 8x7B -- The Evolving Transformer",
// section 05 (MoERouter and the formula y = sum_k w_k E_{i_k}(x)).
// Page form (the MoERouter's own order of steps): softmax over all E
// logits, top-k of the probabilities, kept probabilities renormalised; the
// probabilities can be written out.
//
// The router matrix (d x E, 64 KiB at the 8x7B shape) is read once per
// workgroup from L2 and reused for its tokens; the kernel is bound by
// reading x once (T*d*elem bytes).
#include "moe_internal.h"

namespace moe {
namespace {

template <typename T>
__device__ __forceinline__ void load8(const T *p, float (&v)[8]);

template <>
__device__ __forceinline__ void load8<float>(const float *p, float (&v)[8]) {
    float4 a = *reinterpret_cast<const float4 *>(p);
    float4 b = *reinterpret_cast<const float4 *>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t *p, float (&v)[8]) {
    uint4 a = *reinterpret_cast<const uint4 *>(p);
    uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_to_f32(w[i] & 0xffffu);
        v[2 * i + 1] = bf16_to_f32(w[i] >> 16);
    }
}

// Eight fp32 values rounded to the element type and stored (16 or 32 B).
template <typename T>
__device__ __forceinline__ void store8(T *p, const float (&v)[8]);

template <>
__device__ __forceinline__ void store8<float>(float *p, const float (&v)[8]) {
    *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4 *>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

template <>
__device__ __forceinline__ void store8<uint16_t>(uint16_t *p, const float (&v)[8]) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = f32_to_bf16(v[2 * i]) | (f32_to_bf16(v[2 * i + 1]) << 16);
    *reinterpret_cast<uint4 *>(p) = make_uint4(w[0], w[1], w[2], w[3]);
}

// fp32 value rounded to the element type and widened back.
template <typename T>
__device__ __forceinline__ float round_to(float v);
template <>
__device__ __forceinline__ float round_to<float>(float v) { return v; }
template <>
__device__ __forceinline__ float round_to<uint16_t>(float v) {
    return bf16_to_f32(f32_to_bf16(v));
}

template <typename T>
__device__ __forceinline__ float load1(const T *p);
template <>
__device__ __forceinline__ float load1<float>(const float *p) { return *p; }
template <>
__device__ __forceinline__ float load1<uint16_t>(const uint16_t *p) { return bf16_to_f32(*p); }

// Router row j (E values) widened to fp32.  VEC (E a multiple of the values
// per 16 bytes): every row is 16-byte aligned (w_gate is 16-byte aligned),
// so it is read with vector loads; a 16-byte group past E re-reads the
// row's first group (in bounds) and its slots are set to 0.  Every load is
// unconditional, so a chunk's row loads are all in flight together rather
// than each waiting behind a branch.  Otherwise element by element, slots
// e >= E repeating column E-1 (their sums are never read).  The clamp
// bound sits in a vector register so that the compiler does not hoist EMAX
// uniform compares or offsets out of the loop into scalar registers.
template <typename T, int EMAX, bool VEC>
__device__ __forceinline__ void load_router_row(const T *row, int E, float (&wr)[EMAX]) {
    constexpr int per16 = 16 / (int)sizeof(T);
    if constexpr (VEC) {
#pragma unroll
        for (int v = 0; v < (EMAX + per16 - 1) / per16; ++v) {
            const bool in = v == 0 || v * per16 < E;
            const int g = in ? v : 0;
            float t[8];
            if constexpr (sizeof(T) == 2) {
                load8<T>(row + g * 8, t);
            } else {
                float4 q = reinterpret_cast<const float4 *>(row)[g];
                t[0] = q.x; t[1] = q.y; t[2] = q.z; t[3] = q.w;
            }
#pragma unroll
            for (int i = 0; i < per16 && v * per16 + i < EMAX; ++i)
                wr[v * per16 + i] = in ? t[i] : 0.0f;
        }
    } else {
        int last;
        asm volatile("v_mov_b32 %0, %1" : "=v"(last) : "s"(E - 1));
#pragma unroll
        for (int e = 0; e < EMAX; ++e) wr[e] = load1<T>(row + min(e, last));
    }
}

// One token's routing from its E logits l[0..E) (a register array, with
// U = EMAX to unroll every loop over experts, or a row of LDS with U = 1).
//
// Page form: the logits become their softmax over all E experts (max
// subtracted, sum in expert order), written to probs when it is not NULL,
// and the picks and weights are taken on those probabilities.
// Top-k, picked greedily: each pick is the largest value among the experts
// not yet picked; strict '>' keeps the lowest index among equal values.
// Weights: softmax over the picked logits relative to the first, e_0 = 1,
// e_s = exp(l_s - l_0), w_s = e_s / sum (for k = 2: w_0 = 1/(1+q),
// w_1 = q/(1+q)); page form: w_s = p_s / (sum of the kept p).
template <int EMAX, int U, typename Row>
__device__ __forceinline__ void finish_token(Row &l, int E, int k, int page, float *probs,
                                             int t, int32_t *__restrict__ idx,
                                             float *__restrict__ wout) {
    if (page) {
        float m = l[0];
#pragma unroll U
        for (int e = 1; e < EMAX; ++e) {
            if (e >= E) break;
            m = fmaxf(m, l[e]);
        }
        float z = 0.0f;
#pragma unroll U
        for (int e = 0; e < EMAX; ++e) {
            if (e >= E) break;
            const float pe = expf(l[e] - m);
            l[e] = pe;
            z += pe;
        }
#pragma unroll U
        for (int e = 0; e < EMAX; ++e) {
            if (e >= E) break;
            l[e] = l[e] / z;
            if (probs) probs[(size_t)t * E + e] = l[e];
        }
    }
    int sel[kMaxTopK];
    float ls[kMaxTopK];
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s) {
        sel[s] = -1;
        ls[s] = 0.0f;
        if (s >= k) continue;
#pragma unroll U
        for (int e = 0; e < EMAX; ++e) {
            if (e >= E) break;
            bool taken = false;
#pragma unroll
            for (int r = 0; r < s; ++r) taken |= sel[r] == e;
            const float le = l[e];
            if (!taken && (sel[s] < 0 || le > ls[s])) { sel[s] = e; ls[s] = le; }
        }
    }
    float ex[kMaxTopK], sum = 0.0f;
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s) {
        ex[s] = page ? ls[s] : s == 0 ? 1.0f : expf(ls[s] - ls[0]);
        if (s < k) sum += ex[s];
    }
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s) {
        if (s >= k) break;
        idx[k * t + s] = sel[s];
        wout[k * t + s] = ex[s] / sum;
    }
}

// One workgroup (4 wavefronts) owns TPB consecutive tokens.  Thread i walks
// d in 8-element chunks i, i+256, ...; per-thread partial logits are summed
// across each wavefront with a butterfly and then across the four
// wavefronts in LDS, in a fixed order.
//
// NORM: the router input is the RMSNorm of the rows ("Mixtral 8x7B -- The
// Evolving Transformer", section 03 RMSNORM; section 06 BLOCK applies
// rms_2 before the MoE).
// A first pass sums each row's squares (fixed-order reduction as above),
// rstd = 1/sqrt(sum/d + eps); the second pass re-reads the row (from L2),
// forms xn = round(x * rstd * g) in the element type, writes it to xn_out
// for the experts, and feeds the rounded values to the router.
template <typename T, int EMAX, int TPB, bool NORM>
__global__ __launch_bounds__(256) void route_kernel(const T *__restrict__ x,
                                                    const T *__restrict__ wg, int n_tok,
                                                    int d, int E, int k,
                                                    int32_t *__restrict__ idx,
                                                    float *__restrict__ wout,
                                                    const T *__restrict__ g, float eps,
                                                    T *__restrict__ xn_out, int page,
                                                    float *__restrict__ probs) {
    __shared__ float part[4][TPB][EMAX];
    __shared__ float ssq[4][TPB];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t0 = blockIdx.x * TPB;
    const int nchunk = d >> 3;

    float rstd[TPB];
    if constexpr (NORM) {
        float sq[TPB];
#pragma unroll
        for (int tt = 0; tt < TPB; ++tt) sq[tt] = 0.0f;
        for (int c = tid; c < nchunk; c += 256) {
#pragma unroll
            for (int tt = 0; tt < TPB; ++tt) {
                float v[8];
                load8<T>(x + (size_t)min(t0 + tt, n_tok - 1) * d + c * 8, v);
#pragma unroll
                for (int i = 0; i < 8; ++i) sq[tt] += v[i] * v[i];
            }
        }
#pragma unroll
        for (int tt = 0; tt < TPB; ++tt) {
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) sq[tt] += __shfl_xor(sq[tt], off, 64);
            if (lane == 0) ssq[wave][tt] = sq[tt];
        }
        __syncthreads();
#pragma unroll
        for (int tt = 0; tt < TPB; ++tt)
            rstd[tt] = 1.0f / sqrtf(((ssq[0][tt] + ssq[1][tt]) + (ssq[2][tt] + ssq[3][tt])) /
                                        (float)d + eps);
    }

    float acc[TPB][EMAX];
#pragma unroll
    for (int tt = 0; tt < TPB; ++tt)
#pragma unroll
        for (int e = 0; e < EMAX; ++e) acc[tt][e] = 0.0f;

    // The row loader's form is fixed for the whole loop (E is uniform), so
    // the loop body holds no branch around its loads.
    auto chunks = [&](auto vec_c) __attribute__((always_inline)) {
        constexpr bool VEC = decltype(vec_c)::value;
        for (int c = tid; c < nchunk; c += 256) {
            float xv[TPB][8];
#pragma unroll
            for (int tt = 0; tt < TPB; ++tt) {
                const int t = min(t0 + tt, n_tok - 1);
                load8<T>(x + (size_t)t * d + c * 8, xv[tt]);
            }
            if constexpr (NORM) {
                float gv[8];
                load8<T>(g + c * 8, gv);
#pragma unroll
                for (int tt = 0; tt < TPB; ++tt) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) xv[tt][i] = xv[tt][i] * rstd[tt] * gv[i];
                    store8<T>(xn_out + (size_t)min(t0 + tt, n_tok - 1) * d + c * 8, xv[tt]);
                    // the router sees the rounded values the experts will see
#pragma unroll
                    for (int i = 0; i < 8; ++i) xv[tt][i] = round_to<T>(xv[tt][i]);
                }
            }
            // Router rows are read 8 at a time when few values are accumulated;
            // wider rows (32+ experts per token) go one or two at a time so that
            // the accumulators and the row stay in registers.
            constexpr int RU = EMAX >= 64 ? 1 : EMAX >= 32 ? 2 : 8;
#pragma unroll RU
            for (int r = 0; r < 8; ++r) {
                float wr[EMAX];
                load_router_row<T, EMAX, VEC>(wg + (size_t)(c * 8 + r) * E, E, wr);
#pragma unroll
                for (int tt = 0; tt < TPB; ++tt)
#pragma unroll
                    for (int e = 0; e < EMAX; ++e) acc[tt][e] += xv[tt][r] * wr[e];
            }
        }
    };
    if (E % (16 / (int)sizeof(T)) == 0)
        chunks(std::true_type{});
    else
        chunks(std::false_type{});
    // Reduce-scatter butterfly over the wavefront: at each step a lane keeps
    // half of its remaining values and adds its partner's copy of that half,
    // so after log2(64) steps lane l holds the wavefront sum of value l
    // (63 exchanges instead of 6 per value).  The pairing is fixed, so the
    // result is the same on every call.
    constexpr int NV = TPB * EMAX;   // values per lane (8 .. 64)
    constexpr int RS = NV >= 64 ? 6 : NV >= 32 ? 5 : NV >= 16 ? 4 : 3;  // log2(NV)
    static_assert((1 << RS) == NV, "values per lane must be a power of two");
    float v[NV];
#pragma unroll
    for (int tt = 0; tt < TPB; ++tt)
#pragma unroll
        for (int e = 0; e < EMAX; ++e) v[tt * EMAX + e] = acc[tt][e];
    // Steps with partner distance 32, 16, ... (RS of them): lanes with that
    // bit clear keep the lower half of the remaining values, the others the
    // upper half.  Afterwards lane l holds value l >> (6 - RS), summed over
    // the lanes that differ from it in the top RS bits; a plain butterfly
    // over the remaining low bits completes the sum.
#pragma unroll
    for (int st = 0, n = NV; st < RS; ++st, n >>= 1) {
        const int off = 32 >> st;
        const bool upper = (lane & off) != 0;
#pragma unroll
        for (int i = 0; i < n / 2; ++i) {
            const float send = upper ? v[i] : v[i + n / 2];
            const float keep = upper ? v[i + n / 2] : v[i];
            v[i] = keep + __shfl_xor(send, off, 64);
        }
    }
#pragma unroll
    for (int off = 32 >> RS; off >= 1; off >>= 1) v[0] += __shfl_xor(v[0], off, 64);
    if ((lane & ((64 >> RS) - 1)) == 0) {
        const int vi = lane >> (6 - RS);
        part[wave][vi / EMAX][vi % EMAX] = v[0];
    }
    __syncthreads();
    if (tid >= TPB) return;
    const int t = t0 + tid;
    if (t >= n_tok) return;
    // The token's logits, summed over the four wavefronts in a fixed order.
    // Up to 16 experts they sit in registers and every loop over experts is
    // unrolled; wider rows stay in this thread's row of LDS (no other
    // thread touches it) and the loops stay rolled.
    if constexpr (EMAX <= 16) {
        float l[EMAX];
#pragma unroll
        for (int e = 0; e < EMAX; ++e)
            l[e] = ((part[0][tid][e] + part[1][tid][e]) + part[2][tid][e]) + part[3][tid][e];
        finish_token<EMAX, EMAX>(l, E, k, page, probs, t, idx, wout);
    } else {
        float *l = part[0][tid];
#pragma unroll 1
        for (int e = 0; e < E; ++e)
            l[e] = ((part[0][tid][e] + part[1][tid][e]) + part[2][tid][e]) + part[3][tid][e];
        finish_token<EMAX, 1>(l, E, k, page, probs, t, idx, wout);
    }
}

// Router options: RMSNorm in front (g, eps, xn) and the page form (page,
// probs).
struct RouteOpts {
    const void *g = nullptr;
    float eps = 0.0f;
    void *xn = nullptr;
    int page = 0;
    float *probs = nullptr;
};

template <typename T, int EMAX, int TPB>
hipError_t launch_route_t(const moe_shape_t &s, const void *x, const void *wg, int32_t *idx,
                          float *w, const RouteOpts &o, hipStream_t stream) {
    const int blocks = (s.T + TPB - 1) / TPB;
    if (o.g)
        hipLaunchKernelGGL((route_kernel<T, EMAX, TPB, true>), dim3(blocks), dim3(256), 0,
                           stream, static_cast<const T *>(x), static_cast<const T *>(wg), s.T,
                           s.d_model, s.n_experts, s.top_k, idx, w, static_cast<const T *>(o.g),
                           o.eps, static_cast<T *>(o.xn), o.page, o.probs);
    else
        hipLaunchKernelGGL((route_kernel<T, EMAX, TPB, false>), dim3(blocks), dim3(256), 0,
                           stream, static_cast<const T *>(x), static_cast<const T *>(wg), s.T,
                           s.d_model, s.n_experts, s.top_k, idx, w, nullptr, 0.0f, nullptr,
                           o.page, o.probs);
    return hipGetLastError();
}

// Few tokens: one token per workgroup, so that enough workgroups share the
// reduction over d.  Many tokens: eight per workgroup, reusing each router
// row read for all of them.
template <typename T>
hipError_t launch_route_dtype(const moe_shape_t &s, const void *x, const void *wg,
                              int32_t *idx, float *w, const RouteOpts &o, hipStream_t stream) {
    const bool few = s.T <= 256;
    if (s.n_experts <= 8)
        return few ? launch_route_t<T, 8, 1>(s, x, wg, idx, w, o, stream)
                   : launch_route_t<T, 8, 8>(s, x, wg, idx, w, o, stream);
    if (s.n_experts <= 16)
        return few ? launch_route_t<T, 16, 1>(s, x, wg, idx, w, o, stream)
                   : launch_route_t<T, 16, 4>(s, x, wg, idx, w, o, stream);
    if (s.n_experts <= 32)
        return few ? launch_route_t<T, 32, 1>(s, x, wg, idx, w, o, stream)
                   : launch_route_t<T, 32, 2>(s, x, wg, idx, w, o, stream);
    // 64 logits per token already fill the reduce-scatter's 64 lanes
    return launch_route_t<T, 64, 1>(s, x, wg, idx, w, o, stream);
}

}  // namespace

hipError_t launch_route(const moe_shape_t &s, const void *x, const void *w_gate, int32_t *idx,
                        float *w, hipStream_t stream) {
    return launch_route_norm(s, x, nullptr, 0.0f, w_gate, nullptr, idx, w, stream);
}

namespace {
hipError_t launch_route_opts(const moe_shape_t &s, const void *x, const void *w_gate,
                             int32_t *idx, float *w, const RouteOpts &o, hipStream_t stream) {
    if (s.T == 0) return hipSuccess;
    if (s.dtype == MOE_BF16) return launch_route_dtype<uint16_t>(s, x, w_gate, idx, w, o, stream);
    return launch_route_dtype<float>(s, x, w_gate, idx, w, o, stream);
}
}  // namespace

hipError_t launch_route_norm(const moe_shape_t &s, const void *x, const void *g, float eps,
                             const void *w_gate, void *xn, int32_t *idx, float *w,
                             hipStream_t stream) {
    RouteOpts o;
    o.g = g;
    o.eps = eps;
    o.xn = xn;
    return launch_route_opts(s, x, w_gate, idx, w, o, stream);
}

hipError_t launch_route_probs(const moe_shape_t &s, const void *x, const void *w_gate,
                              float *probs, int32_t *idx, float *w, hipStream_t stream) {
    RouteOpts o;
    o.page = 1;
    o.probs = probs;
    return launch_route_opts(s, x, w_gate, idx, w, o, stream);
}

}  // namespace moe
