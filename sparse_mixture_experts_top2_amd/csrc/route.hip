// Router: logits = x w_gate (fp32), top-2 with lowest-index ties, softmax
// over the two kept logits.  "Mixtral 8x7B -- The Evolving Transformer",
// section 05 (MoERouter and the formula y = sum_k w_k E_{i_k}(x)).
//
// One wavefront owns TPW tokens.  Lane l walks d in 8-element chunks
// l, l+64, l+128, ... and keeps per-expert partial sums for its tokens;
// a butterfly across the 64 lanes then completes every logit in every lane.
// The router matrix (d x E, 64 KiB at the 8x7B shape) is read once per
// wavefront from L2 and reused for its TPW tokens.  The kernel is bound by
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

template <typename T>
__device__ __forceinline__ float load1(const T *p);
template <>
__device__ __forceinline__ float load1<float>(const float *p) { return *p; }
template <>
__device__ __forceinline__ float load1<uint16_t>(const uint16_t *p) { return bf16_to_f32(*p); }

template <typename T, int EMAX, int TPW>
__global__ __launch_bounds__(256) void route_kernel(const T *__restrict__ x,
                                                    const T *__restrict__ wg, int n_tok,
                                                    int d, int E, int32_t *__restrict__ idx,
                                                    float *__restrict__ wout) {
    const int lane = threadIdx.x & 63;
    const int t0 = (blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)) * TPW;
    if (t0 >= n_tok) return;

    float acc[TPW][EMAX];
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
        for (int e = 0; e < EMAX; ++e) acc[tt][e] = 0.0f;

    const int nchunk = d >> 3;
    for (int c = lane; c < nchunk; c += 64) {
        float xv[TPW][8];
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) {
            int t = t0 + tt < n_tok ? t0 + tt : n_tok - 1;
            load8<T>(x + (size_t)t * d + c * 8, xv[tt]);
        }
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const T *wrow = wg + (size_t)(c * 8 + r) * E;
            float wr[EMAX];
#pragma unroll
            for (int e = 0; e < EMAX; ++e) wr[e] = e < E ? load1<T>(wrow + e) : 0.0f;
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
                for (int e = 0; e < EMAX; ++e) acc[tt][e] += xv[tt][r] * wr[e];
        }
    }
    // Butterfly over the wavefront: fixed pairing, so the result is the same
    // on every call (and identical in every lane).
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
            for (int e = 0; e < EMAX; ++e) acc[tt][e] += __shfl_xor(acc[tt][e], off, 64);

#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
        const int t = t0 + tt;
        if (lane != tt || t >= n_tok) continue;
        int i0 = 0;
        float l0 = acc[tt][0];
#pragma unroll
        for (int e = 1; e < EMAX; ++e)
            if (e < E && acc[tt][e] > l0) { i0 = e; l0 = acc[tt][e]; }
        int i1 = -1;
        float l1 = 0.0f;
#pragma unroll
        for (int e = 0; e < EMAX; ++e)
            if (e < E && e != i0 && (i1 < 0 || acc[tt][e] > l1)) { i1 = e; l1 = acc[tt][e]; }
        const float q = expf(l1 - l0);
        idx[2 * t] = i0;
        idx[2 * t + 1] = i1;
        wout[2 * t] = 1.0f / (1.0f + q);
        wout[2 * t + 1] = q / (1.0f + q);
    }
}

template <typename T, int EMAX, int TPW>
hipError_t launch_route_t(const moe_shape_t &s, const void *x, const void *wg, int32_t *idx,
                          float *w, hipStream_t stream) {
    const int waves = (s.T + TPW - 1) / TPW;
    const int blocks = (waves + 3) / 4;
    hipLaunchKernelGGL((route_kernel<T, EMAX, TPW>), dim3(blocks), dim3(256), 0, stream,
                       static_cast<const T *>(x), static_cast<const T *>(wg), s.T, s.d_model,
                       s.n_experts, idx, w);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_route_dtype(const moe_shape_t &s, const void *x, const void *wg,
                              int32_t *idx, float *w, hipStream_t stream) {
    if (s.n_experts <= 8) return launch_route_t<T, 8, 4>(s, x, wg, idx, w, stream);
    if (s.n_experts <= 16) return launch_route_t<T, 16, 2>(s, x, wg, idx, w, stream);
    return launch_route_t<T, 32, 1>(s, x, wg, idx, w, stream);
}

}  // namespace

hipError_t launch_route(const moe_shape_t &s, const void *x, const void *w_gate, int32_t *idx,
                        float *w, hipStream_t stream) {
    if (s.T == 0) return hipSuccess;
    if (s.dtype == MOE_BF16)
        return launch_route_dtype<uint16_t>(s, x, w_gate, idx, w, stream);
    return launch_route_dtype<float>(s, x, w_gate, idx, w, stream);
}

}  // namespace moe
