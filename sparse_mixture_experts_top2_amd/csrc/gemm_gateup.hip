// Prefill gate/up product (h = silu(A W1[e]) * (A W3[e]), bf16; in the
// backward also g and u) on the pipelined tile body of gemm_bf16.h.
#include "gemm_bf16.h"

namespace moe {
namespace {

__global__ __launch_bounds__(QT, 1) void q_gateup_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B0,
    const uint16_t *__restrict__ B1, uint16_t *__restrict__ C, const int32_t *__restrict__ counts,
    const int32_t *__restrict__ offsets, int E, int K, int N, int a_rows, int cu_per_xcd) {
    QArgs g{};
    g.A = A; g.B0 = B0; g.B1 = B1; g.C = C;
    g.K = K; g.N = N; g.a_lines = a_rows; g.lda = K;
    q_body<QMode<2, QE_SWIGLU>>(g, counts, offsets, E, 1, cu_per_xcd, nullptr);
}

__global__ __launch_bounds__(QT, 1) void q_gateup_gu_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B0,
    const uint16_t *__restrict__ B1, uint16_t *__restrict__ C, const int32_t *__restrict__ counts,
    const int32_t *__restrict__ offsets, int E, int K, int N, int a_rows, int cu_per_xcd,
    float *__restrict__ gp, float *__restrict__ up) {
    QArgs g{};
    g.A = A; g.B0 = B0; g.B1 = B1; g.C = C;
    g.K = K; g.N = N; g.a_lines = a_rows; g.lda = K;
    g.g_out = gp; g.u_out = up;
    q_body<QMode<2, QE_SWIGLU, true>>(g, counts, offsets, E, 1, cu_per_xcd, nullptr);
}

}  // namespace

bool q_gateup_supported(int rows, int K, int N) { return q_fits(rows, K, N, QBN / 2); }

hipError_t q_launch_gateup(int rows, int E, const uint16_t *xp, const int32_t *counts,
                           const int32_t *offsets, const uint16_t *w1, const uint16_t *w3, int K,
                           int N, uint16_t *h, float *g, float *u, hipStream_t stream) {
    if (!q_gateup_supported(rows, K, N)) return hipErrorNotSupported;
    const int cpx = q_cus_per_xcd();
    if (cpx < 0) return hipErrorNotSupported;
    if (g)
        hipLaunchKernelGGL(q_gateup_gu_kernel, dim3(8 * cpx), dim3(QT), 0, stream, xp, w1, w3, h,
                           counts, offsets, E, K, N, rows, cpx, g, u);
    else
        hipLaunchKernelGGL(q_gateup_kernel, dim3(8 * cpx), dim3(QT), 0, stream, xp, w1, w3, h,
                           counts, offsets, E, K, N, rows, cpx);
    return hipGetLastError();
}

}  // namespace moe
