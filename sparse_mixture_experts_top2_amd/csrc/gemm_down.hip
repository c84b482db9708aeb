// Prefill down product (o = h W2[e], fp32, whole or in K parts) on the
// pipelined tile body of gemm_bf16.h.
#include "gemm_bf16.h"

namespace moe {
namespace {

__global__ __launch_bounds__(QT, 1) void q_down_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B, float *__restrict__ C,
    const int32_t *__restrict__ counts, const int32_t *__restrict__ offsets, int E, int K, int N,
    int a_rows, int cu_per_xcd) {
    QArgs g{};
    g.A = A; g.B0 = B; g.C = C;
    g.K = K; g.N = N; g.a_lines = a_rows; g.lda = K;
    q_body<QMode<1, QE_F32>>(g, counts, offsets, E, 1, cu_per_xcd, nullptr);
}

__global__ __launch_bounds__(QT, 1) void q_down_split_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B, float *__restrict__ C,
    const int32_t *__restrict__ counts, const int32_t *__restrict__ offsets, int E, int K, int N,
    int a_rows, int parts, size_t part_stride, int cu_per_xcd, int *__restrict__ parts_out) {
    QArgs g{};
    g.A = A; g.B0 = B; g.C = C;
    g.K = K; g.N = N; g.a_lines = a_rows; g.lda = K;
    g.part_stride = part_stride;
    q_body<QMode<1, QE_F32, false, true>>(g, counts, offsets, E, parts, cu_per_xcd, parts_out);
}

}  // namespace

bool q_down_supported(int rows, int K, int N) { return q_fits(rows, K, N, QBN); }

hipError_t q_launch_down(int rows, int E, const uint16_t *h, const int32_t *counts,
                         const int32_t *offsets, const uint16_t *w2, int K, int N, float *o,
                         int parts, size_t part_stride, int /*cu_per_xcd*/, int *parts_out,
                         hipStream_t stream) {
    if (!q_down_supported(rows, K, N)) return hipErrorNotSupported;
    const int cpx = q_cus_per_xcd();
    if (cpx < 0) return hipErrorNotSupported;
    if (parts == 1 && !parts_out) {
        hipLaunchKernelGGL(q_down_kernel, dim3(8 * cpx), dim3(QT), 0, stream, h, w2, o, counts,
                           offsets, E, K, N, rows, cpx);
        return hipGetLastError();
    }
    if (K / QBK < QMAXSPLIT) return hipErrorNotSupported;
    hipLaunchKernelGGL(q_down_split_kernel, dim3(8 * cpx), dim3(QT), 0, stream, h, w2, o, counts,
                       offsets, E, K, N, rows, parts, part_stride, cpx, parts_out);
    return hipGetLastError();
}

}  // namespace moe
