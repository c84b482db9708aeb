// Backward products through the transposed weights (da = dO W2[e]^T with
// the dSwiGLU epilogue; dXp = dG W1[e]^T + dU W3[e]^T in K parts) on the
// pipelined tile body of gemm_bf16.h.
#include "gemm_bf16.h"

namespace moe {
namespace {

// Backward: z = dY W2[e]^T for the routed rows' dy, da = w z with dg, du
// in the epilogue, and the per-column-tile partial sums of h . z (B
// K-contiguous: W2[e] [f, d] read along d).
__global__ __launch_bounds__(QT, 1) void q_bt_dswiglu_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B,
    const int32_t *__restrict__ counts, const int32_t *__restrict__ offsets, int E, int K1, int N,
    int a_rows, const float *__restrict__ gin, const float *__restrict__ uin,
    uint16_t *__restrict__ dg, uint16_t *__restrict__ du, const float *__restrict__ w_row,
    const uint16_t *__restrict__ h, float *__restrict__ dw_part, int cu_per_xcd) {
    QArgs g{};
    g.A = A; g.B0 = B; g.C = dg; g.C2 = du;
    g.K = K1; g.N = N; g.a_lines = a_rows; g.lda = K1; g.ldb = K1;
    g.g_in = gin; g.u_in = uin;
    g.w_row = w_row; g.h_in = h; g.dw_part = dw_part;
    q_body<QMode<1, QE_DSWIGLU, false, false, true>>(g, counts, offsets, E, 1, cu_per_xcd,
                                                     nullptr);
}

// Backward: dXp = dG W1[e]^T + dU W3[e]^T over a reduction of 2 K1, cut in
// parts (B, B2 K-contiguous: W1[e], W3[e] [d, f] read along f).
__global__ __launch_bounds__(QT, 1) void q_bt_store_split_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B, const uint16_t *__restrict__ A2,
    const uint16_t *__restrict__ B2, float *__restrict__ C, const int32_t *__restrict__ counts,
    const int32_t *__restrict__ offsets, int E, int K1, int N, int a_rows, size_t part_stride,
    int cu_per_xcd, int *__restrict__ parts_out) {
    QArgs g{};
    g.A = A; g.B0 = B; g.A2 = A2; g.B2 = B2; g.C = C;
    g.K = 2 * K1; g.K1 = K1; g.N = N; g.a_lines = a_rows; g.lda = K1; g.ldb = K1;
    g.part_stride = part_stride;
    q_body<QMode<1, QE_F32, false, true, true, true>>(g, counts, offsets, E, 0, cu_per_xcd,
                                                      parts_out);
}

}  // namespace

// Backward products with K-contiguous weights (see moe_internal.h).
bool q_bt_dswiglu_supported(int rows, int K1, int N) {
    return q_fits(rows, K1, N, QBN) && (uint64_t)N * K1 * 2 < ((uint64_t)1 << 32);
}

hipError_t q_launch_bt_dswiglu(int rows, int E, const uint16_t *dyp, const uint16_t *w2, int K1,
                               int N, const int32_t *counts, const int32_t *offsets,
                               const float *g, const float *u, uint16_t *dg, uint16_t *du,
                               const float *w_row, const uint16_t *h, float *dw_part,
                               hipStream_t stream) {
    if (!q_bt_dswiglu_supported(rows, K1, N)) return hipErrorNotSupported;
    const int cpx = q_cus_per_xcd();
    if (cpx < 0) return hipErrorNotSupported;
    hipLaunchKernelGGL(q_bt_dswiglu_kernel, dim3(8 * cpx), dim3(QT), 0, stream, dyp, w2, counts,
                       offsets, E, K1, N, rows, g, u, dg, du, w_row, h, dw_part, cpx);
    return hipGetLastError();
}

hipError_t q_launch_bt_store_split(int rows, int E, const uint16_t *A, const uint16_t *B,
                                   const uint16_t *A2, const uint16_t *B2, int K1, int N,
                                   const int32_t *counts, const int32_t *offsets, float *C,
                                   size_t part_stride, int *parts_out, hipStream_t stream) {
    if (!q_fits(rows, K1, N, QBN) || (uint64_t)N * K1 * 2 >= ((uint64_t)1 << 32) || !parts_out)
        return hipErrorNotSupported;
    const int cpx = q_cus_per_xcd();
    if (cpx < 0) return hipErrorNotSupported;
    hipLaunchKernelGGL(q_bt_store_split_kernel, dim3(8 * cpx), dim3(QT), 0, stream, A, B, A2, B2,
                       C, counts, offsets, E, K1, N, rows, part_stride, cpx, parts_out);
    return hipGetLastError();
}

}  // namespace moe
