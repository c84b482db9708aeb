// Backward weight gradients (per-expert products over the expert's rows)
// and the K-contiguous padded copies they read, on the pipelined tile body
// of gemm_bf16.h.
#include "gemm_bf16.h"

namespace moe {
namespace {

// Backward weight gradients from K-contiguous padded copies: NMAT = 2:
// dW1[e] = Xt_e^T dGt_e and dW3[e] = Xt_e^T dUt_e (B0 = dGt, B1 = dUt, C, C2);
// NMAT = 1: dW2[e] = Ht_e^T dOt_e.  At [M, ldk], B [N, ldk].
template <int NMAT>
__global__ __launch_bounds__(QT, 1) void q_dw_kernel(
    const uint16_t *__restrict__ At, const uint16_t *__restrict__ B0t,
    const uint16_t *__restrict__ B1t, float *__restrict__ C, float *__restrict__ C2,
    const int32_t *__restrict__ counts, int E, int M, int N, int ldk, int cu_per_xcd) {
    QArgs g{};
    g.A = At; g.B0 = B0t; g.B1 = B1t; g.C = C; g.C2 = C2;
    g.M = M; g.N = N; g.a_lines = M; g.lda = ldk; g.ldb = ldk;
    g.K = ldk;
    q_body_dw<QMode<NMAT, QE_DW, false, false, true, false, true>>(g, counts, E, cu_per_xcd);
}

// K-contiguous padded copy for the weight gradients: dst [C, ldk] with
// dst[c][kp_e + r] = src[offsets[e] + r][c] for each expert e and its rows
// r < counts[e], where kp_e = sum over experts before e of their counts
// rounded up to 64; the columns from kp_e + counts[e] up to the next
// multiple of 64 are zero.  One block per 64 padded rows of one expert and
// 64 columns, transposed through LDS; every global access is 16 bytes.
__global__ __launch_bounds__(256) void q_transpose_pad_kernel(
    const uint16_t *__restrict__ src, int C, const int32_t *__restrict__ counts,
    const int32_t *__restrict__ offsets, int E, uint16_t *__restrict__ dst, int ldk) {
    int e = -1, lt = 0, kp = 0;
    for (int i = 0, acc = 0; i < E; ++i) {
        const int nt = (counts[i] + 63) / 64;
        if ((int)blockIdx.x < acc + nt) {
            e = i;
            lt = blockIdx.x - acc;
            break;
        }
        acc += nt;
        kp += nt * 64;
    }
    if (e < 0) return;
    const int c0 = blockIdx.y * 64, r_lo = lt * 64, cnt = counts[e], s0 = offsets[e];
    // Row pitch 65 (130 bytes): the column reads of 8 rows 8 apart fall on
    // distinct banks (the writes at most 2 to a bank).
    __shared__ uint16_t tile[64][65];
    const int tid = threadIdx.x;
#pragma unroll
    for (int ch = tid; ch < 512; ch += 256) {
        const int r = ch >> 3, cc = (ch & 7) * 8;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (r_lo + r < cnt)
            v = *reinterpret_cast<const uint4 *>(src + (size_t)(s0 + r_lo + r) * C + c0 + cc);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            tile[r][cc + 2 * k] = (uint16_t)(w[k] & 0xffffu);
            tile[r][cc + 2 * k + 1] = (uint16_t)(w[k] >> 16);
        }
    }
    __syncthreads();
#pragma unroll
    for (int ch = tid; ch < 512; ch += 256) {
        const int c = ch >> 3, rr = (ch & 7) * 8;
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            w[k] = (uint32_t)tile[rr + 2 * k][c] | ((uint32_t)tile[rr + 2 * k + 1][c] << 16);
        *reinterpret_cast<uint4 *>(dst + (size_t)(c0 + c) * ldk + kp + r_lo + rr) =
            make_uint4(w[0], w[1], w[2], w[3]);
    }
}

}  // namespace

int q_dw_ldk(int rows, int E) { return (rows + 63) / 64 * 64 + 64 * E; }

bool q_dw_supported(int rows, int E, int d, int f) {
    const uint64_t ldk = (uint64_t)q_dw_ldk(rows, E);
    return rows > 0 && d % QBN == 0 && f % QBN == 0 && (uint64_t)f * ldk * 2 < ((uint64_t)1 << 32);
}

hipError_t q_launch_transpose_pad(const uint16_t *src, int rows, int C, const int32_t *counts,
                                  const int32_t *offsets, int E, uint16_t *dst, int ldk,
                                  hipStream_t stream) {
    if (rows <= 0 || C % 64 != 0) return hipErrorNotSupported;
    const dim3 grid((unsigned)((rows + 63) / 64 + E), (unsigned)(C / 64));
    hipLaunchKernelGGL(q_transpose_pad_kernel, grid, dim3(256), 0, stream, src, C, counts,
                       offsets, E, dst, ldk);
    return hipGetLastError();
}

hipError_t q_launch_dw(int nmat, const uint16_t *At, const uint16_t *B0t, const uint16_t *B1t,
                       float *C, float *C2, const int32_t *counts, int E, int M, int N, int ldk,
                       hipStream_t stream) {
    const int cpx = q_cus_per_xcd();
    if (cpx < 0 || M % QBM != 0 || N % (QBN / nmat) != 0) return hipErrorNotSupported;
    if (nmat == 2)
        hipLaunchKernelGGL(q_dw_kernel<2>, dim3(8 * cpx), dim3(QT), 0, stream, At, B0t, B1t, C,
                           C2, counts, E, M, N, ldk, cpx);
    else
        hipLaunchKernelGGL(q_dw_kernel<1>, dim3(8 * cpx), dim3(QT), 0, stream, At, B0t, nullptr,
                           C, nullptr, counts, E, M, N, ldk, cpx);
    return hipGetLastError();
}

}  // namespace moe
