// fp32 expert path: grouped SwiGLU ("Mixtral 8x7B -- The Evolving
// Transformer", section 04: down(silu(gate x) * up x)) over the expert-sorted
// rows, with plain fp32 FMA on LDS tiles.  This path serves fp32 layers,
// which are small parity configurations here; the bf16 paths carry the
// large shapes on the matrix cores.
//
// Each workgroup computes a 64 x 64 output tile of one expert: the gate/up
// kernel keeps two accumulators (gate and up) per output and applies
// silu(g) * u in its epilogue, the down kernel keeps one.  Each thread owns
// a 4 x 4 sub-tile; the reduction over K runs in ascending order.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int BM = 64, BN = 64, BK = 16;

template <int NMAT>
__global__ __launch_bounds__(256) void gemm_f32_kernel(
    const float *__restrict__ A, const float *__restrict__ B0, const float *__restrict__ B1,
    float *__restrict__ C, const int32_t *__restrict__ counts,
    const int32_t *__restrict__ offsets, int E, int K, int N, int a_rows) {
    int e, row0, row_end;
    if (!find_row_tile(counts, offsets, E, BM, blockIdx.y, e, row0, row_end)) return;
    const int n0 = blockIdx.x * BN;
    __shared__ float As[BK][BM + 4];
    __shared__ float Bs[NMAT][BK][BN];

    const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
    const float *Bm[2] = {B0 + (size_t)e * K * N, NMAT > 1 ? B1 + (size_t)e * K * N : nullptr};
    float acc[NMAT][4][4] = {};

    for (int k0 = 0; k0 < K; k0 += BK) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int v = tid + 256 * i;
            const int r = v / BK, kk = v % BK;
            // rows past the end of A are clamped (their results are not stored)
            const size_t ar = (size_t)min(row0 + r, a_rows - 1);
            As[kk][r] = k0 + kk < K ? A[ar * K + k0 + kk] : 0.0f;
        }
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int v = tid + 256 * i;
                const int kk = v / BN, c = v % BN;
                Bs[m][kk][c] = (k0 + kk < K && n0 + c < N)
                                   ? Bm[m][(size_t)(k0 + kk) * N + n0 + c] : 0.0f;
            }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < BK; ++kk) {
            float a[4], b[NMAT][4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
#pragma unroll
                for (int j = 0; j < 4; ++j) b[m][j] = Bs[m][kk][tx * 4 + j];
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[m][i][j] += a[i] * b[m][j];
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = row0 + ty * 4 + i;
        if (row >= row_end) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = n0 + tx * 4 + j;
            if (col >= N) continue;
            float v = acc[0][i][j];
            if (NMAT == 2) v = silu_f32(v) * acc[NMAT - 1][i][j];
            C[(size_t)row * N + col] = v;
        }
    }
}

}  // namespace

hipError_t launch_gateup_f32(const moe_shape_t &s, const float *xp, const int32_t *counts,
                             const int32_t *offsets, const float *w1, const float *w3,
                             float *h, hipStream_t stream) {
    const int d = s.d_model, f = s.d_ff, E = s.n_experts;
    const int m_tiles = (routed_rows(s) + BM - 1) / BM + E;
    hipLaunchKernelGGL(gemm_f32_kernel<2>, dim3((f + BN - 1) / BN, m_tiles), dim3(256), 0,
                       stream, xp, w1, w3, h, counts, offsets, E, d, f, routed_rows(s));
    return hipGetLastError();
}

hipError_t launch_down_f32(const moe_shape_t &s, const float *h, const int32_t *counts,
                           const int32_t *offsets, const float *w2, float *o,
                           hipStream_t stream) {
    const int d = s.d_model, f = s.d_ff, E = s.n_experts;
    const int m_tiles = (routed_rows(s) + BM - 1) / BM + E;
    hipLaunchKernelGGL(gemm_f32_kernel<1>, dim3((d + BN - 1) / BN, m_tiles), dim3(256), 0,
                       stream, h, w2, nullptr, o, counts, offsets, E, f, d, routed_rows(s));
    return hipGetLastError();
}

}  // namespace moe
