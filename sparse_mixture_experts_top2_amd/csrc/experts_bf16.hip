// bf16 expert path on the CDNA4 matrix cores: the SwiGLU block of
// "Mixtral 8x7B -- The Evolving Transformer", section 04
// (down(silu(gate x) * up x)), applied to every expert's rows of the
// expert-sorted activations (section 05's per-expert batches).
//
// Weights keep the caller's layout: w1/w3 [E, d, f] and w2 [E, f, d], i.e.
// the reduction index K is the slow one and N is contiguous.  MFMA wants K
// contiguous inside each lane's operand, so every kernel here transposes
// the weight operand on the fly: a thread loads an 8 x 8 block of bf16
// (8 rows of K, 16 bytes = 8 columns of N each) and swaps it in registers,
// giving 8 vectors of 8 consecutive K values, one per column.
//
// Two variants:
//  * prefill (many rows per expert): 128 x 256 output tiles staged through
//    LDS, v_mfma_f32_32x32x16_bf16, four wavefronts in a 2 x 2 arrangement.
//    MFMA-bound when an expert has more rows than the ridge point.
//  * decode (at most 32 rows in total per expert): each workgroup streams
//    one 128-column slab of an expert's weights over the whole K range
//    exactly once, with v_mfma_f32_16x16x32_bf16 covering the few rows.
//    Eight wavefronts split K; their partial sums are added in LDS in a
//    fixed tree order.  HBM-bound: only the selected experts' weights are
//    read, each byte once.
// Both fuse silu(g) * u into the gate/up epilogue and round h to bf16.
#include "moe_internal.h"

namespace moe {
namespace {

__device__ __forceinline__ uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

// r[i] holds row i (8 bf16 along N, two per dword, lower column in the low
// half).  out[c] receives column c: 8 bf16 along K, row 0 in the low half
// of dword 0.
__device__ __forceinline__ void transpose8x8(const uint4 (&r)[8], uint4 (&out)[8]) {
    const uint32_t *w = reinterpret_cast<const uint32_t *>(r);  // w[4*i + p]
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const int p = c >> 1;
        uint32_t q[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t lo = w[4 * (2 * j) + p], hi = w[4 * (2 * j + 1) + p];
            q[j] = (c & 1) ? ((lo >> 16) | (hi & 0xffff0000u))
                           : ((lo & 0x0000ffffu) | (hi << 16));
        }
        out[c] = make_uint4(q[0], q[1], q[2], q[3]);
    }
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) {
    return __builtin_bit_cast(bf16x8_t, v);
}

// ---------------------------------------------------------------------------
// Prefill: LDS-tiled grouped GEMM.
//   NMAT = 2: C = bf16(silu(A B0[e]) * (A B1[e]))   (gate/up, C = h)
//   NMAT = 1: C = fp32(A B0[e])                     (down,    C = o)

constexpr int PBM = 128, PBN = 256, PBK = 64;
constexpr int PLD = PBK + 8;  // LDS row pitch in bf16: 144 bytes keeps 8-lane groups of
                              // 16-byte reads on distinct banks

template <int NMAT>
__global__ __launch_bounds__(256, 2) void prefill_gemm_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B0,
    const uint16_t *__restrict__ B1, void *__restrict__ C, const int32_t *__restrict__ counts,
    const int32_t *__restrict__ offsets, int E, int K, int N, int a_rows) {
    constexpr int BNM = PBN / NMAT;  // columns of each weight matrix in this tile
    int e, row0, row_end;
    if (!find_row_tile(counts, offsets, E, PBM, blockIdx.y, e, row0, row_end)) return;
    const int n0 = blockIdx.x * BNM;

    __shared__ __attribute__((aligned(16))) uint16_t As[PBM * PLD];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[PBN * PLD];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    // Global -> register assignment.  A: four 16-byte vectors per thread.
    // B: one 8 x 8 block per thread (kb = K block, nb = N block).
    const int kb = tid & 7;
    const int mat = NMAT == 2 ? (tid >> 7) : 0;
    const int nb = NMAT == 2 ? ((tid & 127) >> 3) : (tid >> 3);
    const int bcol = n0 + nb * 8;
    const bool bcol_ok = bcol < N;
    const uint16_t *Bp = (mat ? B1 : B0) + (size_t)e * K * N + (bcol_ok ? bcol : 0);
    // Rows past the last expert-sorted row are clamped onto it: a row tile
    // may run past the end of A, and those rows are never stored.
    const uint16_t *Arow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        Arow[i] = A + (size_t)min(row0 + ((tid + 256 * i) >> 3), a_rows - 1) * K;

    uint4 ra[4], rb[8];
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int k = k0 + ((tid + 256 * i) & 7) * 8;
            ra[i] = k < K ? *reinterpret_cast<const uint4 *>(Arow[i] + k) : zero4();
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int k = k0 + kb * 8 + i;
            rb[i] = (k < K && bcol_ok) ? *reinterpret_cast<const uint4 *>(Bp + (size_t)k * N)
                                       : zero4();
        }
    };
    auto lstore = [&]() {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int v = tid + 256 * i;
            *reinterpret_cast<uint4 *>(&As[(v >> 3) * PLD + (v & 7) * 8]) = ra[i];
        }
        uint4 tb[8];
        transpose8x8(rb, tb);
#pragma unroll
        for (int c = 0; c < 8; ++c)
            *reinterpret_cast<uint4 *>(&Bs[(mat * BNM + nb * 8 + c) * PLD + kb * 8]) = tb[c];
    };
    // LDS row (within Bs) of this wave's N block j (0..3).
    auto bcol_lds = [&](int j) {
        if (NMAT == 2) return (j >> 1) * 128 + wn * 64 + (j & 1) * 32;
        return wn * 128 + j * 32;
    };

    f32x16_t acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

    const int nk = (K + PBK - 1) / PBK;
    gload(0);
    for (int kt = 0; kt < nk; ++kt) {
        __syncthreads();
        lstore();
        __syncthreads();
        if (kt + 1 < nk) gload((kt + 1) * PBK);
#pragma unroll
        for (int kk = 0; kk < PBK; kk += 16) {
            const int koff = kk + (lane >> 5) * 8;
            bf16x8_t af[2], bfr[4];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                af[i] = as_bf16x8(*reinterpret_cast<const uint4 *>(
                    &As[(wm * 64 + i * 32 + (lane & 31)) * PLD + koff]));
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bfr[j] = as_bf16x8(*reinterpret_cast<const uint4 *>(
                    &Bs[(bcol_lds(j) + (lane & 31)) * PLD + koff]));
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j],
                                                                         acc[i][j], 0, 0, 0);
        }
    }

    // Epilogue.  32x32 accumulator layout: value q of lane l is row
    // 8*(q/4) + 4*(l/32) + q%4, column l%32 of the block.
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int j = 0; j < (NMAT == 2 ? 2 : 4); ++j) {
            const int col = n0 + (NMAT == 2 ? wn * 64 + j * 32 : wn * 128 + j * 32) + (lane & 31);
            if (col >= N) continue;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int row = row0 + wm * 64 + i * 32 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
                if (row >= row_end) continue;
                if (NMAT == 2) {
                    const float h = silu_f32(acc[i][j][q]) * acc[i][j + 2][q];
                    static_cast<uint16_t *>(C)[(size_t)row * N + col] = (uint16_t)f32_to_bf16(h);
                } else {
                    static_cast<float *>(C)[(size_t)row * N + col] = acc[i][j][q];
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Decode: weight-streaming grouped GEMM for experts with at most 16*MB rows.

constexpr int DWAVES = 8;     // wavefronts per workgroup, splitting K
constexpr int DCOLS = 128;    // weight columns per workgroup

template <int MB, int NMAT>
__global__ __launch_bounds__(DWAVES * 64) void decode_gemm_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B0,
    const uint16_t *__restrict__ B1, void *__restrict__ C, const int32_t *__restrict__ counts,
    const int32_t *__restrict__ offsets, int K, int N, int a_rows) {
    const int e = blockIdx.y;
    const int Me = counts[e];
    if (Me == 0) return;  // an expert no token chose: its weights are never read
    const int r0 = offsets[e];
    const int nmb = min(MB, (Me + 15) >> 4);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kg = lane >> 4, nb = lane & 15;
    const int col = blockIdx.x * DCOLS + nb * 8;
    const bool col_ok = col < N;

    const uint16_t *Bp[NMAT];
    Bp[0] = B0 + (size_t)e * K * N + (col_ok ? col : 0);
    if (NMAT == 2) Bp[NMAT - 1] = B1 + (size_t)e * K * N + (col_ok ? col : 0);
    // Row i*16 + lane%16 of this expert; rows past the end of A are clamped
    // onto its last row (their results are never stored).
    const uint16_t *Arow[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
        Arow[i] = A + (size_t)min(r0 + i * 16 + (lane & 15), a_rows - 1) * K;

    f32x4_t acc[NMAT][MB][8];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[m][i][c] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    const int nks = (K + 31) >> 5;
    const int ks0 = (nks * wave) / DWAVES, ks1 = (nks * (wave + 1)) / DWAVES;
    for (int ks = ks0; ks < ks1; ++ks) {
        const int k = ks * 32 + kg * 8;
        uint4 rb[NMAT][8];
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int i = 0; i < 8; ++i)
                rb[m][i] = (k + i < K && col_ok)
                               ? *reinterpret_cast<const uint4 *>(Bp[m] + (size_t)(k + i) * N)
                               : zero4();
        bf16x8_t af[MB];
#pragma unroll
        for (int i = 0; i < MB; ++i)
            af[i] = as_bf16x8((i < nmb && k < K)
                                  ? *reinterpret_cast<const uint4 *>(Arow[i] + k)
                                  : zero4());
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
            uint4 tb[8];
            transpose8x8(rb[m], tb);
#pragma unroll
            for (int i = 0; i < MB; ++i) {
                if (i >= nmb) continue;
#pragma unroll
                for (int c = 0; c < 8; ++c)
                    acc[m][i][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        af[i], as_bf16x8(tb[c]), acc[m][i][c], 0, 0, 0);
            }
        }
    }

    // Fixed-order tree over the eight wavefronts' partial sums:
    // ((w0+w4)+(w2+w6)) + ((w1+w5)+(w3+w7)).
    __shared__ f32x4_t red[DWAVES / 2][NMAT * 8][64];
#pragma unroll
    for (int i = 0; i < MB; ++i) {
        if (i >= nmb) break;
#pragma unroll
        for (int half = DWAVES / 2; half >= 1; half >>= 1) {
            if (wave >= half && wave < 2 * half)
#pragma unroll
                for (int m = 0; m < NMAT; ++m)
#pragma unroll
                    for (int c = 0; c < 8; ++c) red[wave - half][m * 8 + c][lane] = acc[m][i][c];
            __syncthreads();
            if (wave < half)
#pragma unroll
                for (int m = 0; m < NMAT; ++m)
#pragma unroll
                    for (int c = 0; c < 8; ++c) acc[m][i][c] += red[wave][m * 8 + c][lane];
            __syncthreads();
        }
        if (wave != 0 || !col_ok) continue;
        // 16x16 accumulator layout: value j of lane l is row 4*(l/16) + j,
        // column l%16 of the block; block c holds weight columns 8*(l%16) + c.
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = i * 16 + 4 * kg + j;
            if (row >= Me) continue;
            if (NMAT == 2) {
                uint32_t p[4];
#pragma unroll
                for (int c = 0; c < 8; c += 2) {
                    const float h0 = silu_f32(acc[0][i][c][j]) * acc[NMAT - 1][i][c][j];
                    const float h1 = silu_f32(acc[0][i][c + 1][j]) * acc[NMAT - 1][i][c + 1][j];
                    p[c >> 1] = f32_to_bf16(h0) | (f32_to_bf16(h1) << 16);
                }
                *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(C) + (size_t)(r0 + row) * N +
                                           col) = make_uint4(p[0], p[1], p[2], p[3]);
            } else {
                float *dst = static_cast<float *>(C) + (size_t)(r0 + row) * N + col;
                *reinterpret_cast<float4 *>(dst) =
                    make_float4(acc[0][i][0][j], acc[0][i][1][j], acc[0][i][2][j], acc[0][i][3][j]);
                *reinterpret_cast<float4 *>(dst + 4) =
                    make_float4(acc[0][i][4][j], acc[0][i][5][j], acc[0][i][6][j], acc[0][i][7][j]);
            }
        }
    }
}

}  // namespace

hipError_t launch_gateup_bf16(const moe_shape_t &s, const uint16_t *xp, const int32_t *counts,
                              const int32_t *offsets, const uint16_t *w1, const uint16_t *w3,
                              uint16_t *h, hipStream_t stream) {
    const int d = s.d_model, f = s.d_ff, E = s.n_experts, rows = 2 * s.T;
    if (s.T <= 16) {
        hipLaunchKernelGGL((decode_gemm_kernel<1, 2>), dim3((f + DCOLS - 1) / DCOLS, E),
                           dim3(DWAVES * 64), 0, stream, xp, w1, w3, h, counts, offsets, d, f,
                           rows);
    } else if (s.T <= kDecodeMaxT) {
        hipLaunchKernelGGL((decode_gemm_kernel<2, 2>), dim3((f + DCOLS - 1) / DCOLS, E),
                           dim3(DWAVES * 64), 0, stream, xp, w1, w3, h, counts, offsets, d, f,
                           rows);
    } else {
        const int m_tiles = (rows + PBM - 1) / PBM + E;
        hipLaunchKernelGGL(prefill_gemm_kernel<2>, dim3((f + PBN / 2 - 1) / (PBN / 2), m_tiles),
                           dim3(256), 0, stream, xp, w1, w3, h, counts, offsets, E, d, f, rows);
    }
    return hipGetLastError();
}

hipError_t launch_down_bf16(const moe_shape_t &s, const uint16_t *h, const int32_t *counts,
                            const int32_t *offsets, const uint16_t *w2, float *o,
                            hipStream_t stream) {
    const int d = s.d_model, f = s.d_ff, E = s.n_experts, rows = 2 * s.T;
    if (s.T <= 16) {
        hipLaunchKernelGGL((decode_gemm_kernel<1, 1>), dim3((d + DCOLS - 1) / DCOLS, E),
                           dim3(DWAVES * 64), 0, stream, h, w2, nullptr, o, counts, offsets, f,
                           d, rows);
    } else if (s.T <= kDecodeMaxT) {
        hipLaunchKernelGGL((decode_gemm_kernel<2, 1>), dim3((d + DCOLS - 1) / DCOLS, E),
                           dim3(DWAVES * 64), 0, stream, h, w2, nullptr, o, counts, offsets, f,
                           d, rows);
    } else {
        const int m_tiles = (rows + PBM - 1) / PBM + E;
        hipLaunchKernelGGL(prefill_gemm_kernel<1>, dim3((d + PBN - 1) / PBN, m_tiles),
                           dim3(256), 0, stream, h, w2, nullptr, o, counts, offsets, E, f, d,
                           rows);
    }
    return hipGetLastError();
}

}  // namespace moe
