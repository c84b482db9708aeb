// Weight-only int8 expert weights for the decode path.  The KerasFormers
// Mixtral page's loading example offers int8 weight quantization with
// low-memory loading for this model but gives no scheme, so the
// plainest is used: symmetric int8 with one fp32 scale per output channel
// of each expert matrix, W[j, n] ~ s[n] * q[j, n].
//
// Decode is bound by streaming the selected experts' weights (section 05 of
// "Mixtral 8x7B -- The Evolving Transformer": only the chosen experts run),
// so int8 codes halve the bytes of the step.  The activations stay bf16:
// each lane turns its codes into bf16 (exact, |q| <= 127) and the product
// runs on the bf16 matrix cores with fp32 accumulation; the scale of each
// output column multiplies the finished sum.
//
//  * quantize_int8_kernel: s[n] = max_j |W[j, n]| / 127 and
//    q = rint(W / s) clamped to [-127, 127], in fp32 (s = 0, q = 0 for a
//    zero column).  One pass for the maxima, one for the codes.  Codes are
//    stored with row pairs interleaved in 8-column groups (code_offset), so
//    that a 16-byte load gives the 8 columns of two rows.
//  * decode_w8_kernel: a workgroup streams a 256-column slab of one
//    expert's codes (256-byte row segments, read once, non-temporal) over
//    its K range.  Eight wavefronts: two column halves of 128 times four K
//    parts, whose partial sums meet in a fixed LDS tree.  Gate/up fuses
//    the scales and silu(g) * u and writes h in bf16; down writes fp32
//    partial sums of one K slice each (the combine adds the slices in
//    order before it weights the slots).
//  * Filling the last round (gate/up): one workgroup runs per CU at a
//    time, so E * ceil(f / 256) slabs make whole rounds plus a part-filled
//    one (8x7B: 448 slabs on 256 CUs, 1.75 rounds, run as 2).  The slabs
//    past the whole rounds are cut so that the pieces fill rounds of half
//    and of a quarter of a slab's time: column halves (128 columns, the
//    whole K, all eight wavefronts along K) and quarters (a column half
//    over one K half, whose fp32 sums a small kernel adds).
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int W8_WAVES = 8;                     // 2 column halves x 4 K parts
constexpr int W8_HALF = 128;                    // columns per wavefront
constexpr int W8_HALVES = 2;                    // column halves per workgroup
constexpr int W8_COLS = W8_HALVES * W8_HALF;    // weight columns per workgroup
constexpr int W8_KPARTS = W8_WAVES / W8_HALVES; // wavefronts along K per column half

// Code `c` (0..7) of an 8-code row segment, as an fp32 value.
__device__ __forceinline__ float code_f32(uint2 r, int c) {
    const uint32_t w = c < 4 ? r.x : r.y;
    return (float)(int)(int8_t)(w >> (8 * (c & 3)));
}

// Two fp32 values that bf16 holds exactly, packed as bf16 (lo in the low
// half); gfx950 converts the pair in one instruction.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_exact_bf16(float lo, float hi) {
    const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// r[i] holds row i of an 8 x 8 block of codes (8 columns, one byte each).
// Returns column c as the MFMA B operand: 8 bf16 along K, row 0 lowest.
__device__ __forceinline__ bf16x8_t column_operand(const uint2 (&r)[8], int c) {
    uint4 v;
    v.x = pack_exact_bf16(code_f32(r[0], c), code_f32(r[1], c));
    v.y = pack_exact_bf16(code_f32(r[2], c), code_f32(r[3], c));
    v.z = pack_exact_bf16(code_f32(r[4], c), code_f32(r[5], c));
    v.w = pack_exact_bf16(code_f32(r[6], c), code_f32(r[7], c));
    return __builtin_bit_cast(bf16x8_t, v);
}

// 16-byte load with the non-temporal hint: each code is read exactly once.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream16(const int8_t *p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}

template <typename T>
__device__ __forceinline__ void load4(const T *p, float (&v)[4]);
template <>
__device__ __forceinline__ void load4<float>(const float *p, float (&v)[4]) {
    const float4 a = *reinterpret_cast<const float4 *>(p);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
}
template <>
__device__ __forceinline__ void load4<uint16_t>(const uint16_t *p, float (&v)[4]) {
    const uint2 a = *reinterpret_cast<const uint2 *>(p);
    v[0] = bf16_to_f32(a.x & 0xffffu); v[1] = bf16_to_f32(a.x >> 16);
    v[2] = bf16_to_f32(a.y & 0xffffu); v[3] = bf16_to_f32(a.y >> 16);
}

// Byte offset of code (j, n) inside a K x N matrix: [K/2][N/8][2][8].
__device__ __forceinline__ size_t code_offset(int j, int n, int N) {
    return ((size_t)(j >> 1) * (N >> 3) + (n >> 3)) * 16 + (j & 1) * 8 + (n & 7);
}

// grid (ceil(N / 256), n_mat), 256 threads: thread (kp, lane) owns columns
// 4*lane .. 4*lane+3 of the workgroup's 256 and the K quarter kp.  The
// column maxima of the four quarters meet in LDS (a maximum is exact in
// any order).
template <typename T>
__global__ __launch_bounds__(256) void quantize_int8_kernel(const T *__restrict__ W, int K,
                                                            int N, int8_t *__restrict__ Q,
                                                            float *__restrict__ S) {
    __shared__ float amax[4][256];
    const int lane = threadIdx.x & 63, kp = threadIdx.x >> 6;
    const int e = blockIdx.y;
    const int col = blockIdx.x * 256 + lane * 4;
    const bool ok = col < N;   // N % 4 == 0: the four columns are all in or all out
    const size_t base = (size_t)e * K * N + (ok ? col : 0);
    const int j0 = (int)((int64_t)K * kp / 4), j1 = (int)((int64_t)K * (kp + 1) / 4);
    float a[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (ok)
        for (int j = j0; j < j1; ++j) {
            float v[4];
            load4<T>(W + base + (size_t)j * N, v);
#pragma unroll
            for (int c = 0; c < 4; ++c) a[c] = fmaxf(a[c], fabsf(v[c]));
        }
#pragma unroll
    for (int c = 0; c < 4; ++c) amax[kp][lane * 4 + c] = a[c];
    __syncthreads();
    float s[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int i = lane * 4 + c;
        s[c] = fmaxf(fmaxf(amax[0][i], amax[1][i]), fmaxf(amax[2][i], amax[3][i])) / 127.0f;
    }
    if (!ok) return;
    if (kp == 0)
        *reinterpret_cast<float4 *>(S + (size_t)e * N + col) = make_float4(s[0], s[1], s[2], s[3]);
    for (int j = j0; j < j1; ++j) {
        float v[4];
        load4<T>(W + base + (size_t)j * N, v);
        uint32_t packed = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            int code = 0;
            if (s[c] > 0.0f) code = (int)fminf(fmaxf(rintf(v[c] / s[c]), -127.0f), 127.0f);
            packed |= (uint32_t)(code & 0xff) << (8 * c);
        }
        // columns col .. col + 3 of row j: 4 bytes inside one 8-column group
        *reinterpret_cast<uint32_t *>(Q + (size_t)e * K * N + code_offset(j, col, N)) = packed;
    }
}

// C[r, n] for the rows r of expert e = blockIdx.y (at most 16 * MB of
// them), columns n of slab blockIdx.x, K slice blockIdx.z of gridDim.z:
//   NMAT = 2: C = bf16(silu(S0 * (A Q0[e])) * (S1 * (A Q1[e])))   (h)
//   NMAT = 1: C + z * part_stride = fp32(S0 * (A Q0[e]) over slice z) (o)
// With src not NULL, grouped row r is row src[r] of A.
//
// Wavefront w covers column half w % 2 (128 columns) and K part w / 2.
// Lane l loads 8 columns (8 * (l % 16) ..) of 8 rows (8 * (l / 16) ..) of
// each 32-row step, as four 16-byte loads of two rows each (the codes'
// row-pair layout); 16 lanes read 256 contiguous bytes.  A lane's 8 columns give 8 MFMA B operands; block c of
// the accumulators holds weight columns 8 * (l % 16) + c.  (Measured: one
// wavefront per SIMD streaming whole 256-byte segments hides less latency,
// and 128-column workgroups reading 128-byte segments stream slower.)
// RANK: counts, offsets and src come from rk.idx, ranked by the first
// wavefront of every workgroup (DecodeRank).
//
// TAIL (gate/up): a 1-D grid of n_full whole slabs (unit u = e * nb_cols +
// slab), then 2 * n_half column halves of the next n_half units, then
// 4 * n_quarter quarters of the last n_quarter units.  Workgroup j of the
// quarters takes column-half slot j / 2 (unit n_full + n_half + j / 4,
// half (j / 2) % 2) and K half j % 2, and stores its scaled fp32 sums
// (s1 * x Q1, s3 * x Q3) to w8_tail_slot(j / 2, j % 2, m) of part for
// w8_tail_finish_kernel.  A column-half workgroup runs its eight
// wavefronts along K ((k0 + k4) + (k2 + k6)) + ((k1 + k5) + (k3 + k7)).
constexpr int W8_TAIL_ROWS = 32;   // rows of a part slot (an expert's rows at decode sizes)
__device__ __forceinline__ size_t w8_tail_slot(int j, int kh, int m) {
    return ((size_t)(j * 2 + kh) * 2 + m) * W8_TAIL_ROWS * W8_HALF;
}
template <int MB, int NMAT, bool RANK = false, bool TAIL = false>
__global__ __launch_bounds__(W8_WAVES * 64) void decode_w8_kernel(
    const uint16_t *__restrict__ A, const int8_t *__restrict__ Q0, const float *__restrict__ S0,
    const int8_t *__restrict__ Q1, const float *__restrict__ S1, void *__restrict__ C,
    const int32_t *__restrict__ counts, const int32_t *__restrict__ offsets, int K, int N,
    int a_rows, const int32_t *__restrict__ src, size_t part_stride,
    DecodeRank rk = DecodeRank{}, int n_exp = 0, float *__restrict__ part = nullptr,
    int n_full = 0, int n_half = 0, int nb_cols = 0, int early = 0) {
    static_assert(!TAIL || (NMAT == 2 && MB * 16 <= W8_TAIL_ROWS), "gate/up, one slot per expert");
    int e = blockIdx.y, slab = blockIdx.x;
    int half_sel = -1;   // column-half and quarter workgroups: their column half
    int kh = -1;         // quarter workgroups: their K half
    int slot = 0;        // quarter workgroups: their part slot
    if constexpr (TAIL) {
        int unit = blockIdx.x;
        if (unit >= n_full) {
            int j = unit - n_full;
            if (j < 2 * n_half) {
                unit = n_full + (j >> 1);
                half_sel = j & 1;
            } else {
                j -= 2 * n_half;
                slot = j >> 1;
                kh = j & 1;
                unit = n_full + n_half + (slot >> 1);
                half_sel = slot & 1;
            }
        }
        e = unit / nb_cols;
        slab = unit - e * nb_cols;
    }
    // The wavefront index is uniform: read it into a scalar so that the K
    // loop bounds are scalar and the loop is not taken for a divergent one.
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const bool narrow = TAIL && half_sel >= 0;   // one column half, eight K parts
    const int half = narrow ? half_sel : wave % W8_HALVES;
    const int kp = narrow ? wave : wave / W8_HALVES;
    const int kparts = narrow ? W8_WAVES : W8_KPARTS;
    const int kg = lane >> 4, nb = lane & 15;
    const int col = slab * W8_COLS + half * W8_HALF + nb * 8;
    const bool col_ok = col < N;   // N % 8 == 0: the 8 columns are all in or all out

    // Codes are addressed as a uniform base (this expert's matrix) plus a
    // 32-bit lane offset (an expert matrix is far below 4 GiB).
    const int8_t *Qb[NMAT];
    Qb[0] = Q0 + (size_t)e * K * N;
    if (NMAT == 2) Qb[NMAT - 1] = Q1 + (size_t)e * K * N;
    const uint32_t lane_col = (uint32_t)(col_ok ? col : 0);

    // 32-row K steps: this workgroup's slice, then this wavefront's quarter.
    const int nks = (K + 31) >> 5;
    int z0 = (int)((int64_t)nks * blockIdx.z / gridDim.z);
    int z1 = (int)((int64_t)nks * (blockIdx.z + 1) / gridDim.z);
    if (TAIL && kh >= 0) {
        z0 = nks * kh / 2;
        z1 = nks * (kh + 1) / 2;
    }
    const int ks0 = z0 + (z1 - z0) * kp / kparts;
    const int ks1 = z0 + (z1 - z0) * (kp + 1) / kparts;

    // NBUF register buffers: the loads of the next NBUF - 1 steps are in
    // flight while a step computes (down, one matrix: three buffers, so
    // that a wavefront keeps as many bytes in flight as gate/up's two
    // matrices do with two).  A step's loads are unconditional, from
    // clamped addresses, so they issue back to back: rows past K
    // (K % 8 == 0, so a lane's 8 rows are all in or all out) meet
    // activations set to zero; lanes past N are not stored.
    constexpr int NBUF = NMAT == 1 ? 3 : 2;
    uint2 rb[NBUF][NMAT][8];   // row i of the lane's 8 x 8 block
    uint4 ar[NBUF][MB];
    uint32_t keep[NBUF];   // all ones, or zero for rows past K (applied at use)
    auto load_b = [&](int b, int ks) __attribute__((always_inline)) {
        const int k = ks * 32 + kg * 8;
        const int kr = min(k, K - 8);
        // rows kr + 2p, kr + 2p + 1 of the lane's 8 columns: 16 bytes at
        // (kr / 2 + p) * 2N + 2 * col (kr and col are multiples of 8)
        const uint32_t off = (uint32_t)kr * (uint32_t)N + 2u * lane_col;
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int pr = 0; pr < 4; ++pr) {
                const uint4 v = load_stream16(Qb[m] + off + (uint32_t)(2 * pr) * (uint32_t)N);
                rb[b][m][2 * pr] = make_uint2(v.x, v.y);
                rb[b][m][2 * pr + 1] = make_uint2(v.z, v.w);
            }
        keep[b] = k < K ? 0xffffffffu : 0u;
    };
    // early: the codes of this wavefront's first NBUF - 1 steps are
    // requested before the routing is read (they do not depend on it), so
    // that the routing's latency overlaps theirs; the launcher sets it only
    // when nearly every expert holds rows.
    const bool pre = early && ks0 < ks1;
    if (pre) {
        load_b(0, ks0);
        if (NBUF == 3 && ks0 + 1 < ks1) load_b(1, ks0 + 1);
    }

    __shared__ int32_t s_counts[RANK ? kMaxExperts : 1], s_offsets[RANK ? kMaxExperts + 1 : 1];
    __shared__ int32_t s_src[RANK ? kDecodeMaxT * kMaxTopK : 1];
    if constexpr (RANK) {
        if (wave == 0)
            decode_rank_wave(rk, n_exp, lane, s_counts, s_offsets, s_src,
                             blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0);
        __syncthreads();
        counts = s_counts;
        offsets = s_offsets;
        src = s_src;
    }
    const int Me = counts[e];
    if (Me == 0) return;  // an expert no token chose: the rest of its codes are never read
    const int r0 = offsets[e];
    const int nmb = min(MB, (Me + 15) >> 4);
    const uint16_t *Arow[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) {
        const int r = min(r0 + i * 16 + (lane & 15), a_rows - 1);
        Arow[i] = A + (size_t)(src ? src[r] : r) * K;
    }

    f32x4_t acc[NMAT][MB][8];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[m][i][c] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    if (ks0 < ks1) {
        auto load_a = [&](int b, int ks) __attribute__((always_inline)) {
            const int kr = min(ks * 32 + kg * 8, K - 8);
#pragma unroll
            for (int i = 0; i < MB; ++i) ar[b][i] = *reinterpret_cast<const uint4 *>(Arow[i] + kr);
        };
        auto load_step = [&](int b, int ks) __attribute__((always_inline)) {
            load_b(b, ks);
            load_a(b, ks);
        };
        auto compute_step = [&](int b) __attribute__((always_inline)) {
            bf16x8_t aop[MB];
#pragma unroll
            for (int i = 0; i < MB; ++i) {
                const uint4 a = ar[b][i];
                aop[i] = __builtin_bit_cast(bf16x8_t, make_uint4(a.x & keep[b], a.y & keep[b],
                                                                 a.z & keep[b], a.w & keep[b]));
            }
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const bf16x8_t bop = column_operand(rb[b][m], c);
#pragma unroll
                    for (int i = 0; i < MB; ++i) {
                        if (i >= nmb) continue;
                        acc[m][i][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop[i], bop,
                                                                               acc[m][i][c], 0, 0, 0);
                    }
                }
        };
        // Step s uses buffer (s - ks0) % NBUF; before it computes, the loads
        // of step s + NBUF - 1 go into the buffer step s - 1 has left.
        auto step = [&](auto b_c, int s) __attribute__((always_inline)) {
            constexpr int b = decltype(b_c)::value;
            if (s < ks1) {
                if (s + NBUF - 1 < ks1) load_step((b + NBUF - 1) % NBUF, s + NBUF - 1);
                compute_step(b);
            }
        };
        if (pre) {
            load_a(0, ks0);
            if (NBUF == 3 && ks0 + 1 < ks1) load_a(1, ks0 + 1);
        } else {
            load_step(0, ks0);
            if (NBUF == 3 && ks0 + 1 < ks1) load_step(1, ks0 + 1);
        }
        for (int ks = ks0; ks < ks1; ks += NBUF) {
            step(std::integral_constant<int, 0>{}, ks);
            step(std::integral_constant<int, 1>{}, ks + 1);
            if constexpr (NBUF == 3) step(std::integral_constant<int, 2>{}, ks + 2);
        }
    }

    // Fixed-order tree over the K parts of each column half: four parts,
    // (k0 + k2) + (k1 + k3); a column-half workgroup's eight, as above.
    constexpr int SLOTS = W8_KPARTS / 2;
    __shared__ f32x4_t red[W8_HALVES * SLOTS][NMAT * 8][64];
    const int rbase = narrow ? 0 : half * SLOTS;
#pragma unroll
    for (int i = 0; i < MB; ++i) {
        if (i >= nmb) break;
        for (int hs = kparts / 2; hs >= 1; hs >>= 1) {
            if (kp >= hs && kp < 2 * hs)
#pragma unroll
                for (int m = 0; m < NMAT; ++m)
#pragma unroll
                    for (int c = 0; c < 8; ++c)
                        red[rbase + kp - hs][m * 8 + c][lane] = acc[m][i][c];
            __syncthreads();
            if (kp < hs)
#pragma unroll
                for (int m = 0; m < NMAT; ++m)
#pragma unroll
                    for (int c = 0; c < 8; ++c) acc[m][i][c] += red[rbase + kp][m * 8 + c][lane];
            __syncthreads();
        }
        if (kp != 0 || !col_ok) continue;
        float sc[NMAT][8];
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
            const float4 *sp =
                reinterpret_cast<const float4 *>((m == 0 ? S0 : S1) + (size_t)e * N + col);
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const float4 v = sp[q];
                sc[m][4 * q] = v.x; sc[m][4 * q + 1] = v.y;
                sc[m][4 * q + 2] = v.z; sc[m][4 * q + 3] = v.w;
            }
        }
        // 16x16 accumulator layout: value j of lane l is row 4*(l/16) + j,
        // column l%16 of the block; block c holds weight columns 8*(l%16) + c.
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = i * 16 + 4 * kg + j;
            if (row >= Me) continue;
            if (TAIL && kh >= 0) {
#pragma unroll
                for (int m = 0; m < NMAT; ++m) {
                    float *dst = part + w8_tail_slot(slot, kh, m) + (size_t)row * W8_HALF + nb * 8;
#pragma unroll
                    for (int q = 0; q < 2; ++q)
                        reinterpret_cast<float4 *>(dst)[q] =
                            make_float4(sc[m][4 * q] * acc[m][i][4 * q][j],
                                        sc[m][4 * q + 1] * acc[m][i][4 * q + 1][j],
                                        sc[m][4 * q + 2] * acc[m][i][4 * q + 2][j],
                                        sc[m][4 * q + 3] * acc[m][i][4 * q + 3][j]);
                }
            } else if (NMAT == 2) {
                uint32_t p[4];
#pragma unroll
                for (int c = 0; c < 8; c += 2) {
                    const float g0 = sc[0][c] * acc[0][i][c][j];
                    const float g1 = sc[0][c + 1] * acc[0][i][c + 1][j];
                    const float u0 = sc[NMAT - 1][c] * acc[NMAT - 1][i][c][j];
                    const float u1 = sc[NMAT - 1][c + 1] * acc[NMAT - 1][i][c + 1][j];
                    p[c >> 1] = f32_to_bf16(silu_f32(g0) * u0) |
                                (f32_to_bf16(silu_f32(g1) * u1) << 16);
                }
                *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(C) + (size_t)(r0 + row) * N +
                                           col) = make_uint4(p[0], p[1], p[2], p[3]);
            } else {
                float4 *dst = reinterpret_cast<float4 *>(static_cast<float *>(C) +
                                                         blockIdx.z * part_stride +
                                                         (size_t)(r0 + row) * N + col);
#pragma unroll
                for (int q = 0; q < 2; ++q)
                    dst[q] = make_float4(sc[0][4 * q] * acc[0][i][4 * q][j],
                                         sc[0][4 * q + 1] * acc[0][i][4 * q + 1][j],
                                         sc[0][4 * q + 2] * acc[0][i][4 * q + 2][j],
                                         sc[0][4 * q + 3] * acc[0][i][4 * q + 3][j]);
            }
        }
    }
}

// The quarters of a TAIL launch: workgroup j adds the two K halves of part
// slot j (half 0 first) and writes h = bf16(silu(g) * u) for column half
// j % 2 of unit first_unit + j / 2.
__global__ __launch_bounds__(256) void w8_tail_finish_kernel(
    const float *__restrict__ part, const int32_t *__restrict__ counts,
    const int32_t *__restrict__ offsets, int first_unit, int nb_cols, int N,
    uint16_t *__restrict__ h) {
    const int j = blockIdx.x, unit = first_unit + (j >> 1);
    const int e = unit / nb_cols, slab = unit - e * nb_cols;
    const int Me = counts[e], r0 = offsets[e];
    const int col0 = slab * W8_COLS + (j & 1) * W8_HALF;
    // four consecutive columns per thread (N % 8 == 0: all in or all out)
    const float4 *g0 = reinterpret_cast<const float4 *>(part + w8_tail_slot(j, 0, 0));
    const float4 *g1 = reinterpret_cast<const float4 *>(part + w8_tail_slot(j, 1, 0));
    const float4 *u0 = reinterpret_cast<const float4 *>(part + w8_tail_slot(j, 0, 1));
    const float4 *u1 = reinterpret_cast<const float4 *>(part + w8_tail_slot(j, 1, 1));
    for (int i = threadIdx.x; i < Me * (W8_HALF / 4); i += 256) {
        const int row = i / (W8_HALF / 4), col = col0 + 4 * (i % (W8_HALF / 4));
        if (col >= N) continue;
        const float4 a = g0[i], b = g1[i], c = u0[i], d = u1[i];
        const float g[4] = {a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w};
        const float u[4] = {c.x + d.x, c.y + d.y, c.z + d.z, c.w + d.w};
        uint32_t hv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) hv[q] = f32_to_bf16(silu_f32(g[q]) * u[q]);
        *reinterpret_cast<uint2 *>(h + (size_t)(r0 + row) * N + col) =
            make_uint2(hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16));
    }
}

// How a gate/up launch of `units` slabs fills its last round (see TAIL):
// false when it runs every slab whole.  With r = the slabs past the whole
// rounds over the CU count: r <= 1/4 runs quarters, r <= 1/2 column
// halves, r <= 3/4 one round of column halves and one of quarters.
struct W8Tail {
    int n_full, n_half, n_quarter;
};
bool w8_tail_plan(int units, W8Tail &p) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0 || units <= cus)
        return false;
    const int rem = units % cus;
    if (rem == 0) return false;
    p.n_full = units - rem;
    if (4 * rem <= cus) {
        p.n_half = 0;
        p.n_quarter = rem;
    } else if (2 * rem <= cus) {
        p.n_half = rem;
        p.n_quarter = 0;
    } else if (4 * rem <= 3 * cus) {
        p.n_half = cus / 2;
        p.n_quarter = rem - cus / 2;
    } else {
        return false;
    }
    // two part slots per quarter unit, each 2 K halves x 2 matrices x
    // 32 rows x 128 columns of fp32: the decode partial-sum region
    return 2 * p.n_quarter <= kDecodeTailMaxUnits;
}

}  // namespace

hipError_t launch_quantize_int8(int n_mat, int K, int N, int dtype, const void *w, int8_t *q,
                                float *scale, hipStream_t stream) {
    const dim3 grid((N + 255) / 256, n_mat);
    if (dtype == MOE_BF16)
        hipLaunchKernelGGL(quantize_int8_kernel<uint16_t>, grid, dim3(256), 0, stream,
                           static_cast<const uint16_t *>(w), K, N, q, scale);
    else
        hipLaunchKernelGGL(quantize_int8_kernel<float>, grid, dim3(256), 0, stream,
                           static_cast<const float *>(w), K, N, q, scale);
    return hipGetLastError();
}

namespace {
template <int MB, bool RANK>
hipError_t launch_gateup_w8_tail(const moe_shape_t &s, const uint16_t *xp,
                                 const int32_t *counts, const int32_t *offsets, const int8_t *q1,
                                 const float *s1, const int8_t *q3, const float *s3, uint16_t *h,
                                 hipStream_t stream, const int32_t *src, const DecodeRank &rk,
                                 float *part, const W8Tail &p, int nb_cols) {
    const int d = s.d_model, f = s.d_ff, E = s.n_experts, rows = routed_rows(s);
    const int grid = p.n_full + 2 * p.n_half + 4 * p.n_quarter;
    hipLaunchKernelGGL((decode_w8_kernel<MB, 2, RANK, true>), dim3(grid), dim3(W8_WAVES * 64), 0,
                       stream, xp, q1, s1, q3, s3, h, counts, offsets, d, f, rows, src, (size_t)0,
                       rk, E, part, p.n_full, p.n_half, nb_cols, decode_early_weights(rows, E));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.n_quarter == 0) return e;
    hipLaunchKernelGGL(w8_tail_finish_kernel, dim3(2 * p.n_quarter), dim3(256), 0, stream, part,
                       counts, offsets, p.n_full + p.n_half, nb_cols, f, h);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_gateup_w8(const moe_shape_t &s, const uint16_t *xp, const int32_t *counts,
                            const int32_t *offsets, const int8_t *q1, const float *s1,
                            const int8_t *q3, const float *s3, uint16_t *h, hipStream_t stream,
                            const int32_t *src, const DecodeRank *rank, float *part) {
    const int d = s.d_model, f = s.d_ff, E = s.n_experts, rows = routed_rows(s);
    const dim3 grid((f + W8_COLS - 1) / W8_COLS, E, 1), block(W8_WAVES * 64);
    if (s.T > kDecodeMaxT || (rank && (!src || E > kMaxExperts)))
        return hipErrorInvalidValue;
    const DecodeRank rk = rank ? *rank : DecodeRank{};
    const int early = decode_early_weights(rows, E);
    W8Tail tp{};
    if (part && w8_tail_plan((int)grid.x * E, tp)) {
        if (s.T <= 16)
            return rank ? launch_gateup_w8_tail<1, true>(s, xp, counts, offsets, q1, s1, q3, s3, h,
                                                         stream, src, rk, part, tp, grid.x)
                        : launch_gateup_w8_tail<1, false>(s, xp, counts, offsets, q1, s1, q3, s3,
                                                          h, stream, src, rk, part, tp, grid.x);
        return rank ? launch_gateup_w8_tail<2, true>(s, xp, counts, offsets, q1, s1, q3, s3, h,
                                                     stream, src, rk, part, tp, grid.x)
                    : launch_gateup_w8_tail<2, false>(s, xp, counts, offsets, q1, s1, q3, s3, h,
                                                      stream, src, rk, part, tp, grid.x);
    }
    if (s.T <= 16 && rank)
        hipLaunchKernelGGL((decode_w8_kernel<1, 2, true>), grid, block, 0, stream, xp, q1, s1, q3,
                           s3, h, counts, offsets, d, f, rows, src, (size_t)0, rk, E,
                           nullptr, 0, 0, 0, early);
    else if (s.T <= 16)
        hipLaunchKernelGGL((decode_w8_kernel<1, 2>), grid, block, 0, stream, xp, q1, s1, q3, s3,
                           h, counts, offsets, d, f, rows, src, (size_t)0, rk, E,
                           nullptr, 0, 0, 0, early);
    else if (rank)
        hipLaunchKernelGGL((decode_w8_kernel<2, 2, true>), grid, block, 0, stream, xp, q1, s1, q3,
                           s3, h, counts, offsets, d, f, rows, src, (size_t)0, rk, E,
                           nullptr, 0, 0, 0, early);
    else
        hipLaunchKernelGGL((decode_w8_kernel<2, 2>), grid, block, 0, stream, xp, q1, s1, q3, s3,
                           h, counts, offsets, d, f, rows, src, (size_t)0, rk, E,
                           nullptr, 0, 0, 0, early);
    return hipGetLastError();
}

hipError_t launch_down_w8(const moe_shape_t &s, const uint16_t *h, const int32_t *counts,
                          const int32_t *offsets, const int8_t *q2, const float *s2, float *o,
                          int parts, hipStream_t stream) {
    const int d = s.d_model, f = s.d_ff, E = s.n_experts, rows = routed_rows(s);
    const size_t part_stride = (size_t)rows * d;
    const dim3 grid((d + W8_COLS - 1) / W8_COLS, E, parts), block(W8_WAVES * 64);
    if (s.T <= 16)
        hipLaunchKernelGGL((decode_w8_kernel<1, 1>), grid, block, 0, stream, h, q2, s2, nullptr,
                           nullptr, o, counts, offsets, f, d, rows, nullptr, part_stride,
                           DecodeRank{}, 0, nullptr, 0, 0, 0, decode_early_weights(rows, E));
    else if (s.T <= kDecodeMaxT)
        hipLaunchKernelGGL((decode_w8_kernel<2, 1>), grid, block, 0, stream, h, q2, s2, nullptr,
                           nullptr, o, counts, offsets, f, d, rows, nullptr, part_stride,
                           DecodeRank{}, 0, nullptr, 0, 0, 0, decode_early_weights(rows, E));
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace moe
