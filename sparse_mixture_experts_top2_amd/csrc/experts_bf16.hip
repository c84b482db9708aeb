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
//  * prefill (many rows per expert): 256 x 256 output tiles staged through
//    double-buffered LDS, v_mfma_f32_32x32x16_bf16, tiles ordered so that
//    the workgroups resident on one XCD share weight tiles in its L2.
//    MFMA-bound when an expert has more rows than the ridge point.
//  * decode (at most 32 rows in total per expert): each workgroup streams
//    one 128-column slab of an expert's weights over the whole K range
//    exactly once, with v_mfma_f32_16x16x32_bf16 covering the few rows.
//    Eight wavefronts split K; their partial sums are added in LDS in a
//    fixed tree order.  HBM-bound: only the selected experts' weights are
//    read, each byte once.
// Both fuse silu(g) * u into the gate/up epilogue and round h to bf16.
#include <algorithm>

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

// 16-byte load with the non-temporal hint, for data read exactly once (the
// decode path's weights): it streams past the caches instead of evicting
// the activations that every workgroup re-reads.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream16(const uint16_t *p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// 16-byte store with the non-temporal hint: output written once and not
// re-read by this kernel, kept from displacing the operand tiles that the
// workgroups on this XCD share through L2.
__device__ __forceinline__ void store_stream16(uint16_t *p, uint4 v) {
    __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_t *>(p));
}

// ---------------------------------------------------------------------------
// Prefill: LDS-tiled grouped GEMM.
//   NMAT = 2: C = bf16(silu(A B0[e]) * (A B1[e]))   (gate/up, C = h)
//   NMAT = 1: C = fp32(A B0[e])                     (down,    C = o)
//
// Workgroup tile 256 rows x 256 columns (for gate/up: 128 gate + the same
// 128 up columns, so the epilogue pairs them in registers), K step 64.
// WM x WN wavefronts; each owns a (256/WM) x (256/WN) sub-tile of 32x32
// MFMA blocks.  Both operands are staged in LDS, double-buffered: the
// global loads of step k+1 are in flight while step k computes, and one
// barrier per step separates the two buffers.  The weight operand is
// transposed in registers on its way into LDS (K contiguous per column).

constexpr int PBM = 256, PBN = 256, PBK = 64;
constexpr int PLD = PBK + 8;  // LDS row pitch in bf16 (144 bytes): consecutive rows start
                              // 16 bytes apart modulo 128, so 8-lane groups of 16-byte
                              // reads and writes fall on distinct banks
constexpr int PGM = 4;                 // row tiles per scheduling group (see prefill_tile)
constexpr int PWM = 2, PWN = 4;        // wavefront rows x columns

// Work decomposition shared by the prefill kernels.  Row tiles of PBM rows
// are numbered expert after expert; the flat tile list orders them in
// groups of PGM row tiles, with all column tiles of a group before the
// next group (row tile fastest inside a group).  Workgroup b runs on XCD
// b % 8 (round-robin dispatch); each XCD takes a contiguous eighth of the
// flat list, so the ~32 workgroups resident on one XCD share the same few
// weight column tiles and activation row tiles through that XCD's L2.
__device__ __forceinline__ bool prefill_tile(const int32_t *counts, const int32_t *offsets,
                                             int E, int n_tiles, int &e, int &row0,
                                             int &row_end, int &nt) {
    int mt_total = 0;
    for (int i = 0; i < E; ++i) mt_total += (counts[i] + PBM - 1) / PBM;
    const int total = mt_total * n_tiles;
    const int per_xcd = (total + 7) >> 3;
    const int li = blockIdx.x >> 3;
    if (li >= per_xcd) return false;
    const int L = (blockIdx.x & 7) * per_xcd + li;
    if (L >= total) return false;
    const int group = L / (PGM * n_tiles);
    const int first = group * PGM;
    const int gm = min(PGM, mt_total - first);
    const int within = L - group * PGM * n_tiles;
    const int mt = first + within % gm;
    nt = within / gm;
    return find_row_tile(counts, offsets, E, PBM, mt, e, row0, row_end);
}

template <int NMAT>
__global__ __launch_bounds__(PWM * PWN * 64, 1) void prefill_gemm_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B0,
    const uint16_t *__restrict__ B1, void *__restrict__ C, const int32_t *__restrict__ counts,
    const int32_t *__restrict__ offsets, int E, int K, int N, int a_rows) {
    constexpr int NT = PWM * PWN * 64;            // threads
    constexpr int TM = PBM / PWM, TN = PBN / PWN;  // wave sub-tile
    constexpr int MB = TM / 32, NB = TN / 32;      // 32x32 blocks per wave
    constexpr int BNM = PBN / NMAT;                // columns of each matrix per tile
    constexpr int AV = PBM * PBK / 8 / NT;         // 16-byte A vectors per thread
    static_assert(NMAT == 1 || NB % 2 == 0, "gate/up blocks come in pairs");

    const int n_tiles = (N + BNM - 1) / BNM;
    int e, row0, row_end, nt;
    if (!prefill_tile(counts, offsets, E, n_tiles, e, row0, row_end, nt)) return;
    const int n0 = nt * BNM;

    __shared__ __attribute__((aligned(16))) uint16_t smem[2][(PBM + PBN) * PLD];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / PWN, wn = wave % PWN;

    // A: vector v = tid + NT*i covers row v/8, K chunk v%8.  Rows past the
    // end of A are clamped onto its last row (never stored).
    const uint16_t *Arow[AV];
#pragma unroll
    for (int i = 0; i < AV; ++i)
        Arow[i] = A + (size_t)min(row0 + ((tid + NT * i) >> 3), a_rows - 1) * K;
    // B: 256 blocks of 8 K-rows x 8 columns, one per thread of the first 256
    // threads.  kb (K block) is the fastest index so that the 8 lanes that
    // write one LDS row after the transpose hit 8 consecutive 16-byte chunks.
    const bool do_b = tid < 256;
    const int kb = tid & 7, nb = (tid & 255) >> 3;          // nb: 0..31
    const int mat = NMAT == 2 ? nb >> 4 : 0;
    const int bcol = n0 + (NMAT == 2 ? (nb & 15) : nb) * 8;
    const bool bcol_ok = bcol < N;
    const uint16_t *Bp = (mat ? B1 : B0) + (size_t)e * K * N + (bcol_ok ? bcol : 0);

    uint4 ra[AV], rb[8];
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < AV; ++i) {
            const int k = k0 + ((tid + NT * i) & 7) * 8;
            ra[i] = k < K ? *reinterpret_cast<const uint4 *>(Arow[i] + k) : zero4();
        }
        if (do_b)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int k = k0 + kb * 8 + i;
                rb[i] = (k < K && bcol_ok) ? *reinterpret_cast<const uint4 *>(Bp + (size_t)k * N)
                                           : zero4();
            }
    };
    auto lstore = [&](int st) {
        uint16_t *As = smem[st], *Bs = smem[st] + PBM * PLD;
#pragma unroll
        for (int i = 0; i < AV; ++i) {
            const int v = tid + NT * i;
            *reinterpret_cast<uint4 *>(&As[(v >> 3) * PLD + (v & 7) * 8]) = ra[i];
        }
        if (do_b) {
            uint4 tb[8];
            transpose8x8(rb, tb);
#pragma unroll
            for (int c = 0; c < 8; ++c)
                *reinterpret_cast<uint4 *>(&Bs[(nb * 8 + c) * PLD + kb * 8]) = tb[c];
        }
    };
    // LDS row of this wave's column block j: gate/up waves take TN/2 gate
    // columns (LDS rows 0..127) and the same TN/2 up columns (rows 128..255).
    auto brow = [&](int j) {
        if (NMAT == 2) return (j / (NB / 2)) * 128 + wn * (TN / 2) + (j % (NB / 2)) * 32;
        return wn * TN + j * 32;
    };

    f32x16_t acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

    const int nk = (K + PBK - 1) / PBK;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * PBK);
        const uint16_t *As = smem[cur], *Bs = smem[cur] + PBM * PLD;
#pragma unroll
        for (int kk = 0; kk < PBK; kk += 16) {
            const int koff = kk + (lane >> 5) * 8;
            bf16x8_t af[MB], bfr[NB];
#pragma unroll
            for (int i = 0; i < MB; ++i)
                af[i] = as_bf16x8(*reinterpret_cast<const uint4 *>(
                    &As[(wm * TM + i * 32 + (lane & 31)) * PLD + koff]));
#pragma unroll
            for (int j = 0; j < NB; ++j)
                bfr[j] = as_bf16x8(*reinterpret_cast<const uint4 *>(
                    &Bs[(brow(j) + (lane & 31)) * PLD + koff]));
#pragma unroll
            for (int i = 0; i < MB; ++i)
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j],
                                                                         acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) lstore(cur ^ 1);
        __syncthreads();
    }

    // Epilogue.  32x32 accumulator layout: value q of lane l is row
    // 8*(q/4) + 4*(l/32) + q%4, column l%32 of the block.
#pragma unroll
    for (int i = 0; i < MB; ++i) {
#pragma unroll
        for (int j = 0; j < (NMAT == 2 ? NB / 2 : NB); ++j) {
            const int col = n0 + (NMAT == 2 ? wn * (TN / 2) + j * 32 : wn * TN + j * 32) +
                            (lane & 31);
            if (col >= N) continue;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int row =
                    row0 + wm * TM + i * 32 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
                if (row >= row_end) continue;
                if (NMAT == 2) {
                    const float h = silu_f32(acc[i][j][q]) * acc[i][j + NB / 2][q];
                    static_cast<uint16_t *>(C)[(size_t)row * N + col] = (uint16_t)f32_to_bf16(h);
                } else {
                    static_cast<float *>(C)[(size_t)row * N + col] = acc[i][j][q];
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Prefill, direct-to-LDS variant (K % 64 == 0 and N a multiple of the tile's
// columns per matrix, which every Mixtral shape satisfies).  Same tiles and
// schedule as prefill_gemm_kernel, but operands go from global memory
// straight into LDS rings (global_load_lds_dwordx4: no registers, no VALU
// work).  The activation operand A has a 2-deep ring; the weight operand B,
// whose tiles mostly come from HBM rather than L2, has a 3-deep ring, so its
// loads are issued two K steps ahead.  Both rings together fill the 160 KiB
// of LDS.
//
// LDS layouts (16-byte chunks are XOR-swizzled by row so that MFMA operand
// reads from consecutive rows fall on distinct banks):
//   A stage: 256 rows x 64 bf16 (128 B = 8 chunks); chunk c of row r holds
//            K chunk c ^ aswz(r).
//   B stage: 64 K rows x 256 columns (512 B = 32 chunks), the weights'
//            own row-major layout (for gate/up: 128 gate then 128 up
//            columns); chunk c of row r holds column chunk c ^ bswz(r).
// A fragments are plain 16-byte reads.  B fragments use the CDNA4 LDS
// transpose read ds_read_b64_tr_b16: within each 16-lane group, lane 4i+q
// points at 4 consecutive columns of K row i and lane j receives column j
// of those 4 rows, i.e. 4 consecutive K values of one column.  Two such
// reads give the 8 K values a 32x32x16 operand lane holds.

constexpr int DBK = 64;                       // K per stage: every A row segment is
                                              // one full 128-byte line
constexpr int DAS = 2;                        // A ring depth
constexpr int DBS = 3;                        // B ring depth
static_assert(DAS >= 2 && DBS >= 2 && DAS + DBS <= 5, "five 32 KiB slots fit in LDS");
constexpr int DA_BYTES = PBM * DBK * 2;       // 32 KiB
constexpr int DB_BYTES = DBK * PBN * 2;       // 32 KiB
constexpr int DACH = DBK / 8;                 // 16-byte chunks per A row

// A swizzle: any 8 (and 16) consecutive rows reading the same K chunk land
// on distinct 16-byte bank groups.
__device__ __forceinline__ int aswz(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); }
__device__ __forceinline__ int bswz(int r) { return (r & 7) << 2; }

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

// Barrier of the LDS rings.  Each wavefront first waits until at most N of
// its own LDS-DMA loads are outstanding (so its part of the stage about to
// be read has landed) and until its LDS reads have returned (so the stage
// about to be refilled is no longer being read), then all wavefronts meet.
// __syncthreads() is not used here: its release fence waits for every
// outstanding load, which would drain the rings.  The empty asm statements
// keep the compiler from moving memory accesses across the barrier.  gfx9
// s_waitcnt encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4 (left at its
// maximum), lgkmcnt 11:8 (zero).
template <int N>
__device__ __forceinline__ void ring_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// The stage loop is built from lambdas; each must be inlined, or ring slots
// would become run-time pointers (and every LDS read would wait for every
// outstanding load).
#define MOE_INLINE __attribute__((always_inline))

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1, so that i is a
// constant inside f.
template <int I, int N, typename F>
__device__ __forceinline__ void static_for_from(F &&f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for_from<I + 1, N>(f);
    }
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) { static_for_from<0, N>(f); }

// Parts for the prefill down product.  A launch runs ceil(tiles / 8) tiles
// per XCD, cu_per_xcd at a time (one workgroup per CU); when the last round
// is mostly empty, cutting every tile's reduction in S parts makes S times
// as many tiles of 1/S the length, which fill the rounds better.  Each
// extra part costs a pass over the fp32 partial sums (written here, read by
// the combine), about a fifth of a round at the 8x7B shape.  Returns the S
// in 1..kMaxDownSplit with the least estimated time (ties: fewer parts).
__host__ __device__ inline int down_split_parts(int mt_total, int n_cols, int cu_per_xcd,
                                                int k_stages) {
    if (cu_per_xcd <= 0) return 1;
    const int64_t tiles = (int64_t)mt_total * n_cols;
    int best = 1;
    float best_cost = 0.0f;
    for (int S = 1; S <= kMaxDownSplit && S <= k_stages; ++S) {
        const int64_t per_xcd = (tiles * S + 7) / 8;
        const int64_t rounds = (per_xcd + cu_per_xcd - 1) / cu_per_xcd;
        const float cost = (float)rounds / (float)S + 0.2f * (float)(S - 1);
        if (S == 1 || cost < best_cost) {
            best = S;
            best_cost = cost;
        }
    }
    return best;
}

// With NMAT = 2 and GU, the body also stores the gate and up products
// themselves (fp32, row-major like h) to g_out / u_out, for the backward,
// which needs them for the SwiGLU derivative.
//
// BT (backward products, NMAT = 1): B is K-contiguous, B0 + e * N * K1 +
// n * K1 + k (a transposed weight matrix), staged and read like A.  With A2
// / B2 not NULL the reduction runs over K = 2 * K1: the first K1 from (A,
// B0), the second from (A2, B2), all with row stride K1 (two products
// added in one pass).  BT_STORE writes C fp32; BT_DSWIGLU takes the result
// as da and writes dg = da * u * silu'(g) and du = da * silu(g) (bf16) from
// g_in / u_in (fp32), all [rows, N].
//
// KSPLIT (NMAT = 1): the reduction is cut into `parts` contiguous runs of
// whole K stages, part p writing its fp32 partial sums to C + p *
// part_stride.  The flat tile list treats (part, column tile) as one column
// index, part slowest, so the parts of a tile run in the same tile group.
// With parts = 0 the body picks the count itself from the expert counts
// (down_split_parts, cu_per_xcd CUs per XCD) and workgroup 0 stores it to
// parts_out for the combine.
//
// Kernels wrap the body (below); the forward's take exactly the parameters
// they always had, so their registers and code do not change.
enum { BT_NONE = 0, BT_STORE = 1, BT_DSWIGLU = 2 };
template <int NMAT, bool GU, int BT = BT_NONE, bool KSPLIT = false>
__device__ __forceinline__ void prefill_dma_body(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B0,
    const uint16_t *__restrict__ B1, void *__restrict__ C, const int32_t *__restrict__ counts,
    const int32_t *__restrict__ offsets, int E, int K, int N, int a_rows,
    float *__restrict__ g_out, float *__restrict__ u_out,
    const uint16_t *__restrict__ A2 = nullptr, const uint16_t *__restrict__ B2 = nullptr,
    int K1 = 0, const float *__restrict__ g_in = nullptr, const float *__restrict__ u_in = nullptr,
    uint16_t *__restrict__ dg_out = nullptr, uint16_t *__restrict__ du_out = nullptr,
    int parts = 1, size_t part_stride = 0, int cu_per_xcd = 0, int *parts_out = nullptr) {
    static_assert(BT == BT_NONE || (NMAT == 1 && !GU), "backward products take one matrix");
    static_assert(!KSPLIT || (NMAT == 1 && BT != BT_DSWIGLU), "split reductions store fp32 C");
    constexpr int NW = PWM * PWN;
    constexpr int TM = PBM / PWM, TN = PBN / PWN;
    constexpr int MB = TM / 32, NB = TN / 32;
    constexpr int BNM = PBN / NMAT;
    constexpr int AI = DA_BYTES / 1024 / NW;   // A load instructions per wave per stage
    constexpr int BI = DB_BYTES / 1024 / NW;   // B load instructions per wave per stage
    static_assert(NMAT == 1 || NB % 2 == 0, "gate/up blocks come in pairs");

    const int n_cols = N / BNM;
    if constexpr (KSPLIT) {
        if (parts == 0) {
            int mt_total = 0;
            for (int i = 0; i < E; ++i) mt_total += (counts[i] + PBM - 1) / PBM;
            const int stages = (BT != BT_NONE ? (A2 ? 2 * K1 : K1) : K) / DBK;
            parts = down_split_parts(mt_total, n_cols, cu_per_xcd, stages);
            if (blockIdx.x == 0 && threadIdx.x == 0) *parts_out = parts;
        }
    }
    const int n_tiles = KSPLIT ? n_cols * parts : n_cols;
    int e, row0, row_end, nt;
    if (!prefill_tile(counts, offsets, E, n_tiles, e, row0, row_end, nt)) return;
    int part = 0;
    if constexpr (KSPLIT) {
        part = nt / n_cols;
        nt -= part * n_cols;
    }
    const int n0 = nt * BNM;

    // One array per ring slot: the compiler then knows that the LDS-DMA
    // writes into one slot never alias the fragment reads from another and
    // keeps them overlapped (with a single array it waits for every
    // outstanding load before each read, about 15% slower).
    __shared__ __attribute__((aligned(1024))) uint8_t sa0[DA_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t sa1[DA_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t sa2[DAS > 2 ? DA_BYTES : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t sb0[DB_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t sb1[DB_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t sb2[DBS > 2 ? DB_BYTES : 16];
    // Slot of stage i in each ring (i a compile-time constant at every use).
    auto slot_a = [&](auto i_c) MOE_INLINE {
        constexpr int i = decltype(i_c)::value % DAS;
        return i == 0 ? sa0 : i == 1 ? sa1 : sa2;
    };
    auto slot_b = [&](auto i_c) MOE_INLINE {
        constexpr int i = decltype(i_c)::value % DBS;
        return i == 0 ? sb0 : i == 1 ? sb1 : sb2;
    };

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / PWN, wn = wave % PWN;

    // Global sources of this wave's load instructions.  A instruction g
    // covers 8 rows (8 lanes x 16 B per row); B instruction g covers 2 K rows
    // (32 lanes x 16 B each).  Addresses are recomputed at each issue from a
    // few per-lane values, which keeps register use low.
    constexpr int AROWS = 64 / DACH;           // A rows per load instruction
    const int a_r0 = wave * AI * AROWS + lane / DACH;  // row of instruction 0
    int a_kc[2];                               // K chunk for even / odd instructions
#pragma unroll
    for (int p = 0; p < 2; ++p) a_kc[p] = (lane % DACH) ^ aswz(a_r0 + p * AROWS);
    // B: the swizzle pattern repeats every 4 instructions (bswz uses r & 7).
    size_t b_base[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int r = (wave * BI + p) * 2 + (lane >> 5);
        const int cc = (lane & 31) ^ bswz(r);
        const uint16_t *base;
        int col;
        if (NMAT == 2) {
            base = cc < 16 ? B0 : B1;
            col = n0 + (cc & 15) * 8;
        } else {
            base = B0;
            col = n0 + cc * 8;
        }
        b_base[p] = (size_t)(base - B0) + (size_t)e * K * N + (size_t)r * N + col;
    }

    auto issue_a = [&](uint8_t *sa, int k0) MOE_INLINE {
        if constexpr (BT == BT_NONE) {
#pragma unroll
            for (int j = 0; j < AI; ++j) {
                const int r = min(row0 + a_r0 + j * AROWS, a_rows - 1);
                const uint16_t *src = A + (size_t)r * K + k0 + a_kc[j & 1] * 8;
                __builtin_amdgcn_global_load_lds(src, (lds_void_t *)(sa + (wave * AI + j) * 1024),
                                                 16, 0, 0);
            }
        } else {
            const uint16_t *Ab = A;
            int ka = k0;
            if (A2 && k0 >= K1) { Ab = A2; ka = k0 - K1; }
#pragma unroll
            for (int j = 0; j < AI; ++j) {
                const int r = min(row0 + a_r0 + j * AROWS, a_rows - 1);
                const uint16_t *src = Ab + (size_t)r * K1 + ka + a_kc[j & 1] * 8;
                __builtin_amdgcn_global_load_lds(src, (lds_void_t *)(sa + (wave * AI + j) * 1024),
                                                 16, 0, 0);
            }
        }
    };
    auto issue_b = [&](uint8_t *sb, int k0) MOE_INLINE {
        if constexpr (BT == BT_NONE) {
#pragma unroll
            for (int j = 0; j < BI; ++j) {
                const uint16_t *src = B0 + b_base[j & 3] + (size_t)(k0 + (j & ~3) * 2) * N;
                __builtin_amdgcn_global_load_lds(src, (lds_void_t *)(sb + (wave * BI + j) * 1024),
                                                 16, 0, 0);
            }
        } else {
            // K-contiguous B: the tile's 256 columns are lines of 64 K values,
            // staged exactly like A's rows (same swizzle).
            const uint16_t *Bb = B0;
            int kb = k0;
            if (B2 && k0 >= K1) { Bb = B2; kb = k0 - K1; }
            Bb += (size_t)e * N * K1;
#pragma unroll
            for (int j = 0; j < BI; ++j) {
                const int n = min(n0 + a_r0 + j * AROWS, N - 1);
                const uint16_t *src = Bb + (size_t)n * K1 + kb + a_kc[j & 1] * 8;
                __builtin_amdgcn_global_load_lds(src, (lds_void_t *)(sb + (wave * BI + j) * 1024),
                                                 16, 0, 0);
            }
        }
    };

    // Operand read offsets inside a stage.  The A swizzle depends only on
    // the row modulo 16, i.e. on the lane, so M blocks and K steps become
    // immediate offsets; the B swizzle depends only on the K row modulo 8.
    constexpr int KS = DBK / 16;                   // 32x32x16 steps per stage
    const int a_row = wm * TM + (lane & 31);
    int a_off[KS];
#pragma unroll
    for (int h = 0; h < KS; ++h)
        a_off[h] = a_row * (DBK * 2) + (((h * 2 + (lane >> 5)) ^ aswz(a_row)) << 4);
    const int G = lane >> 4, jq = (lane & 15) >> 2, q = lane & 3;
    int b_off[NB][2];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        int nb;
        if (NMAT == 2) nb = (j / (NB / 2)) * 128 + wn * (TN / 2) + (j % (NB / 2)) * 32;
        else nb = wn * TN + j * 32;
        const int n = nb + 16 * (G & 1) + 4 * q;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int r = 8 * (G >> 1) + 4 * u + jq;     // + 16 * step (immediate)
            b_off[j][u] = r * 512 + ((((n >> 3) ^ bswz(r))) << 4) + (n & 7) * 2;
        }
    }

    // K-contiguous B (BT): fragments read like A's, line wn * TN + 32 j + l % 32.
    const int bt_row = wn * TN + (lane & 31);
    int bt_off[KS];
#pragma unroll
    for (int h = 0; h < KS; ++h)
        bt_off[h] = bt_row * (DBK * 2) + (((h * 2 + (lane >> 5)) ^ aswz(bt_row)) << 4);

    f32x16_t acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int qq = 0; qq < 16; ++qq) acc[i][j][qq] = 0.0f;

    // One stage, in halves of KH steps: the operand fragments of a half are
    // read first (in step order, so the waits before each step's MFMAs are
    // partial), and the scheduler interleaves the reads of one half with
    // the MFMAs of the other (iglp strategy 0).
    constexpr int KH = 1;
    static_assert(KS % KH == 0, "whole halves");
    auto compute = [&](const uint8_t *sa, const uint8_t *sb) MOE_INLINE {
        __builtin_amdgcn_iglp_opt(0);
#pragma unroll
        for (int h0 = 0; h0 < KS; h0 += KH) {
            bf16x8_t af[KH][MB], bfr[KH][NB];
#pragma unroll
            for (int hh = 0; hh < KH; ++hh) {
                const int h = h0 + hh;
#pragma unroll
                for (int i = 0; i < MB; ++i)
                    af[hh][i] = as_bf16x8(*reinterpret_cast<const uint4 *>(
                        sa + a_off[h] + i * 32 * (DBK * 2)));
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    if constexpr (BT == BT_NONE) {
                        s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) s16x4_t *)(sb + b_off[j][0] +
                                                                          h * 8192));
                        s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) s16x4_t *)(sb + b_off[j][1] +
                                                                          h * 8192));
                        bfr[hh][j] = __builtin_bit_cast(
                            bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                    } else {
                        bfr[hh][j] = as_bf16x8(*reinterpret_cast<const uint4 *>(
                            sb + bt_off[h] + j * 32 * (DBK * 2)));
                    }
                }
            }
#pragma unroll
            for (int hh = 0; hh < KH; ++hh)
#pragma unroll
                for (int i = 0; i < MB; ++i)
#pragma unroll
                    for (int j = 0; j < NB; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            af[hh][i], bfr[hh][j], acc[i][j], 0, 0, 0);
        }
    };

    // Issue order: at step kt, A_{kt+DAS-1} and B_{kt+DBS-1}, the operand
    // with the shorter lookahead first; the prologue issues what steps -2
    // and -1 would have.  Stage kt has landed once at most the loads issued
    // after its later operand are outstanding: those of the deeper ring's
    // operand issued in the same step (none when both rings are 2 deep).
    // Loads are issued unconditionally, past the last stage with K clamped
    // to it (harmless re-reads into free slots), so the steady-state loop has
    // no branches and every wait count is a constant; the rings are drained
    // before the epilogue reuses them.
    int nk = K / DBK, kt0 = 0;
    if constexpr (BT != BT_NONE) nk = (A2 ? 2 * K1 : K1) / DBK;
    if constexpr (KSPLIT) {
        const int all = nk;
        kt0 = (int)((int64_t)all * part / parts);
        nk = (int)((int64_t)all * (part + 1) / parts) - kt0;
    }
    auto kclamp = [&](int kt) { return (kt0 + min(kt, nk - 1)) * DBK; };
    constexpr int LA = DAS - 1, LB = DBS - 1;      // lookahead of each ring
    constexpr int WAIT = DAS > DBS ? AI : DBS > DAS ? BI : 0;
    auto issue_step = [&](auto s_c, int kt) MOE_INLINE {   // loads of step kt (slot s)
        constexpr int s = decltype(s_c)::value;
        auto a = [&]() MOE_INLINE {
            if (kt + LA >= 0)
                issue_a(slot_a(std::integral_constant<int, s + LA>{}), kclamp(kt + LA));
        };
        auto b = [&]() MOE_INLINE {
            if (kt + LB >= 0)
                issue_b(slot_b(std::integral_constant<int, s + LB>{}), kclamp(kt + LB));
        };
        if (LA <= LB) { a(); b(); } else { b(); a(); }
    };
    constexpr int U = DAS == 3 || DBS == 3 ? 6 : 2;   // unroll: every ring slot is static
    issue_step(std::integral_constant<int, U - 2>{}, -2);
    issue_step(std::integral_constant<int, U - 1>{}, -1);
    auto step = [&](auto s_c, int kt) MOE_INLINE {
        ring_barrier<WAIT>();
        issue_step(s_c, kt);
        compute(slot_a(s_c), slot_b(s_c));
    };
    int kt = 0;
    for (; kt + U <= nk; kt += U)
        static_for<U>([&](auto s_c) MOE_INLINE { step(s_c, kt + decltype(s_c)::value); });
    static_for<U - 1>([&](auto s_c) MOE_INLINE {
        if (kt + decltype(s_c)::value < nk) step(s_c, kt + decltype(s_c)::value);
    });
    ring_barrier<0>();

    if constexpr (NMAT == 2) {
        // h = silu(g) * u for the tile's 256 rows x 128 columns, staged
        // through LDS (the rings are free now) as row-major bf16, then
        // written out as full 16-byte row segments.  Storing 2-byte elements
        // straight from the MFMA layout (one column per lane) cost a quarter
        // of the kernel's time.  Rows are split into four pieces of 64, piece
        // p held by ring slot p.
        constexpr int HP = BNM + 8;                      // LDS row pitch (bf16)
        constexpr int RQ = 64;
        static_assert(RQ * HP * 2 <= DA_BYTES && RQ * HP * 2 <= DB_BYTES, "piece fits a slot");
        static_assert(PBM / RQ == 4 && TM % RQ == 0, "four pieces, 32-row blocks inside one");
        auto piece = [&](int pc) {
            uint8_t *pp = sa0;
            if (pc == 1) pp = sa1;
            if (pc == 2) pp = sb0;
            if (pc == 3) pp = sb1;
            return reinterpret_cast<uint16_t *>(pp);
        };
        __syncthreads();
#pragma unroll
        for (int i = 0; i < MB; ++i) {
            const int rb = wm * TM + i * 32;             // first row of this block
            uint16_t *const hw = piece(rb / RQ) + (rb % RQ) * HP;
#pragma unroll
            for (int j = 0; j < NB / 2; ++j)
#pragma unroll
                for (int qq = 0; qq < 16; ++qq) {
                    const int r = 8 * (qq >> 2) + 4 * (lane >> 5) + (qq & 3);
                    const int cl = wn * (TN / 2) + j * 32 + (lane & 31);
                    const float hv = silu_f32(acc[i][j][qq]) * acc[i][j + NB / 2][qq];
                    hw[r * HP + cl] = (uint16_t)f32_to_bf16(hv);
                }
        }
        __syncthreads();
        if constexpr (GU) {
            // 32x32 accumulator layout: value q of lane l is row
            // 8*(q/4) + 4*(l/32) + q%4, column l%32 of the block.
#pragma unroll
            for (int i = 0; i < MB; ++i)
#pragma unroll
                for (int j = 0; j < NB / 2; ++j) {
                    const int col = n0 + wn * (TN / 2) + j * 32 + (lane & 31);
#pragma unroll
                    for (int qq = 0; qq < 16; ++qq) {
                        const int row =
                            row0 + wm * TM + i * 32 + 8 * (qq >> 2) + 4 * (lane >> 5) + (qq & 3);
                        if (row < row_end) {
                            g_out[(size_t)row * N + col] = acc[i][j][qq];
                            u_out[(size_t)row * N + col] = acc[i][j + NB / 2][qq];
                        }
                    }
                }
        }
        constexpr int CH = BNM / 8;                      // 16-byte chunks per row
        uint16_t *H = static_cast<uint16_t *>(C);
        for (int v = tid; v < PBM * CH; v += NW * 64) {
            const int r = v / CH, c8 = (v % CH) * 8;
            if (row0 + r < row_end)
                store_stream16(H + (size_t)(row0 + r) * N + n0 + c8,
                               *reinterpret_cast<const uint4 *>(piece(r / RQ) + (r % RQ) * HP + c8));
        }
    } else {
        // 32x32 accumulator layout: value q of lane l is row
        // 8*(q/4) + 4*(l/32) + q%4, column l%32 of the block.
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int col = n0 + wn * TN + j * 32 + (lane & 31);
                // dswiglu: the block's 16 g and 16 u values are loaded
                // first, unconditionally (rows clamped into the tile), so
                // they are all in flight at once; only the stores depend on
                // the row being inside the tile.
                float gv[16], uv[16];
                if constexpr (BT == BT_DSWIGLU) {
#pragma unroll
                    for (int qq = 0; qq < 16; ++qq) {
                        const int row = min(row0 + wm * TM + i * 32 + 8 * (qq >> 2) +
                                                4 * (lane >> 5) + (qq & 3),
                                            row_end - 1);
                        gv[qq] = g_in[(size_t)row * N + col];
                        uv[qq] = u_in[(size_t)row * N + col];
                    }
                }
#pragma unroll
                for (int qq = 0; qq < 16; ++qq) {
                    const int row =
                        row0 + wm * TM + i * 32 + 8 * (qq >> 2) + 4 * (lane >> 5) + (qq & 3);
                    if constexpr (BT == BT_DSWIGLU) {
                        const float da = acc[i][j][qq], g = gv[qq], u = uv[qq];
                        const float sg = 1.0f / (1.0f + expf(-g));
                        const uint16_t dgv =
                            (uint16_t)f32_to_bf16(da * u * sg * (1.0f + g * (1.0f - sg)));
                        const uint16_t duv = (uint16_t)f32_to_bf16(da * g * sg);
                        if (row < row_end) {
                            const size_t ci = (size_t)row * N + col;
                            dg_out[ci] = dgv;
                            du_out[ci] = duv;
                        }
                    } else if constexpr (KSPLIT) {
                        if (row < row_end)
                            static_cast<float *>(C)[(size_t)part * part_stride +
                                                    (size_t)row * N + col] = acc[i][j][qq];
                    } else {
                        if (row < row_end)
                            static_cast<float *>(C)[(size_t)row * N + col] = acc[i][j][qq];
                    }
                }
            }
    }
}

template <int NMAT>
__global__ __launch_bounds__(PWM * PWN * 64, 1) void prefill_dma_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B0,
    const uint16_t *__restrict__ B1, void *__restrict__ C, const int32_t *__restrict__ counts,
    const int32_t *__restrict__ offsets, int E, int K, int N, int a_rows) {
    prefill_dma_body<NMAT, false>(A, B0, B1, C, counts, offsets, E, K, N, a_rows, nullptr,
                                  nullptr);
}

// The gate/up kernel that also stores g and u (for the backward).
__global__ __launch_bounds__(PWM * PWN * 64, 1) void prefill_dma_gu_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B0,
    const uint16_t *__restrict__ B1, uint16_t *__restrict__ C, const int32_t *__restrict__ counts,
    const int32_t *__restrict__ offsets, int E, int K, int N, int a_rows,
    float *__restrict__ g_out, float *__restrict__ u_out) {
    prefill_dma_body<2, true>(A, B0, B1, C, counts, offsets, E, K, N, a_rows, g_out, u_out);
}

// The down product with its reduction cut into `parts` partial sums.
__global__ __launch_bounds__(PWM * PWN * 64, 1) void prefill_dma_down_split_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B, float *__restrict__ C,
    const int32_t *__restrict__ counts, const int32_t *__restrict__ offsets, int E, int K, int N,
    int a_rows, int parts, size_t part_stride, int cu_per_xcd, int *__restrict__ parts_out) {
    prefill_dma_body<1, false, BT_NONE, true>(A, B, nullptr, C, counts, offsets, E, K, N, a_rows,
                                              nullptr, nullptr, nullptr, nullptr, 0, nullptr,
                                              nullptr, nullptr, nullptr, parts, part_stride,
                                              cu_per_xcd, parts_out);
}

// dXp-style product (K-contiguous B, optional second operand pair) with its
// reduction cut into parts, as the down product above.
__global__ __launch_bounds__(PWM * PWN * 64, 1) void prefill_dma_bt_store_split_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B, const uint16_t *__restrict__ A2,
    const uint16_t *__restrict__ B2, float *__restrict__ C, const int32_t *__restrict__ counts,
    const int32_t *__restrict__ offsets, int E, int K1, int N, int a_rows, size_t part_stride,
    int cu_per_xcd, int *__restrict__ parts_out) {
    prefill_dma_body<1, false, BT_STORE, true>(A, B, nullptr, C, counts, offsets, E, K1, N,
                                               a_rows, nullptr, nullptr, A2, B2, K1, nullptr,
                                               nullptr, nullptr, nullptr, 0, part_stride,
                                               cu_per_xcd, parts_out);
}

// Backward products with a K-contiguous B (see prefill_dma_body).
__global__ __launch_bounds__(PWM * PWN * 64, 1) void prefill_dma_bt_dswiglu_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B,
    const int32_t *__restrict__ counts, const int32_t *__restrict__ offsets, int E, int K1, int N,
    int a_rows, const float *__restrict__ g_in, const float *__restrict__ u_in,
    uint16_t *__restrict__ dg_out, uint16_t *__restrict__ du_out) {
    prefill_dma_body<1, false, BT_DSWIGLU>(A, B, nullptr, nullptr, counts, offsets, E, K1, N,
                                           a_rows, nullptr, nullptr, nullptr, nullptr, K1, g_in,
                                           u_in, dg_out, du_out);
}

// Grid for the prefill kernels: worst-case tile count (every expert may
// end with a partial row tile), rounded up to a multiple of the 8 XCDs.
inline int prefill_grid(int rows, int E, int n_tiles) {
    const long tiles = (long)((rows + PBM - 1) / PBM + E) * n_tiles;
    return (int)((tiles + 7) / 8 * 8);
}

// ---------------------------------------------------------------------------
// Decode: weight-streaming grouped GEMM for experts with at most 16*MB rows.

constexpr int DWAVES = 8;     // wavefronts per workgroup, splitting K
constexpr int DCOLS = 128;    // weight columns per workgroup

// Decode workgroup units are (expert, column block) pairs, unit u = e * nb +
// column block.  TAIL: a 1-D grid where the first n_full units run whole
// and the rest are cut in two K halves (workgroups n_full + 2 j and
// n_full + 2 j + 1 for unit n_full + j), which store their fp32 sums (of
// x W1 and x W3 for gate/up, of h W2 for down) to part slot j (see
// decode_tail_slot) for decode_tail_finish_kernel.  One workgroup per CU at
// a time: when the units leave the last round at most half full, its units
// cut in halves fill one round of half the length.
constexpr int DTAIL_ROWS = 32;   // rows of a part slot (an expert's rows at decode sizes)
__device__ __forceinline__ size_t decode_tail_slot(int j, int half, int m) {
    return ((size_t)(j * 2 + half) * 2 + m) * DTAIL_ROWS * DCOLS;
}
template <int MB, int NMAT, bool TAIL = false, bool RANK = false>
__global__ __launch_bounds__(DWAVES * 64) void decode_gemm_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B0,
    const uint16_t *__restrict__ B1, void *__restrict__ C, const int32_t *__restrict__ counts,
    const int32_t *__restrict__ offsets, int K, int N, int a_rows,
    const int32_t *__restrict__ src, float *__restrict__ part = nullptr, int n_full = 0,
    int nb_cols = 0, DecodeRank rk = DecodeRank{}, int n_exp = 0, int early = 0) {
    static_assert(!TAIL || MB * 16 <= DTAIL_ROWS, "a part slot holds an expert's rows");
    static_assert(kDecodeMaxT * kMaxTopK <= 128 && kMaxExperts <= 64, "one wavefront ranks");
    int e = blockIdx.y, cblk = blockIdx.x, half = -1, slot = 0;
    if constexpr (TAIL) {
        int unit = blockIdx.x;
        if (unit >= n_full) {
            slot = (unit - n_full) >> 1;
            half = (unit - n_full) & 1;
            unit = n_full + slot;
        }
        e = unit / nb_cols;
        cblk = unit - e * nb_cols;
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kg = lane >> 4, nb = lane & 15;
    const int col = cblk * DCOLS + nb * 8;
    const bool col_ok = col < N;

    const uint16_t *Bp[NMAT];
    Bp[0] = B0 + (size_t)e * K * N + (col_ok ? col : 0);
    if (NMAT == 2) Bp[NMAT - 1] = B1 + (size_t)e * K * N + (col_ok ? col : 0);
    int nks = (K + 31) >> 5, kbase = 0;
    if constexpr (TAIL) {
        if (half >= 0) {
            const int all = nks;
            kbase = (all * half) / 2;
            nks = (all * (half + 1)) / 2 - kbase;
        }
    }
    const int ks0 = kbase + (nks * wave) / DWAVES, ks1 = kbase + (nks * (wave + 1)) / DWAVES;
    auto load_b = [&](uint4 (&rb)[NMAT][8], int ks) __attribute__((always_inline)) {
        const int k = ks * 32 + kg * 8;
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int i = 0; i < 8; ++i)
                rb[m][i] = (k + i < K && col_ok) ? load_stream16(Bp[m] + (size_t)(k + i) * N)
                                                 : zero4();
    };
    // early: the weights of this wavefront's first step are requested before
    // the routing is read (they do not depend on it), so that the routing's
    // latency overlaps theirs.  The launcher sets it only when nearly every
    // expert holds rows; an expert with none wastes that one step.
    uint4 rb0[NMAT][8];
    const bool pre = early && ks0 < ks1;
    if (pre) load_b(rb0, ks0);
    __shared__ int32_t s_counts[RANK ? kMaxExperts : 1], s_offsets[RANK ? kMaxExperts + 1 : 1];
    __shared__ int32_t s_src[RANK ? kDecodeMaxT * kMaxTopK : 1];
    if constexpr (RANK) {
        if (wave == 0)
            decode_rank_wave(rk, n_exp, lane, s_counts, s_offsets, s_src,
                             blockIdx.x == 0 && blockIdx.y == 0);
        __syncthreads();
        counts = s_counts;
        offsets = s_offsets;
        src = s_src;
    }
    const int Me = counts[e];
    if (Me == 0) return;  // an expert no token chose: its weights are never read
    const int r0 = offsets[e];
    const int nmb = min(MB, (Me + 15) >> 4);
    // Row i*16 + lane%16 of this expert; rows past the end of A are clamped
    // onto its last row (their results are never stored).  With src, grouped
    // row r is row src[r] of A (A is then x itself: a gather, no copy).
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

    auto step = [&](const uint4 (&rb)[NMAT][8], int ks) __attribute__((always_inline)) {
        const int k = ks * 32 + kg * 8;
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
    };
    int ks = ks0;
    if (pre) step(rb0, ks++);
    for (; ks < ks1; ++ks) {
        uint4 rb[NMAT][8];
        load_b(rb, ks);
        step(rb, ks);
    }

    // Output row `row` (of this expert) from block i, value j of this lane's
    // accumulators: h = bf16(silu(g) * u) for gate/up, o fp32 for down.
    auto store_out = [&](int i, int j, int row) __attribute__((always_inline)) {
        if constexpr (NMAT == 2) {
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
    };

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
            if (TAIL && half >= 0) {
#pragma unroll
                for (int m = 0; m < NMAT; ++m) {
                    float *dst = part + decode_tail_slot(slot, half, m) + (size_t)row * DCOLS +
                                 nb * 8;
                    *reinterpret_cast<float4 *>(dst) =
                        make_float4(acc[m][i][0][j], acc[m][i][1][j], acc[m][i][2][j],
                                    acc[m][i][3][j]);
                    *reinterpret_cast<float4 *>(dst + 4) =
                        make_float4(acc[m][i][4][j], acc[m][i][5][j], acc[m][i][6][j],
                                    acc[m][i][7][j]);
                }
            } else {
                store_out(i, j, row);
            }
        }
    }
}

// The units a TAIL launch cut in two: workgroup j takes part slot j (unit
// n_full + j) and adds its halves, half 0 first.  Gate/up (NMAT = 2):
// h = silu(g0 + g1) * (u0 + u1), bf16.  Down (NMAT = 1): o = o0 + o1, fp32.
template <int NMAT>
__global__ __launch_bounds__(256) void decode_tail_finish_kernel(
    const float *__restrict__ part, const int32_t *__restrict__ counts,
    const int32_t *__restrict__ offsets, int n_full, int nb_cols, int N, void *__restrict__ out) {
    const int j = blockIdx.x, unit = n_full + j;
    const int e = unit / nb_cols, cblk = unit - e * nb_cols;
    const int Me = counts[e], r0 = offsets[e];
    // four consecutive columns per thread (N % 8 == 0: all in or all out)
    const float4 *g0 = reinterpret_cast<const float4 *>(part + decode_tail_slot(j, 0, 0));
    const float4 *g1 = reinterpret_cast<const float4 *>(part + decode_tail_slot(j, 1, 0));
    const float4 *u0 = reinterpret_cast<const float4 *>(part + decode_tail_slot(j, 0, 1));
    const float4 *u1 = reinterpret_cast<const float4 *>(part + decode_tail_slot(j, 1, 1));
    for (int i = threadIdx.x; i < Me * (DCOLS / 4); i += 256) {
        const int row = i / (DCOLS / 4), col = cblk * DCOLS + 4 * (i % (DCOLS / 4));
        if (col >= N) continue;
        const float4 a = g0[i], b = g1[i];
        const float g[4] = {a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w};
        if constexpr (NMAT == 2) {
            const float4 c = u0[i], d = u1[i];
            const float u[4] = {c.x + d.x, c.y + d.y, c.z + d.z, c.w + d.w};
            uint32_t hv[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) hv[q] = f32_to_bf16(silu_f32(g[q]) * u[q]);
            *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(out) + (size_t)(r0 + row) * N +
                                       col) = make_uint2(hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16));
        } else {
            *reinterpret_cast<float4 *>(static_cast<float *>(out) + (size_t)(r0 + row) * N + col) =
                make_float4(g[0], g[1], g[2], g[3]);
        }
    }
}

// Units of a decode product to run whole (the rest are cut in K halves),
// or -1 for none cut: with every expert holding rows (as at decode sizes)
// a launch has E * ceil(N / 128) units, one per CU at a time; cutting pays
// when the last round would be at most half full.
int decode_tail_full_units(int N, int E) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        return -1;
    const int units = (N + DCOLS - 1) / DCOLS * E;
    const int rem = units % cus;
    if (units <= cus || rem == 0 || 2 * rem > cus || rem > kDecodeTailMaxUnits) return -1;
    return units - rem;
}

template <int MB, bool RANK>
hipError_t launch_decode_gateup(const moe_shape_t &s, const uint16_t *xp,
                                const int32_t *counts, const int32_t *offsets,
                                const uint16_t *w1, const uint16_t *w3, uint16_t *h,
                                hipStream_t stream, const int32_t *src, float *gpart,
                                const DecodeRank &rk) {
    const int d = s.d_model, f = s.d_ff, E = s.n_experts, rows = routed_rows(s);
    const int nb_cols = (f + DCOLS - 1) / DCOLS;
    const int n_full = gpart ? decode_tail_full_units(f, E) : -1;
    const int early = decode_early_weights(rows, E);
    if (n_full >= 0) {
        const int n_cut = nb_cols * E - n_full;
        hipLaunchKernelGGL((decode_gemm_kernel<MB, 2, true, RANK>), dim3(n_full + 2 * n_cut),
                           dim3(DWAVES * 64), 0, stream, xp, w1, w3, h, counts, offsets, d, f,
                           rows, src, gpart, n_full, nb_cols, rk, E, early);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(decode_tail_finish_kernel<2>, dim3(n_cut), dim3(256), 0, stream,
                           gpart, counts, offsets, n_full, nb_cols, f, h);
    } else {
        hipLaunchKernelGGL((decode_gemm_kernel<MB, 2, false, RANK>), dim3(nb_cols, E),
                           dim3(DWAVES * 64), 0, stream, xp, w1, w3, h, counts, offsets, d, f,
                           rows, src, nullptr, 0, 0, rk, E, early);
    }
    return hipGetLastError();
}

// The decode down product, o = h W2[e]: with gpart, the units past the last
// full round are cut in K halves as in launch_decode_gateup.
template <int MB>
hipError_t launch_decode_down(const moe_shape_t &s, const uint16_t *h, const int32_t *counts,
                              const int32_t *offsets, const uint16_t *w2, float *o,
                              hipStream_t stream, float *gpart) {
    const int d = s.d_model, f = s.d_ff, E = s.n_experts, rows = routed_rows(s);
    const int nb_cols = (d + DCOLS - 1) / DCOLS;
    const int n_full = gpart ? decode_tail_full_units(d, E) : -1;
    const int early = decode_early_weights(rows, E);
    if (n_full >= 0) {
        const int n_cut = nb_cols * E - n_full;
        hipLaunchKernelGGL((decode_gemm_kernel<MB, 1, true>), dim3(n_full + 2 * n_cut),
                           dim3(DWAVES * 64), 0, stream, h, w2, nullptr, o, counts, offsets, f,
                           d, rows, nullptr, gpart, n_full, nb_cols, DecodeRank{}, 0, early);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(decode_tail_finish_kernel<1>, dim3(n_cut), dim3(256), 0, stream,
                           gpart, counts, offsets, n_full, nb_cols, d, o);
    } else {
        hipLaunchKernelGGL((decode_gemm_kernel<MB, 1>), dim3(nb_cols, E), dim3(DWAVES * 64), 0,
                           stream, h, w2, nullptr, o, counts, offsets, f, d, rows, nullptr,
                           nullptr, 0, 0, DecodeRank{}, 0, early);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gateup_bf16(const moe_shape_t &s, const uint16_t *xp, const int32_t *counts,
                              const int32_t *offsets, const uint16_t *w1, const uint16_t *w3,
                              uint16_t *h, hipStream_t stream, const int32_t *src,
                              float *gpart, const DecodeRank *rank) {
    const int d = s.d_model, f = s.d_ff, E = s.n_experts, rows = routed_rows(s);
    if (rank && (s.T > kDecodeMaxT || !src || s.n_experts > kMaxExperts ||
                 rank->n_assign > kDecodeMaxT * kMaxTopK))
        return hipErrorInvalidValue;
    const DecodeRank rk = rank ? *rank : DecodeRank{};
    if (s.T <= 16) {
        return rank ? launch_decode_gateup<1, true>(s, xp, counts, offsets, w1, w3, h, stream,
                                                    src, gpart, rk)
                    : launch_decode_gateup<1, false>(s, xp, counts, offsets, w1, w3, h, stream,
                                                     src, gpart, rk);
    } else if (s.T <= kDecodeMaxT) {
        return rank ? launch_decode_gateup<2, true>(s, xp, counts, offsets, w1, w3, h, stream,
                                                    src, gpart, rk)
                    : launch_decode_gateup<2, false>(s, xp, counts, offsets, w1, w3, h, stream,
                                                     src, gpart, rk);
    } else if (src) {
        return hipErrorInvalidValue;   // the gather is only built into the decode kernels
    } else {
        const int grid = prefill_grid(rows, E, (f + PBN / 2 - 1) / (PBN / 2));
        if (q_gateup_supported(rows, d, f))
            return q_launch_gateup(rows, E, xp, counts, offsets, w1, w3, d, f, h, nullptr,
                                   nullptr, stream);
        else if (d % DBK == 0 && f % (PBN / 2) == 0)
            hipLaunchKernelGGL(prefill_dma_kernel<2>, dim3(grid), dim3(PWM * PWN * 64), 0,
                               stream, xp, w1, w3, h, counts, offsets, E, d, f, rows);
        else
            hipLaunchKernelGGL(prefill_gemm_kernel<2>, dim3(grid), dim3(PWM * PWN * 64), 0,
                               stream, xp, w1, w3, h, counts, offsets, E, d, f, rows);
    }
    return hipGetLastError();
}

hipError_t launch_gateup_bf16_gu(const moe_shape_t &s, const uint16_t *xp,
                                 const int32_t *counts, const int32_t *offsets,
                                 const uint16_t *w1, const uint16_t *w3, uint16_t *h, float *g,
                                 float *u, hipStream_t stream) {
    const int d = s.d_model, f = s.d_ff, E = s.n_experts, rows = routed_rows(s);
    if (s.T <= kDecodeMaxT || d % DBK != 0 || f % (PBN / 2) != 0) return hipErrorNotSupported;
    if (q_gateup_supported(rows, d, f))
        return q_launch_gateup(rows, E, xp, counts, offsets, w1, w3, d, f, h, g, u, stream);
    const int grid = prefill_grid(rows, E, (f + PBN / 2 - 1) / (PBN / 2));
    hipLaunchKernelGGL(prefill_dma_gu_kernel, dim3(grid), dim3(PWM * PWN * 64), 0, stream, xp,
                       w1, w3, h, counts, offsets, E, d, f, rows, g, u);
    return hipGetLastError();
}

static bool bt_shape_ok(int rows, int K1, int N) {
    return rows > 0 && K1 % DBK == 0 && N % PBN == 0;
}

static int cus_per_xcd() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return -1;
    return std::max(1, cus / 8);
}

hipError_t launch_bt_store_split_bf16(int rows, int E, const uint16_t *A, const uint16_t *B,
                                      const uint16_t *A2, const uint16_t *B2, int K1, int N,
                                      const int32_t *counts, const int32_t *offsets, float *C,
                                      size_t part_stride, int *parts_out, hipStream_t stream) {
    if (!bt_shape_ok(rows, K1, N) || !parts_out) return hipErrorNotSupported;
    {
        const hipError_t qe = q_launch_bt_store_split(rows, E, A, B, A2, B2, K1, N, counts,
                                                      offsets, C, part_stride, parts_out, stream);
        if (qe != hipErrorNotSupported) return qe;
    }
    const int cpx = cus_per_xcd();
    if (cpx < 0) return hipErrorNotSupported;
    const int grid = prefill_grid(rows, E, (N / PBN) * kMaxDownSplit);
    hipLaunchKernelGGL(prefill_dma_bt_store_split_kernel, dim3(grid), dim3(PWM * PWN * 64), 0,
                       stream, A, B, A2, B2, C, counts, offsets, E, K1, N, rows, part_stride, cpx,
                       parts_out);
    return hipGetLastError();
}

hipError_t launch_bt_dswiglu_bf16(int rows, int E, const uint16_t *A, const uint16_t *B, int K1,
                                  int N, const int32_t *counts, const int32_t *offsets,
                                  const float *g, const float *u, uint16_t *dg, uint16_t *du,
                                  hipStream_t stream) {
    if (!bt_shape_ok(rows, K1, N)) return hipErrorNotSupported;
    const int grid = prefill_grid(rows, E, N / PBN);
    hipLaunchKernelGGL(prefill_dma_bt_dswiglu_kernel, dim3(grid), dim3(PWM * PWN * 64), 0,
                       stream, A, B, counts, offsets, E, K1, N, rows, g, u, dg, du);
    return hipGetLastError();
}

hipError_t launch_down_split_bf16(int rows, int E, const uint16_t *h, const int32_t *counts,
                                  const int32_t *offsets, const uint16_t *w2, int K, int N,
                                  int parts, size_t part_stride, float *o, int *parts_out,
                                  hipStream_t stream) {
    if (rows <= 0 || parts < 0 || parts > kMaxDownSplit || K % DBK != 0 ||
        K / DBK < kMaxDownSplit || N % PBN != 0 || (parts == 0 && !parts_out))
        return hipErrorNotSupported;
    int cu_per_xcd = 0;
    if (parts == 0) {
        cu_per_xcd = cus_per_xcd();
        if (cu_per_xcd < 0) return hipErrorNotSupported;
    }
    if (q_down_supported(rows, K, N))
        return q_launch_down(rows, E, h, counts, offsets, w2, K, N, o, parts, part_stride,
                             cu_per_xcd, parts_out, stream);
    const int grid = prefill_grid(rows, E, (N / PBN) * (parts ? parts : kMaxDownSplit));
    hipLaunchKernelGGL(prefill_dma_down_split_kernel, dim3(grid), dim3(PWM * PWN * 64), 0, stream,
                       h, w2, o, counts, offsets, E, K, N, rows, parts, part_stride, cu_per_xcd,
                       parts_out);
    return hipGetLastError();
}

hipError_t launch_down_bf16(const moe_shape_t &s, const uint16_t *h, const int32_t *counts,
                            const int32_t *offsets, const uint16_t *w2, float *o,
                            hipStream_t stream, float *gpart) {
    const int d = s.d_model, f = s.d_ff, E = s.n_experts, rows = routed_rows(s);
    if (s.T <= 16) {
        return launch_decode_down<1>(s, h, counts, offsets, w2, o, stream, gpart);
    } else if (s.T <= kDecodeMaxT) {
        return launch_decode_down<2>(s, h, counts, offsets, w2, o, stream, gpart);
    } else {
        const int grid = prefill_grid(rows, E, (d + PBN - 1) / PBN);
        if (q_down_supported(rows, f, d))
            return q_launch_down(rows, E, h, counts, offsets, w2, f, d, o, 1, 0, 0, nullptr,
                                 stream);
        else if (f % DBK == 0 && d % PBN == 0)
            hipLaunchKernelGGL(prefill_dma_kernel<1>, dim3(grid), dim3(PWM * PWN * 64), 0,
                               stream, h, w2, nullptr, o, counts, offsets, E, f, d, rows);
        else
            hipLaunchKernelGGL(prefill_gemm_kernel<1>, dim3(grid), dim3(PWM * PWN * 64), 0,
                               stream, h, w2, nullptr, o, counts, offsets, E, f, d, rows);
    }
    return hipGetLastError();
}

}  // namespace moe
