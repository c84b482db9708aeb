// Grouped GEMMs on the CDNA4 matrix cores, software-pipelined for one
// wavefront per SIMD: the tile body and the persistent schedules shared by
// gemm_gateup.hip, gemm_down.hip, gemm_bt.hip and gemm_dw.hip (one
// translation unit each, so that they compile in parallel).  The forward
// products are the two of the SwiGLU expert
// of "Mixtral 8x7B -- The Evolving Transformer", section 04
// (down(silu(gate x) * up x)), applied to the per-expert row batches of
// section 05: gate/up (h = silu(A W1[e]) * (A W3[e]), bf16) and down
// (o = h W2[e], fp32, optionally in K parts).
//
// Tile and wavefront layout.  A workgroup computes a 256-row x 256-column
// output tile (gate/up: 128 gate + the same 128 up columns) with four
// wavefronts, one per SIMD.  Each wavefront owns ALL 256 rows and 64
// columns (gate/up: 32 gate + the matching 32 up columns), i.e. 8 x 2
// blocks of v_mfma_f32_32x32x16_bf16 with 256 fp32 accumulators held in
// AGPRs.  Every weight fragment is therefore read from LDS by exactly one
// wavefront (the transpose read ds_read_b64_tr_b16 is the expensive LDS
// read), and every activation fragment by four.  Per 16-deep K step a
// wavefront issues 16 MFMAs (512 cycles of its SIMD's matrix core), 8
// ds_read_b128 and 4 ds_read_b64_tr_b16.
//
// Schedule.  With one wavefront per SIMD nothing else hides LDS latency,
// so the K loop is written as an explicit pipeline: the 12 fragment reads
// of step k+1 are interleaved one per MFMA with the 16 MFMAs of step k
// (double-buffered fragment registers), and the global->LDS copies of later
// stages go into the remaining MFMA slots.  sched_barrier pins that order.
// Each 64-deep stage has one workgroup barrier, placed after the first MFMA
// of the stage's last step, so that it and the first reads of the next
// stage run while the matrix core is busy.
//
// Operands reach LDS by buffer_load ... lds (no registers, no VALU): the
// activations in a 2-slot ring and the weights (mostly fetched from beyond
// L2) in a 3-slot ring, five 32 KiB slots filling the 160 KiB of LDS.  The
// buffer resource of the activations ends at their last row, so rows past
// it read as zeros.  Loads past the last stage re-read the last stage into
// a free slot, so every wait count in the loop is a constant.
#pragma once
#include <algorithm>
#include <type_traits>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int QBM = 256;               // rows per tile
constexpr int QBN = 256;               // columns per tile
constexpr int QBK = 64;                // reduction depth of one stage
constexpr int QW = 4;                  // wavefronts per workgroup
constexpr int QT = QW * 64;            // threads per workgroup
constexpr int QSLOT = QBM * QBK * 2;   // bytes of one stage of either operand: 32 KiB
constexpr int QAS = 2, QBS = 3;        // ring depths (activations, weights)
constexpr int QU = 6;                  // stages per unrolled loop body (lcm of the depths)
constexpr int QPGM = 4;                // row tiles per scheduling group
constexpr int QMAXSPLIT = kMaxDownSplit;

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
#define Q_INLINE __attribute__((always_inline))

// The thread index, taken afresh for each tile: the empty asm hides that it
// is the same on every tile, so the copy and fragment offsets derived from
// it are recomputed per tile (a few integer ops) instead of being held
// across the whole persistent loop, where they were spilled to scratch and
// reloaded in every epilogue.
__device__ __forceinline__ int q_tid() {
    int t = (int)threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
}

template <int I, int N, typename F>
__device__ __forceinline__ void q_for_from(F &&f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        q_for_from<I + 1, N>(f);
    }
}
// f(integral_constant<int, i>) for i = 0 .. N-1.
template <int N, typename F>
__device__ __forceinline__ void q_for(F &&f) { q_for_from<0, N>(f); }

// Raw buffer resource over `bytes` bytes at `base` (gfx9 word 3: 32-bit
// untyped data).  Offsets at or past `bytes` read as zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t q_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// 16 bytes per lane from rsrc + voffset + soffset into LDS at dst + 16 * lane.
__device__ __forceinline__ void q_dma(__amdgpu_buffer_rsrc_t r, uint8_t *dst, uint32_t voff,
                                      uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)dst, 16, (int)voff, (int)soff, 0, 0);
}

// Swizzles (16-byte chunk index XOR a function of the LDS row) that keep
// the fragment reads of consecutive rows on distinct banks.
//   activations: 8 chunks per 128-byte row;
//   weights, one matrix: 32 chunks per 512-byte row;
//   weights, gate | up: two sub-tiles of 16 chunks per 256-byte row.
__device__ __forceinline__ int q_aswz(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); }
__device__ __forceinline__ int q_bswz1(int r) { return (r & 7) << 2; }
__device__ __forceinline__ int q_bswz2(int r) { return (r & 3) << 2; }

// Workgroup barrier of the rings: this wavefront's LDS copies up to the
// last N issued have landed and its LDS reads have returned, then all
// wavefronts meet.  (__syncthreads would wait for every outstanding copy.)
// gfx9 s_waitcnt: vmcnt bits 3:0 and 15:14, expcnt 6:4 (left at its
// maximum), lgkmcnt 11:8 (zero).
template <int N>
__device__ __forceinline__ void q_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// Persistent schedule.  The grid is one workgroup per CU (8 XCDs x
// cu_per_xcd); each workgroup runs a list of tiles.
//
// Row tiles (256 rows of one expert) fall into three classes by the 32-row
// blocks they need: class 0 (more than 128 rows: 8 blocks), class 1 (65 to
// 128 rows: 4 blocks) and class 2 (at most 64 rows: 2 blocks), so that an
// expert's short last tile costs about a quarter of a full one instead of
// a whole one.  Within a class the tiles are listed in groups of QPGM row
// tiles, all column tiles of a group before the next (row tile fastest),
// so that tiles next to each other in the list share weight and activation
// tiles.  Each class list is cut into 8 contiguous chunks, one per XCD
// (workgroup b runs on XCD b % 8); XCD x's list is its class 0 chunk, then
// its class 1 and class 2 chunks, and its workgroups take that list round
// robin (workgroup j of the XCD: entries j, j + cu_per_xcd, ...).  The
// workgroups resident on one XCD therefore work on neighbouring tiles at
// any time, and the cheap tiles come last, after the full ones, filling
// the end of the schedule.
constexpr float QCOST[3] = {1.0f, 0.6f, 0.4f};   // rough cost of a tile of each class

__device__ __forceinline__ int q_class(int rows) { return rows > 128 ? 0 : rows > 64 ? 1 : 2; }

// Row tiles of class c per expert: class 0 takes the full tiles and a last
// tile of more than 128 rows; classes 1 and 2 a last tile of their size.
__device__ __forceinline__ int q_class_tiles(int count, int c) {
    const int full = count / QBM, tail = count % QBM;
    return (c == 0 ? full : 0) + (tail > 0 && q_class(tail) == c ? 1 : 0);
}

// Row tile mt of class c -> (expert, first row, end of the expert's rows).
__device__ __forceinline__ void q_row_tile(const int32_t *counts, const int32_t *offsets, int E,
                                           int c, int mt, int &e_out, int &row0, int &row_end) {
    int acc = 0;
    for (int e = 0; e < E; ++e) {
        const int cnt = counts[e];
        const int n = q_class_tiles(cnt, c);
        if (mt < acc + n) {
            const int k = mt - acc;
            e_out = e;
            row0 = offsets[e] + (c == 0 && k < cnt / QBM ? k : cnt / QBM) * QBM;
            row_end = offsets[e] + cnt;
            return;
        }
        acc += n;
    }
    e_out = 0;
    row0 = row_end = 0;   // not reached for mt < the class's tile count
}

// Entry `idx` of a class list with n_tiles column tiles: (row tile, column tile).
__device__ __forceinline__ void q_group_pos(int idx, int m_c, int n_tiles, int &mt, int &nt) {
    const int group = idx / (QPGM * n_tiles);
    const int first = group * QPGM;
    const int gm = min(QPGM, m_c - first);
    const int within = idx - group * QPGM * n_tiles;
    mt = first + within % gm;
    nt = within / gm;
}

// Estimated time of the schedule, in full-tile units, for tiles cut in S
// parts along K: the load of workgroup 0 of the busiest XCD (it takes
// entries 0, cpx, 2 cpx, ... of its XCD's list, the most and the costliest
// of any workgroup there), each entry costing its class's share over S
// plus a fixed per-tile overhead, and a tenth of a tile per extra part for
// writing and re-reading the fp32 partial sums.
__device__ __forceinline__ float q_makespan(const int (&m)[3], int n_cols, int S, int cpx) {
    float worst = 0.0f;
    for (int x = 0; x < 8; ++x) {
        int before = 0, k_done = 0;
        float load = 0.0f;
        for (int c = 0; c < 3; ++c) {
            const int64_t T = (int64_t)m[c] * n_cols * S;
            const int len = (int)(T * (x + 1) / 8 - T * x / 8);
            before += len;
            const int k_end = (before + cpx - 1) / cpx;   // entries k cpx < before
            load += (float)(k_end - k_done) * (QCOST[c] / S + 0.03f);
            k_done = k_end;
        }
        worst = fmaxf(worst, load);
    }
    return worst + 0.1f * (S - 1);
}

// ---------------------------------------------------------------------------
// The tile body, for every product of the layer and its backward.
//
// Output tile: 256 rows x 256 columns (NMAT = 2: 128 columns of each of two
// matrices, paired column for column).  Modes (QMode):
//   BKC    B is K-contiguous: line n of B (a row of B^T) holds the reduction
//          index, staged and read like A (16-byte fragment reads); else B is
//          N-contiguous [K, N] (the weights' own layout), read with the
//          transpose read.
//   DUAL   the reduction runs over two operand pairs: (A, B0) for k < K1
//          and (A2, B2) for the next K1 (one product a B0^T + a2 B2^T).
//   GROUPK per-expert outputs reduced over the expert's rows: A and B are
//          K-contiguous copies [M or N lines, ldk] whose columns hold every
//          expert's rows padded to whole stages with zeros; the tile is
//          (expert, row tile over M, column tile over N) and C is
//          [E, M, N].  Otherwise tiles run over the expert-grouped rows of A
//          (row tiles of one expert) and the tile's expert selects B.
//   EPI    QE_SWIGLU: h = bf16(silu(a b0) * (a b1)) (GU: also g, u fp32);
//          QE_F32:    C = a b fp32 (KSPLIT: part p at C + p * part_stride);
//          QE_DSWIGLU: z = a b with a the routed rows' dy, da = w z (w the
//                     row's routing weight), then dg = da * u * silu'(g) and
//                     du = da * silu(g), bf16, with g, u fp32 inputs; also
//                     the row's h . z over the tile's columns (the
//                     routing-weight gradient dy . o = h . (dy W2^T), per
//                     column tile);
//          QE_DW:     C (and C2 for NMAT = 2) = the fp32 sums, [E, M, N].
enum { QE_SWIGLU = 0, QE_F32 = 1, QE_DSWIGLU = 2, QE_DW = 3 };

template <int NMAT_, int EPI_, bool GU_ = false, bool KSPLIT_ = false, bool BKC_ = false,
          bool DUAL_ = false, bool GROUPK_ = false>
struct QMode {
    static constexpr int NMAT = NMAT_, EPI = EPI_;
    static constexpr bool GU = GU_, KSPLIT = KSPLIT_, BKC = BKC_, DUAL = DUAL_, GROUPK = GROUPK_;
    static_assert(NMAT == 1 || NMAT == 2, "one or two weight matrices");
    static_assert(!GU || EPI == QE_SWIGLU, "g and u come with the SwiGLU epilogue");
    static_assert(EPI != QE_SWIGLU || NMAT == 2, "SwiGLU pairs two matrices");
    static_assert(!KSPLIT || EPI == QE_F32, "split reductions store fp32 sums");
    static_assert(!DUAL || (BKC && NMAT == 1), "the two-pair reduction takes K-contiguous B");
    static_assert(!GROUPK || (BKC && EPI == QE_DW), "per-expert reductions store weight sums");
};

struct QSlots {
    uint8_t *a0, *a1, *b0, *b1, *b2;
};

// Arguments of one product (element strides).
//   A   [a_lines, lda] (grouped rows x K, or GROUPK: M lines x ldk).
//   B0, B1: N-contiguous [E, K, N]; K-contiguous [E, N, ldb] (GROUPK: [N, ldk],
//       no expert offset).  A2, B2 the second pair of DUAL (like A, B0).
//   C, C2 outputs, N columns per row (per matrix).
struct QArgs {
    const uint16_t *A, *B0, *B1, *A2, *B2;
    void *C, *C2;
    int K, N, M;         // reduction length (stages x 64; DUAL: 2 K1), columns, GROUPK rows
    int a_lines, lda, ldb, K1;
    const float *g_in, *u_in;
    const float *w_row;      // QE_DSWIGLU: routing weight of each grouped row
    const uint16_t *h_in;    // QE_DSWIGLU: h [rows, N]
    float *dw_part;          // QE_DSWIGLU: per-row partial sums of h . z, [rows, N / 256]
    float *g_out, *u_out;
    size_t part_stride;
};

// One tile of work: class c (32-row blocks per wavefront 8 >> c), expert
// e, rows row0 .. (stored up to row_end; GROUPK: M lines row0 .. + 256),
// first column n0, reduction stages kt0 .. kt0 + nk (GROUPK: kt0 is the
// expert's first padded stage), K part `part`.
struct QTile {
    int c, e, row0, row_end, n0, kt0, nk, part;
};

// ---- global -> LDS copies of one tile (1 KiB instructions: 64 lanes x 16 B).
// K-contiguous operand (A always, B with BKC): a stage is 256 lines x 64
// K values, 32 instructions of 8 lines; instruction g = lines 8 g ..
// 8 g + 7, lane l line 8 g + l / 8, LDS chunk l % 8 = K chunk c ^
// aswz(line).  A's 32 MBE lines are MBE instructions per wavefront.
// Weights, 32 instructions per stage, 8 per wavefront.
//   N-contiguous, NMAT = 1: instruction g holds K rows 2 g, 2 g + 1 (512 B
//   each), lane l row 2 g + l / 32, LDS chunk l % 32 = column chunk
//   c ^ bswz1(row).  NMAT = 2: instructions 0..15 the first sub-tile,
//   16..31 the second (waves 0, 1 and 2, 3), each 4 K rows of 256 B,
//   lane l row 4 (g % 16) + l / 16, LDS chunk l % 16 = c ^ bswz2(row).
//   K-contiguous: like A, lines n0 .. n0 + 255 (NMAT = 2: lines 0..127
//   of the stage from B0, 128..255 from B1, waves 0, 1 and 2, 3).
// Copies of stage s are clamped to the last stage (harmless re-reads).
// K offsets: K-contiguous operands advance 64 elements per stage, the
// N-contiguous weights 64 rows.
template <typename Mode, int MBE>
struct QLoad {
    static constexpr int NMAT = Mode::NMAT;
    static constexpr bool BKC = Mode::BKC, DUAL = Mode::DUAL, GROUPK = Mode::GROUPK;
    __amdgpu_buffer_rsrc_t ra, ra2, rb, rb2;
    uint32_t a_vo[MBE], b_vo[8];
    int wave, kt0, nk, K1, N;

    __device__ __forceinline__ QLoad(const QArgs &g, const QTile &t) {
        const int tid = q_tid(), lane = tid & 63;
        wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        kt0 = t.kt0;
        nk = t.nk;
        K1 = g.K1;
        N = g.N;
        ra = q_rsrc(g.A, (uint32_t)((size_t)g.a_lines * g.lda * 2));
        ra2 = ra;
        if constexpr (DUAL) ra2 = q_rsrc(g.A2, (uint32_t)((size_t)g.a_lines * g.lda * 2));
#pragma unroll
        for (int j = 0; j < MBE; ++j) {
            const int r = 8 * (wave * MBE + j) + (lane >> 3);
            const int c = (lane & 7) ^ q_aswz(r);
            a_vo[j] = (uint32_t)(((size_t)(t.row0 + r) * g.lda + c * 8) * 2);
        }
        const uint16_t *Bw = (NMAT == 2 && wave >= 2) ? g.B1 : g.B0;
        size_t b_mat = 0;
        uint32_t b_bytes;
        if constexpr (GROUPK) {
            b_bytes = (uint32_t)((size_t)N * g.ldb * 2);
        } else if constexpr (BKC) {
            b_mat = (size_t)t.e * N * g.ldb;
            b_bytes = (uint32_t)((size_t)N * g.ldb * 2);
        } else {
            b_mat = (size_t)t.e * g.K * N;
            b_bytes = (uint32_t)((size_t)g.K * N * 2);
        }
        rb = q_rsrc(Bw + b_mat, b_bytes);
        rb2 = rb;
        if constexpr (DUAL) rb2 = q_rsrc(g.B2 + b_mat, b_bytes);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if constexpr (BKC) {
                const int gi = wave * 8 + j;
                const int r = 8 * gi + (lane >> 3);                    // line of the stage
                const int c = (lane & 7) ^ q_aswz(r);
                const int line = NMAT == 2 ? t.n0 + (r & 127) : t.n0 + r;
                b_vo[j] = (uint32_t)(((size_t)line * g.ldb + c * 8) * 2);
            } else {
                int r, c;
                if constexpr (NMAT == 2) {
                    r = 4 * (((wave & 1) << 3) + j) + (lane >> 4);
                    c = (lane & 15) ^ q_bswz2(r);
                } else {
                    r = 2 * (wave * 8 + j) + (lane >> 5);
                    c = (lane & 31) ^ q_bswz1(r);
                }
                b_vo[j] = (uint32_t)(((size_t)r * N + t.n0 + c * 8) * 2);
            }
        }
    }
    __device__ __forceinline__ int b_dst(int j) const {
        if constexpr (NMAT == 2 && !BKC)
            return (wave >> 1) * (QSLOT / 2) + (((wave & 1) << 3) + j) * 1024;
        else
            return (wave * 8 + j) * 1024;
    }
    __device__ __forceinline__ void a_copy(uint8_t *slot, int s, int j) const {
        const int k0 = (kt0 + min(s, nk - 1)) * QBK;
        if constexpr (DUAL) {
            if (k0 >= K1) {
                q_dma(ra2, slot + (wave * MBE + j) * 1024, a_vo[j], (uint32_t)((k0 - K1) * 2));
                return;
            }
        }
        q_dma(ra, slot + (wave * MBE + j) * 1024, a_vo[j], (uint32_t)(k0 * 2));
    }
    __device__ __forceinline__ void b_copy(uint8_t *slot, int s, int j) const {
        const int k0 = (kt0 + min(s, nk - 1)) * QBK;
        if constexpr (BKC) {
            if constexpr (DUAL) {
                if (k0 >= K1) {
                    q_dma(rb2, slot + b_dst(j), b_vo[j], (uint32_t)((k0 - K1) * 2));
                    return;
                }
            }
            q_dma(rb, slot + b_dst(j), b_vo[j], (uint32_t)(k0 * 2));
        } else {
            q_dma(rb, slot + b_dst(j), b_vo[j], (uint32_t)((size_t)k0 * N * 2));
        }
    }
    // The copies of stages 0 and 1: activations of stage 0, weights of
    // stages 0 and 1, activations of stage 1 (MBE + 16 + MBE instructions).
    __device__ __forceinline__ void prologue(const QSlots &S) const {
#pragma unroll
        for (int j = 0; j < MBE; ++j) a_copy(S.a0, 0, j);
#pragma unroll
        for (int j = 0; j < 8; ++j) b_copy(S.b0, 0, j);
#pragma unroll
        for (int j = 0; j < 8; ++j) b_copy(S.b1, 1, j);
#pragma unroll
        for (int j = 0; j < MBE; ++j) a_copy(S.a1, 1, j);
    }
};

// 4 x 4 transpose across the lanes of a quad (DPP quad permutations):
// before, lane p of the quad holds v[k] = element (row k, column p); after,
// v[k] = element (row p, column k).  Two butterfly stages (partner lanes
// p ^ 1, then p ^ 2).
__device__ __forceinline__ void q_quad_transpose(float (&v)[4], int p) {
    auto swap = [&](int k, int s, int ctrl) Q_INLINE {
        const bool hi = (p & s) != 0;
        const float x = hi ? v[k] : v[k + s];
        float y;
        if (ctrl == 0xB1)
            y = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1,
                                                                    0xF, 0xF, false));
        else
            y = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E,
                                                                    0xF, 0xF, false));
        if (hi) v[k] = y;
        else v[k + s] = y;
    };
    swap(0, 1, 0xB1);
    swap(2, 1, 0xB1);
    swap(0, 2, 0x4E);
    swap(1, 2, 0x4E);
}

template <typename Mode, int MBE>
__device__ __forceinline__ void q_tile_run(const QSlots &S, const QArgs &g, const QTile &t) {
    constexpr int NMAT = Mode::NMAT, EPI = Mode::EPI;
    constexpr bool BKC = Mode::BKC;
    const int N = g.N;
    // The tile's fields are uniform across the workgroup, so they go to
    // scalar registers; held in vector registers they were spilled and
    // reloaded from scratch in the epilogue.
    const int e = __builtin_amdgcn_readfirstlane(t.e);
    const int row0 = __builtin_amdgcn_readfirstlane(t.row0);
    const int row_end = __builtin_amdgcn_readfirstlane(t.row_end);
    const int n0 = __builtin_amdgcn_readfirstlane(t.n0);
    const int nk = __builtin_amdgcn_readfirstlane(t.nk);
    auto slot_a = [&](auto i_c) Q_INLINE {
        constexpr int i = decltype(i_c)::value % QAS;
        if constexpr (i == 0) return S.a0;
        else return S.a1;
    };
    auto slot_b = [&](auto i_c) Q_INLINE {
        constexpr int i = decltype(i_c)::value % QBS;
        if constexpr (i == 0) return S.b0;
        else if constexpr (i == 1) return S.b1;
        else return S.b2;
    };

    const int tid = q_tid(), lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    const QLoad<Mode, MBE> L(g, t);
    auto a_copy = [&](uint8_t *slot, int s, int j) Q_INLINE { L.a_copy(slot, s, j); };
    auto b_copy = [&](uint8_t *slot, int s, int j) Q_INLINE { L.b_copy(slot, s, j); };

    // ---- fragment reads.
    // A block i, step h (16 K values): line 32 i + l % 32, K chunk 2 h + l / 32
    // (and B block j the same way with BKC, lines of the block's columns).
    int a_off[4];
#pragma unroll
    for (int h = 0; h < 4; ++h)
        a_off[h] = (lane & 31) * 128 + (((2 * h + (lane >> 5)) ^ q_aswz(lane & 31)) << 4);
    // B block j (transpose read): lane l of 16-lane group G gets column
    // 16 (G & 1) + l % 16 of K rows 8 (G >> 1) + 4 u + 0..3 (u = 0, 1 the two
    // halves of its 8 K values).
    int b_off[2][2];
    if constexpr (!BKC) {
        const int G = lane >> 4, ii = (lane & 15) >> 2, q = lane & 3;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int r = 8 * (G >> 1) + 4 * u + ii;   // + 16 h
                if constexpr (NMAT == 2) {
                    const int n = wave * 32 + 16 * (G & 1) + 4 * q;
                    b_off[j][u] = j * (QSLOT / 2) + r * 256 + (((n >> 3) ^ q_bswz2(r)) << 4) +
                                  (n & 7) * 2;
                } else {
                    const int n = wave * 64 + 32 * j + 16 * (G & 1) + 4 * q;
                    b_off[j][u] = r * 512 + (((n >> 3) ^ q_bswz1(r)) << 4) + (n & 7) * 2;
                }
            }
    }
    // With BKC, block j's first line inside the stage.
    auto bk_line = [&](int j) Q_INLINE {
        return NMAT == 2 ? j * 128 + wave * 32 : wave * 64 + j * 32;
    };
    constexpr int BSTEP = NMAT == 2 ? 16 * 256 : 16 * 512;   // bytes per 16 K rows

    bf16x8_t fa[2][MBE];
    s16x4_t fb[2][2][2];       // transpose-read halves
    bf16x8_t fk[2][2];         // K-contiguous B fragments
    f32x16_t acc[MBE][2];
#pragma unroll
    for (int i = 0; i < MBE; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

    // Read items of a step into buffer `buf`, in the order the next step's
    // MFMAs use them: B block 0, the A blocks, B block 1 (a transpose-read
    // B block is two items, its halves).
    constexpr int NBI = BKC ? 1 : 2;                 // items per B block
    constexpr int NR = MBE + 2 * NBI;
    auto read_item = [&](auto buf_c, auto r_c, const uint8_t *sa, const uint8_t *sb,
                         int h) Q_INLINE {
        constexpr int bf = decltype(buf_c)::value, r = decltype(r_c)::value;
        if constexpr (r >= NBI && r < MBE + NBI) {
            fa[bf][r - NBI] = __builtin_bit_cast(
                bf16x8_t, *reinterpret_cast<const uint4 *>(sa + a_off[h] + (r - NBI) * 32 * 128));
        } else {
            constexpr int j = r < NBI ? 0 : 1, u = r < NBI ? r : r - MBE - NBI;
            if constexpr (BKC) {
                fk[bf][j] = __builtin_bit_cast(
                    bf16x8_t, *reinterpret_cast<const uint4 *>(sb + a_off[h] + bk_line(j) * 128));
            } else {
                fb[bf][j][u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4_t *)(sb + b_off[j][u] + h * BSTEP));
            }
        }
    };
    // MFMA m of a step: block (i, j) = (m % MBE, m / MBE).
    constexpr int NM = 2 * MBE;
    auto mfma_item = [&](auto buf_c, auto m_c) Q_INLINE {
        constexpr int bf = decltype(buf_c)::value, m = decltype(m_c)::value;
        constexpr int j = m / MBE, i = m % MBE;
        bf16x8_t b;
        if constexpr (BKC)
            b = fk[bf][j];
        else
            b = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(fb[bf][j][0], fb[bf][j][1],
                                                                     0, 1, 2, 3, 4, 5, 6, 7));
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[bf][i], b, acc[i][j], 0, 0, 0);
    };

    // Stage s (ring position t = s mod QU), steps h = 0..3.  Copies issued
    // in the window that follows the barrier of stage s - 1 (step (s-1, 3)
    // after the barrier, steps (s, 0) and (s, 1)): activations of stage
    // s + 1, then weights of stage s + 2, into the slots stage s - 1 has
    // left.  At the barrier of stage s (in its step 3) the activations and
    // weights of stage s + 1 must have landed; only the 8 weight copies of
    // stage s + 2 may still be in flight.  Each step's items (the next
    // step's fragment reads, then its copies) are spread evenly over its
    // MFMAs.
    auto stage = [&](auto t_c, int s) Q_INLINE {
        constexpr int tt = decltype(t_c)::value;
        const uint8_t *sa = slot_a(t_c), *sb = slot_b(t_c);
        const uint8_t *sa_n = slot_a(std::integral_constant<int, tt + 1>{});
        const uint8_t *sb_n = slot_b(std::integral_constant<int, tt + 1>{});
        uint8_t *wa = slot_a(std::integral_constant<int, tt + 2>{});   // activations, stage s + 2
        uint8_t *wb = slot_b(std::integral_constant<int, tt + 2>{});   // weights, stage s + 2
        q_for<4>([&](auto h_c) Q_INLINE {
            constexpr int h = decltype(h_c)::value;
            constexpr int cur = h & 1, nxt = cur ^ 1;
            constexpr int NC = h == 3 ? MBE : h < 2 ? 4 : 0;    // copies in this step
            constexpr int NI = NR + NC;
            q_for<NM>([&](auto m_c) Q_INLINE {
                constexpr int m = decltype(m_c)::value;
                mfma_item(std::integral_constant<int, cur>{}, m_c);
                if constexpr (h == 3 && m == 0) q_barrier<8>();
                constexpr int lo = m * NI / NM, hi = (m + 1) * NI / NM;
                q_for<NI>([&](auto it_c) Q_INLINE {
                    constexpr int it = decltype(it_c)::value;
                    if constexpr (it >= lo && it < hi) {
                        if constexpr (it < NR) {
                            if constexpr (h < 3)
                                read_item(std::integral_constant<int, nxt>{}, it_c, sa, sb, h + 1);
                            else
                                read_item(std::integral_constant<int, nxt>{},
                                          std::integral_constant<int, it>{}, sa_n, sb_n, 0);
                        } else if constexpr (h == 3) {
                            a_copy(wa, s + 2, it - NR);
                        } else {
                            b_copy(wb, s + 2, it - NR + 4 * h);
                        }
                    }
                });
                __builtin_amdgcn_sched_barrier(0);
            });
        });
    };

    if (nk > 0) {
        // Prologue: what the windows of stages -2 and -1 would have issued,
        // then the fragments of step (0, 0).
        L.prologue(S);
        q_barrier<8 + MBE>();
        q_for<NR>([&](auto r_c) Q_INLINE {
            read_item(std::integral_constant<int, 0>{}, r_c,
                      slot_a(std::integral_constant<int, 0>{}),
                      slot_b(std::integral_constant<int, 0>{}), 0);
        });

        int kt = 0;
        for (; kt + QU <= nk; kt += QU)
            q_for<QU>([&](auto t_c) Q_INLINE { stage(t_c, kt + decltype(t_c)::value); });
        q_for<QU - 1>([&](auto t_c) Q_INLINE {
            if (kt + decltype(t_c)::value < nk) stage(t_c, kt + decltype(t_c)::value);
        });
        // Every copy has landed and every wavefront is done with the rings
        // before the next tile's prologue refills them.
        q_barrier<0>();
    }

    // The epilogues take the lane index afresh from the hardware (mbcnt):
    // the one computed at the kernel's start is kept in scratch through
    // the K loop, and each reload's wait (vmcnt, in order) would also wait
    // for the epilogue's prefetched loads.
    const int ln = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    // 32x32 accumulator layout: value q of lane l is row 8 (q / 4) + 4 (l / 32)
    // + q % 4, column l % 32 of the block.
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    const int odd = ln & 1;
    // Store two bf16 values of this lane's column, rows q and q + 1 (v0, v1),
    // as 4-byte column pairs: lanes l and l ^ 1 hold neighbouring columns
    // of the same rows and swap one value (a DPP quad permutation), so that
    // the even lane stores row q and the odd lane row q + 1 (row_q: this
    // lane's row q; col: this lane's column).  The pair is rounded to bf16
    // (nearest even) by one v_cvt_pk_bf16_f32 before the swap.
    auto store_pair = [&](uint16_t *dst, int row_q, int col, float v0, float v1) Q_INLINE {
        const uint32_t hp =
            __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{v0, v1}, bf16x2_t));
        const uint32_t x = odd ? hp : (hp >> 16);
        const uint32_t y = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);
        const uint32_t packed =
            odd ? ((y & 0xffffu) | (hp & 0xffff0000u)) : ((hp & 0xffffu) | (y << 16));
        const int row = row_q + odd;
        if (row < row_end)
            __builtin_nontemporal_store(
                packed, reinterpret_cast<uint32_t *>(dst + (size_t)row * N + col - odd));
    };
    if constexpr (EPI == QE_SWIGLU && !Mode::GU) {
        // h = silu(g) u, silu(g) = g / (1 + 2^(-g log2 e)) with the hardware
        // exp2 and reciprocal, stored as bf16 column pairs.  (Quad-transposed
        // 8-byte row segments, as the GU form below stores, measured 2 %
        // slower here: the transposes lengthen the epilogue more than the
        // halved store count saves.)
        uint16_t *H = static_cast<uint16_t *>(g.C);
        const int col = n0 + wave * 32 + (ln & 31);
#pragma unroll
        for (int i = 0; i < MBE; ++i)
#pragma unroll
            for (int q = 0; q < 16; q += 2) {
                auto hval = [&](int qq) Q_INLINE {
                    const float gv = acc[i][0][qq], uv = acc[i][1][qq];
                    const float den = 1.0f + __builtin_amdgcn_exp2f(gv * -1.44269504088896341f);
                    return gv * __builtin_amdgcn_rcpf(den) * uv;
                };
                const int row_q = row0 + i * 32 + 8 * (q >> 2) + 4 * (ln >> 5) + (q & 3);
                store_pair(H, row_q, col, hval(q), hval(q + 1));
            }
    } else if constexpr (EPI == QE_SWIGLU) {
        // GU: h as above, and g and u themselves in fp32.  Each 4 x 4 block
        // of h, g and u is quad-transposed so that a lane holds 4
        // consecutive columns of one row: h is stored as 8-byte row segments
        // (4 bf16, rounded to nearest even), g and u as 16-byte segments (a
        // quarter of the store instructions of column stores).
        typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
        uint16_t *H = static_cast<uint16_t *>(g.C);
        const int c4 = n0 + wave * 32 + ((ln & 31) & ~3);
#pragma unroll
        for (int i = 0; i < MBE; ++i)
#pragma unroll
            for (int grp = 0; grp < 4; ++grp) {
                float gv[4], uv[4], hv[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    gv[k] = acc[i][0][4 * grp + k];
                    uv[k] = acc[i][1][4 * grp + k];
                    const float den = 1.0f + __builtin_amdgcn_exp2f(gv[k] * -1.44269504088896341f);
                    hv[k] = gv[k] * __builtin_amdgcn_rcpf(den) * uv[k];
                }
                q_quad_transpose(hv, ln & 3);
                q_quad_transpose(gv, ln & 3);
                q_quad_transpose(uv, ln & 3);
                const int row = row0 + i * 32 + 8 * grp + 4 * (ln >> 5) + (ln & 3);
                if (row < row_end) {
                    const size_t o = (size_t)row * N + c4;
                    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
                    __builtin_nontemporal_store(
                        __builtin_bit_cast(u32x2_t, __builtin_convertvector(
                                                        f32x4_t{hv[0], hv[1], hv[2], hv[3]},
                                                        bf16x4_t)),
                        reinterpret_cast<u32x2_t *>(H + o));
                    *reinterpret_cast<f32x4_t *>(g.g_out + o) = f32x4_t{gv[0], gv[1], gv[2], gv[3]};
                    *reinterpret_cast<f32x4_t *>(g.u_out + o) = f32x4_t{uv[0], uv[1], uv[2], uv[3]};
                }
                __builtin_amdgcn_sched_barrier(0);
            }
    } else if constexpr (EPI == QE_DSWIGLU) {
        // z = dy W2^T for the routed rows (the accumulators), da = w z,
        // dg = da u s (1 + g (1 - s)), du = da g s with s = sigmoid(g).
        // Each 4 x 4 block of z is quad-transposed so that a lane holds 4
        // consecutive columns of one row: g, u, h and the row's weight are
        // read and dg, du written as row segments, and the next block's
        // loads are issued before the current block is computed (rows
        // clamped into the tile).  The routing-weight gradient's part from
        // this tile, sum over its 256 columns of h z, is reduced in a fixed
        // order: a lane's 4 columns of both 32-column blocks, the 8 lanes
        // of the row (xor 4, 8, 16), then the 4 wavefronts through LDS
        // ((w0 + w1) + (w2 + w3)).
        uint16_t *dG = static_cast<uint16_t *>(g.C);
        uint16_t *dU = static_cast<uint16_t *>(g.C2);
        typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
        constexpr int NBLK = MBE * 2;
        float4 gb[2][4], ub[2][4];
        uint2 hb[2][4];
        float wr[2][4];
        float hz[4];
        float *red = reinterpret_cast<float *>(S.b2);   // [4 wavefronts][256 rows]
        auto blk_row = [&](int i, int grp) Q_INLINE {
            return row0 + i * 32 + 8 * grp + 4 * (ln >> 5) + (ln & 3);
        };
        auto blk_col = [&](int j) Q_INLINE { return n0 + wave * 64 + j * 32 + ((ln & 31) & ~3); };
        auto load_blk = [&](auto b_c, auto buf_c) Q_INLINE {
            constexpr int b = decltype(b_c)::value, bf = decltype(buf_c)::value;
            constexpr int i = b / 2, j = b % 2;
#pragma unroll
            for (int grp = 0; grp < 4; ++grp) {
                const int r = min(blk_row(i, grp), row_end - 1);
                const size_t o = (size_t)r * N + blk_col(j);
                gb[bf][grp] = *reinterpret_cast<const float4 *>(g.g_in + o);
                ub[bf][grp] = *reinterpret_cast<const float4 *>(g.u_in + o);
                hb[bf][grp] = *reinterpret_cast<const uint2 *>(g.h_in + o);
                wr[bf][grp] = g.w_row[r];
            }
        };
        load_blk(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
        q_for<NBLK>([&](auto b_c) Q_INLINE {
            constexpr int b = decltype(b_c)::value, bf = b & 1;
            constexpr int i = b / 2, j = b % 2;
            if constexpr (b + 1 < NBLK)
                load_blk(std::integral_constant<int, b + 1>{}, std::integral_constant<int, bf ^ 1>{});
#pragma unroll
            for (int grp = 0; grp < 4; ++grp) {
                float v[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) v[k] = acc[i][j][4 * grp + k];
                q_quad_transpose(v, ln & 3);
                const float gg[4] = {gb[bf][grp].x, gb[bf][grp].y, gb[bf][grp].z, gb[bf][grp].w};
                const float uu[4] = {ub[bf][grp].x, ub[bf][grp].y, ub[bf][grp].z, ub[bf][grp].w};
                const float hh[4] = {bf16_to_f32(hb[bf][grp].x & 0xffffu),
                                     bf16_to_f32(hb[bf][grp].x >> 16),
                                     bf16_to_f32(hb[bf][grp].y & 0xffffu),
                                     bf16_to_f32(hb[bf][grp].y >> 16)};
                const float hs = ((hh[0] * v[0] + hh[1] * v[1]) + hh[2] * v[2]) + hh[3] * v[3];
                if constexpr (j == 0) hz[grp] = hs;
                else hz[grp] += hs;
                f32x4_t dg, du;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const float da = wr[bf][grp] * v[k];
                    const float sg = __builtin_amdgcn_rcpf(
                        1.0f + __builtin_amdgcn_exp2f(gg[k] * -1.44269504088896341f));
                    dg[k] = da * uu[k] * sg * (1.0f + gg[k] * (1.0f - sg));
                    du[k] = da * gg[k] * sg;
                }
                const int row = blk_row(i, grp);
                if (row < row_end) {
                    const size_t o = (size_t)row * N + blk_col(j);
                    *reinterpret_cast<uint2 *>(dG + o) =
                        __builtin_bit_cast(uint2, __builtin_convertvector(dg, bf16x4_t));
                    *reinterpret_cast<uint2 *>(dU + o) =
                        __builtin_bit_cast(uint2, __builtin_convertvector(du, bf16x4_t));
                }
                if constexpr (j == 1) {
                    float t = hz[grp];
                    t += __shfl_xor(t, 4, 64);
                    t += __shfl_xor(t, 8, 64);
                    t += __shfl_xor(t, 16, 64);
                    if ((ln & 28) == 0)
                        red[wave * 256 + i * 32 + 8 * grp + 4 * (ln >> 5) + (ln & 3)] = t;
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        });
        // The rings are idle after the K loop's last barrier; the next
        // tile refills slot b2 only after its prologue barrier, and the
        // barrier below keeps every wavefront's reads of red before it.
        __syncthreads();
        const int tid = threadIdx.x;
        if (tid < 32 * MBE && row0 + tid < row_end) {
            const float t = (red[tid] + red[256 + tid]) + (red[512 + tid] + red[768 + tid]);
            g.dw_part[(size_t)(row0 + tid) * (N / QBN) + n0 / QBN] = t;
        }
        __syncthreads();
    } else if constexpr (EPI == QE_F32) {
        // fp32 sums as 16-byte row segments: each 4 x 4 block of a lane
        // quad is quad-transposed so that a lane holds 4 consecutive
        // columns of one row (a quarter of the store instructions of
        // 4-byte column stores).
        static_assert(NMAT == 1, "fp32 stores of one matrix");
        float *O = static_cast<float *>(g.C) + (Mode::KSPLIT ? (size_t)t.part * g.part_stride : 0);
#pragma unroll
        for (int i = 0; i < MBE; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int grp = 0; grp < 4; ++grp) {
                    float v[4];
#pragma unroll
                    for (int k = 0; k < 4; ++k) v[k] = acc[i][j][4 * grp + k];
                    q_quad_transpose(v, ln & 3);
                    const int row = row0 + i * 32 + 8 * grp + 4 * (ln >> 5) + (ln & 3);
                    const int c4 = n0 + wave * 64 + j * 32 + ((ln & 31) & ~3);
                    if (row < row_end)
                        *reinterpret_cast<f32x4_t *>(O + (size_t)row * N + c4) =
                            f32x4_t{v[0], v[1], v[2], v[3]};
                    __builtin_amdgcn_sched_barrier(0);
                }
    } else {
        // The fp32 sums of expert e (C[e], and C2[e] for the second matrix,
        // [M, N]) as 16-byte row segments (quad transposes), streamed
        // (non-temporal: nothing reads them back here).
        float *O0 = static_cast<float *>(g.C) + (size_t)e * g.M * N;
        float *O1 = NMAT == 2 ? static_cast<float *>(g.C2) + (size_t)e * g.M * N : O0;
#pragma unroll
        for (int i = 0; i < MBE; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int grp = 0; grp < 4; ++grp) {
                    float v[4];
#pragma unroll
                    for (int k = 0; k < 4; ++k) v[k] = acc[i][j][4 * grp + k];
                    q_quad_transpose(v, ln & 3);
                    const int row = row0 + i * 32 + 8 * grp + 4 * (ln >> 5) + (ln & 3);
                    const int c4 = (NMAT == 2 ? n0 + wave * 32 : n0 + wave * 64 + j * 32) +
                                   ((ln & 31) & ~3);
                    const f32x4_t out = {v[0], v[1], v[2], v[3]};
                    __builtin_nontemporal_store(
                        out, reinterpret_cast<f32x4_t *>((j == 1 ? O1 : O0) + (size_t)row * N + c4));
                    __builtin_amdgcn_sched_barrier(0);
                }
    }
}

// Persistent body over the expert-grouped rows of A (every product except
// the weight gradients).
template <typename Mode>
__device__ __forceinline__ void q_body(const QArgs &g, const int32_t *__restrict__ counts,
                                       const int32_t *__restrict__ offsets, int E, int parts,
                                       int cu_per_xcd, int *__restrict__ parts_out) {
    constexpr int BNM = QBN / Mode::NMAT;
    const int n_cols = g.N / BNM;
    int m[3] = {0, 0, 0};
    for (int i = 0; i < E; ++i) {
        const int c = counts[i];
#pragma unroll
        for (int k = 0; k < 3; ++k) m[k] += q_class_tiles(c, k);
    }
    if constexpr (Mode::KSPLIT) {
        if (parts == 0) {
            parts = 1;
            float best = q_makespan(m, n_cols, 1, cu_per_xcd);
            for (int S = 2; S <= QMAXSPLIT && S <= g.K / QBK; ++S) {
                const float t = q_makespan(m, n_cols, S, cu_per_xcd);
                if (t < best) { best = t; parts = S; }
            }
            if (blockIdx.x == 0 && threadIdx.x == 0) *parts_out = parts;
        }
    }
    const int n_tiles = Mode::KSPLIT ? n_cols * parts : n_cols;

    __shared__ __attribute__((aligned(1024))) uint8_t sa0[QSLOT];
    __shared__ __attribute__((aligned(1024))) uint8_t sa1[QSLOT];
    __shared__ __attribute__((aligned(1024))) uint8_t sb0[QSLOT];
    __shared__ __attribute__((aligned(1024))) uint8_t sb1[QSLOT];
    __shared__ __attribute__((aligned(1024))) uint8_t sb2[QSLOT];
    const QSlots S{sa0, sa1, sb0, sb1, sb2};

    const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
    int lo[3], len[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const int64_t T = (int64_t)m[k] * n_tiles;
        lo[k] = (int)(T * xcd / 8);
        len[k] = (int)(T * (xcd + 1) / 8) - lo[k];
    }
    const int total = len[0] + len[1] + len[2];
    const int nk_all = g.K / QBK;
    for (int idx = j; idx < total; idx += cu_per_xcd) {
        QTile t{};
        int c = 0, f = idx;
        if (f >= len[0]) {
            f -= len[0];
            c = 1;
            if (f >= len[1]) {
                f -= len[1];
                c = 2;
            }
        }
        int mt, nt;
        q_group_pos(lo[c] + f, m[c], n_tiles, mt, nt);
        t.c = c;
        q_row_tile(counts, offsets, E, c, mt, t.e, t.row0, t.row_end);
        t.kt0 = 0;
        t.nk = nk_all;
        if constexpr (Mode::KSPLIT) {
            t.part = nt / n_cols;
            nt -= t.part * n_cols;
            t.kt0 = (int)((int64_t)nk_all * t.part / parts);
            t.nk = (int)((int64_t)nk_all * (t.part + 1) / parts) - t.kt0;
        }
        t.n0 = nt * BNM;
        if (c == 0)
            q_tile_run<Mode, 8>(S, g, t);
        else if (c == 1)
            q_tile_run<Mode, 4>(S, g, t);
        else
            q_tile_run<Mode, 2>(S, g, t);
    }
}

// Persistent body of the weight gradients: tiles (expert, row tile over M,
// column tile over N), each reduced over its expert's rows (the expert's
// padded stages).  The flat list is ordered expert after expert, in groups
// of QPGM row tiles (row tile fastest); a tile's cost is its stage count
// plus two, and each XCD takes a contiguous run of about an eighth of the
// total cost, taken round robin by its workgroups.
template <typename Mode>
__device__ __forceinline__ void q_body_dw(const QArgs &g, const int32_t *__restrict__ counts,
                                          int E, int cu_per_xcd) {
    constexpr int BNM = QBN / Mode::NMAT;
    const int n_cols = g.N / BNM, m_tiles = g.M / QBM;
    const int per_e = m_tiles * n_cols;

    __shared__ __attribute__((aligned(1024))) uint8_t sa0[QSLOT];
    __shared__ __attribute__((aligned(1024))) uint8_t sa1[QSLOT];
    __shared__ __attribute__((aligned(1024))) uint8_t sb0[QSLOT];
    __shared__ __attribute__((aligned(1024))) uint8_t sb1[QSLOT];
    __shared__ __attribute__((aligned(1024))) uint8_t sb2[QSLOT];
    const QSlots S{sa0, sa1, sb0, sb1, sb2};

    int64_t cost_total = 0;
    for (int i = 0; i < E; ++i) cost_total += (int64_t)per_e * ((counts[i] + QBK - 1) / QBK + 2);
    const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
    // First flat entry whose cost start is at or past cost_total * x / 8.
    auto boundary = [&](int x) Q_INLINE {
        const int64_t target = cost_total * x / 8;
        int64_t acc = 0;
        int base = 0;
        for (int i = 0; i < E; ++i) {
            const int64_t ct = (counts[i] + QBK - 1) / QBK + 2;
            const int64_t span = ct * per_e;
            if (acc + span > target) return base + (int)((target - acc + ct - 1) / ct);
            acc += span;
            base += per_e;
        }
        return base;
    };
    const int lo = boundary(xcd), hi = xcd == 7 ? E * per_e : boundary(xcd + 1);
    auto tile_at = [&](int idx) Q_INLINE {
        QTile t{};
        t.e = idx / per_e;
        int mt, nt;
        q_group_pos(idx - t.e * per_e, m_tiles, n_cols, mt, nt);
        int kstage = 0;
        for (int i = 0; i < t.e; ++i) kstage += (counts[i] + QBK - 1) / QBK;
        t.c = 0;
        t.row0 = mt * QBM;
        t.row_end = t.row0 + QBM;
        t.n0 = nt * BNM;
        t.kt0 = kstage;
        t.nk = (counts[t.e] + QBK - 1) / QBK;
        t.part = 0;
        return t;
    };
    for (int idx = lo + j; idx < hi; idx += cu_per_xcd) q_tile_run<Mode, 8>(S, g, tile_at(idx));
}

inline bool q_fits(int rows, int K, int N, int bnm) {
    return rows > 0 && K % QBK == 0 && K / QBK >= 1 && N % bnm == 0 &&
           (uint64_t)rows * K * 2 < ((uint64_t)1 << 32) &&
           (uint64_t)K * N * 2 < ((uint64_t)1 << 32);
}

// CUs per XCD of the current device (the persistent grid is 8 times that).
inline int q_cus_per_xcd() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return -1;
    return std::max(1, cus / 8);
}

}  // namespace
}  // namespace moe
