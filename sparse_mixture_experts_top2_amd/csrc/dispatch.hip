// Dispatch: group the kT (token, slot) assignments by expert, stably, and
// copy each token's row of x to its k grouped rows of xp.  This is the
// per-expert token batching that "Mixtral 8x7B -- The Evolving Transformer",
// section 05, says production stacks use in place of its per-expert mask
// loop; the order within an expert (token, then slot) is the order in which
// that loop visits the tokens.
//
// Kernel 1 (one workgroup of 16 wavefronts): wavefront w owns a contiguous
// run of assignments and walks it 64 at a time.  For each expert, a ballot
// of the lanes holding that expert gives the number of such assignments in
// the batch (popcount) and each lane's rank among them (popcount of the
// lower lanes).  Pass 1 counts per wavefront and expert; a scan over
// wavefronts and experts (in LDS) gives every wavefront's first rank in each
// expert and the offsets; pass 2 writes pos.  Lane order and wavefront order
// equal assignment order, so the grouping is stable and the integers are
// exact.  Two barriers in all, whatever E is.
// Kernel 2 (many workgroups): one wavefront per token copies the row with
// 16-byte loads and stores; it is bound by HBM (T*d*elem read, 2*T*d*elem
// written).
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kRankWaves = 16;

__device__ __forceinline__ int clamp_expert(int e, int E) {
    return (int)min((unsigned)e, (unsigned)(E - 1));
}

__global__ __launch_bounds__(kRankWaves * 64) void dispatch_rank_kernel(
    const int32_t *__restrict__ idx, int n_assign, int E, int k, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ pos, int32_t *__restrict__ src) {
    __shared__ int32_t wbase[kRankWaves][kMaxExperts];   // per-wavefront counts, then bases
    __shared__ int32_t ebase[kMaxExperts + 1];           // expert offsets
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint64_t lower = (1ull << lane) - 1ull;        // lanes below this one
    // Contiguous runs of whole 64-assignment batches, in wavefront order.
    const int batches = (n_assign + 63) / 64;
    const int per = (batches + kRankWaves - 1) / kRankWaves;
    const int a0 = min(n_assign, wave * per * 64), a1 = min(n_assign, a0 + per * 64);

    // The run is read kLoadBatches batches at a time, all loads issued
    // before any is used, so a pass costs one memory round trip per group
    // rather than one per batch.  Expert ids are clamped into [0, E) so that
    // a corrupt id can never send a row outside xp; valid ids are
    // unaffected; -1 marks lanes past the run.
    constexpr int kLoadBatches = 8;
    auto load_group = [&](int g0, int (&ev)[kLoadBatches]) {
#pragma unroll
        for (int b = 0; b < kLoadBatches; ++b) {
            const int a = g0 + b * 64 + lane;
            ev[b] = a < a1 ? clamp_expert(idx[a], E) : -1;
        }
    };
    // Pass 1: this wavefront's count per expert (lane e holds expert e).
    int my_count = 0;
    for (int g0 = a0; g0 < a1; g0 += kLoadBatches * 64) {
        int ev[kLoadBatches];
        load_group(g0, ev);
#pragma unroll
        for (int b = 0; b < kLoadBatches; ++b) {
            if (g0 + b * 64 >= a1) break;
            for (int x = 0; x < E; ++x) {
                const int c = __popcll(__ballot(ev[b] == x));
                if (lane == x) my_count += c;
            }
        }
    }
    if (lane < E) wbase[wave][lane] = my_count;
    __syncthreads();
    // Scan: for each expert, exclusive prefix over wavefronts; then the
    // exclusive prefix of the expert totals (wave 0, lane e = expert e).
    if (wave == 0) {
        int tot = 0;
        if (lane < E)
            for (int w = 0; w < kRankWaves; ++w) {
                const int c = wbase[w][lane];
                wbase[w][lane] = tot;
                tot += c;
            }
        int inc = tot;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int u = __shfl_up(inc, off, 64);
            if (lane >= off) inc += u;
        }
        if (lane < E) {
            counts[lane] = tot;
            offsets[lane] = inc - tot;
            ebase[lane] = inc - tot;
        }
        if (lane == E - 1) {
            offsets[E] = inc;
            ebase[E] = inc;
        }
    }
    __syncthreads();
    // Pass 2: rank of each assignment = expert offset + wavefront base +
    // assignments of the same expert earlier in this wavefront's run.
    // next[e] (this wavefront's row of LDS) is the next grouped row of
    // expert e; each batch reads it once per lane and lane e advances it.
    int32_t *next = wbase[wave];
    if (lane < E) next[lane] += ebase[lane];
    for (int g0 = a0; g0 < a1; g0 += kLoadBatches * 64) {
        int ev[kLoadBatches];
        load_group(g0, ev);
#pragma unroll
        for (int b = 0; b < kLoadBatches; ++b) {
            const int a = g0 + b * 64;
            if (a >= a1) break;
            uint64_t mine = 0;   // lanes holding this lane's expert
            int added = 0;       // lane e: assignments of expert e in the batch
            for (int x = 0; x < E; ++x) {
                const uint64_t m = __ballot(ev[b] == x);
                if (ev[b] == x) mine = m;
                if (lane == x) added = __popcll(m);
            }
            const int first = ev[b] >= 0 ? next[ev[b]] : 0;
            if (ev[b] >= 0) {
                const int p = first + __popcll(mine & lower);
                pos[a + lane] = p;
                if (src) src[p] = (a + lane) / k;   // token of grouped row p
            }
            if (lane < E) next[lane] += added;   // after every lane has read
        }
    }
}

__global__ __launch_bounds__(256) void scatter_rows_kernel(const uint4 *__restrict__ x,
                                                           const int32_t *__restrict__ pos,
                                                           int n_tok, int k, int row_vecs,
                                                           uint4 *__restrict__ xp) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= n_tok) return;
    const uint4 *src = x + (size_t)t * row_vecs;
    uint4 *dst[kMaxTopK];
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s)
        dst[s] = s < k ? xp + (size_t)pos[k * t + s] * row_vecs : nullptr;
    for (int j = lane; j < row_vecs; j += 64) {
        const uint4 v = src[j];
#pragma unroll
        for (int s = 0; s < kMaxTopK; ++s)
            if (s < k) dst[s][j] = v;
    }
}

}  // namespace

hipError_t launch_rank(const moe_shape_t &s, const int32_t *idx, int32_t *counts,
                       int32_t *offsets, int32_t *pos, int32_t *src, hipStream_t stream) {
    hipLaunchKernelGGL(dispatch_rank_kernel, dim3(1), dim3(kRankWaves * 64), 0, stream, idx,
                       routed_rows(s), s.n_experts, s.top_k, counts, offsets, pos, src);
    return hipGetLastError();
}

hipError_t launch_dispatch(const moe_shape_t &s, const void *x, const int32_t *idx,
                           int32_t *counts, int32_t *offsets, int32_t *pos, void *xp,
                           hipStream_t stream) {
    hipError_t err = launch_rank(s, idx, counts, offsets, pos, nullptr, stream);
    if (err != hipSuccess || s.T == 0) return err;
    const int row_vecs = (int)((size_t)s.d_model * elem_bytes(s.dtype) / 16);
    hipLaunchKernelGGL(scatter_rows_kernel, dim3((s.T + 3) / 4), dim3(256), 0, stream,
                       static_cast<const uint4 *>(x), pos, s.T, s.top_k, row_vecs,
                       static_cast<uint4 *>(xp));
    return hipGetLastError();
}

}  // namespace moe
