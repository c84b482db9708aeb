// Dispatch: group the 2T (token, slot) assignments by expert, stably, and
// copy each token's row of x to its two grouped rows of xp.  This is the
// per-expert token batching that "Mixtral 8x7B -- The Evolving Transformer",
// section 05, says production stacks use in place of its per-expert mask
// loop; the order within an expert (token, then slot) is the order in which
// that loop visits the tokens.
//
// Kernel 1 (one workgroup of 256 threads): thread i owns a contiguous run
// of assignments.  Its per-expert counts go to LDS, one block-wide exclusive
// scan per expert turns them into the thread's first rank inside each
// expert, and a second pass over the run writes pos.  Thread order equals
// assignment order, so the grouping is stable and the integers are exact.
// Kernel 2 (many workgroups): one wavefront per token copies the row with
// 16-byte loads and stores; it is bound by HBM (T*d*elem read, 2*T*d*elem
// written).
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kScanThreads = 256;

__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int u = __shfl_up(v, off, 64);
        if (lane >= off) v += u;
    }
    return v;
}

__device__ __forceinline__ int clamp_expert(int e, int E) {
    return (int)min((unsigned)e, (unsigned)(E - 1));
}

__global__ __launch_bounds__(kScanThreads) void dispatch_rank_kernel(
    const int32_t *__restrict__ idx, int n_assign, int E, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ pos) {
    extern __shared__ int32_t lds[];
    int32_t *hist = lds;                                // [E][kScanThreads]
    int32_t *wave_tot = lds + E * kScanThreads;        // [kScanThreads / 64]
    int32_t *off_sh = wave_tot + kScanThreads / 64;     // [E + 1]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int chunk = (n_assign + kScanThreads - 1) / kScanThreads;
    const int a0 = min(n_assign, tid * chunk), a1 = min(n_assign, a0 + chunk);

    for (int e = 0; e < E; ++e) hist[e * kScanThreads + tid] = 0;
    // Expert ids are clamped into [0, E) so that a corrupt id can never send
    // a row outside xp; valid ids are unaffected.
    for (int a = a0; a < a1; ++a) hist[clamp_expert(idx[a], E) * kScanThreads + tid] += 1;
    __syncthreads();

    // Exclusive scan over threads, one expert at a time.
    for (int e = 0; e < E; ++e) {
        const int v = hist[e * kScanThreads + tid];
        const int inc = wave_inclusive_scan(v, lane);
        if (lane == 63) wave_tot[wave] = inc;
        __syncthreads();
        if (wave == 0) {
            constexpr int nw = kScanThreads / 64;
            int wt = lane < nw ? wave_tot[lane] : 0;
            int winc = wave_inclusive_scan(wt, lane);
            if (lane < nw) wave_tot[lane] = winc - wt;   // exclusive wave bases
            if (lane == nw - 1) off_sh[e] = winc;        // this expert's total
        }
        __syncthreads();
        hist[e * kScanThreads + tid] = wave_tot[wave] + inc - v;
        __syncthreads();
    }
    if (tid == 0) {
        int run = 0;
        for (int e = 0; e < E; ++e) {
            int c = off_sh[e];
            counts[e] = c;
            offsets[e] = run;
            off_sh[e] = run;
            run += c;
        }
        offsets[E] = run;
        off_sh[E] = run;
    }
    __syncthreads();
    for (int a = a0; a < a1; ++a) {
        const int e = clamp_expert(idx[a], E);
        int32_t &r = hist[e * kScanThreads + tid];
        pos[a] = off_sh[e] + r;
        r += 1;
    }
}

__global__ __launch_bounds__(256) void scatter_rows_kernel(const uint4 *__restrict__ x,
                                                           const int32_t *__restrict__ pos,
                                                           int n_tok, int row_vecs,
                                                           uint4 *__restrict__ xp) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= n_tok) return;
    const uint4 *src = x + (size_t)t * row_vecs;
    uint4 *d0 = xp + (size_t)pos[2 * t] * row_vecs;
    uint4 *d1 = xp + (size_t)pos[2 * t + 1] * row_vecs;
    for (int j = lane; j < row_vecs; j += 64) {
        uint4 v = src[j];
        d0[j] = v;
        d1[j] = v;
    }
}

}  // namespace

hipError_t launch_dispatch(const moe_shape_t &s, const void *x, const int32_t *idx,
                           int32_t *counts, int32_t *offsets, int32_t *pos, void *xp,
                           hipStream_t stream) {
    const int E = s.n_experts;
    const size_t lds = sizeof(int32_t) * ((size_t)E * kScanThreads + kScanThreads / 64 + E + 1);
    hipLaunchKernelGGL(dispatch_rank_kernel, dim3(1), dim3(kScanThreads), lds, stream, idx,
                       2 * s.T, E, counts, offsets, pos);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || s.T == 0) return err;
    const int row_vecs = (int)((size_t)s.d_model * elem_bytes(s.dtype) / 16);
    hipLaunchKernelGGL(scatter_rows_kernel, dim3((s.T + 3) / 4), dim3(256), 0, stream,
                       static_cast<const uint4 *>(x), pos, s.T, row_vecs,
                       static_cast<uint4 *>(xp));
    return hipGetLastError();
}

}  // namespace moe
