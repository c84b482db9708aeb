// Combine: y[t] = w[t,0] * o[pos[t,0]] + w[t,1] * o[pos[t,1]] + ..., in slot
// order, fp32 math, rounded once to y's dtype.  "Mixtral 8x7B -- The
// Evolving Transformer", section 05: the formula y = sum_k w_k E_{i_k}(x),
// and the MoE module's accumulation of each slot's weighted expert output
// into a zeroed output.  Here every row of y is written exactly once by a
// gather, so no zero fill and no atomics are needed and the result does not
// depend on scheduling.  One wavefront per (token, column chunk), 16-byte
// fp32 loads; with few tokens each row is cut into chunks so that the reads
// spread over many CUs.  Bound by HBM (k*T*d*4 bytes read, T*d*elem
// written).
#include <algorithm>

#include "moe_internal.h"

namespace moe {
namespace {

// With res (the residual stream, same dtype as y), y = res + combine: the
// block's residual add ("Mixtral 8x7B -- The Evolving Transformer", section
// 06 BLOCK), still rounded once.  y may be res itself: each element
// is read before the same thread writes it.  K (slots per token) is a
// template parameter so that the slot loops are straight-line code.
// With parts > 1, o holds that many partial sums (K slices of the down
// projection), part_stride4 float4s apart; each expert row is their sum,
// slice 0 first, before it is weighted.  With parts_dev the count is read
// from device memory (the prefill down kernel stores its choice there).
template <bool BF16_OUT, int K>
__global__ __launch_bounds__(256) void combine_kernel(const float4 *__restrict__ o,
                                                      const int32_t *__restrict__ pos,
                                                      const float *__restrict__ w, int n_tok,
                                                      int d4, int chunk4, const void *res,
                                                      void *y, int parts,
                                                      size_t part_stride4,
                                                      const int *__restrict__ parts_dev) {
    if (parts_dev) parts = *parts_dev;
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= n_tok) return;
    const float4 *r[K];
    float ws[K];
#pragma unroll
    for (int s = 0; s < K; ++s) {
        r[s] = o + (size_t)pos[K * t + s] * d4;
        ws[s] = w[K * t + s];
    }
    const int j1 = min(d4, (int)(blockIdx.y + 1) * chunk4);
    auto expert_row = [&](int s, int j) {
        float4 a = r[s][j];
        for (int p = 1; p < parts; ++p) {
            const float4 b = r[s][j + p * part_stride4];
            a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
        }
        return a;
    };
    for (int j = blockIdx.y * chunk4 + lane; j < j1; j += 64) {
        // slot order: ((w0 o0 + w1 o1) + w2 o2) + w3 o3
        const float4 a = expert_row(0, j);
        float4 v = make_float4(ws[0] * a.x, ws[0] * a.y, ws[0] * a.z, ws[0] * a.w);
#pragma unroll
        for (int s = 1; s < K; ++s) {
            const float4 b = expert_row(s, j);
            v.x = v.x + ws[s] * b.x;
            v.y = v.y + ws[s] * b.y;
            v.z = v.z + ws[s] * b.z;
            v.w = v.w + ws[s] * b.w;
        }
        if (res) {
            float4 r;
            if (BF16_OUT) {
                const uint2 p = reinterpret_cast<const uint2 *>(res)[(size_t)t * d4 + j];
                r = make_float4(bf16_to_f32(p.x & 0xffffu), bf16_to_f32(p.x >> 16),
                                bf16_to_f32(p.y & 0xffffu), bf16_to_f32(p.y >> 16));
            } else {
                r = reinterpret_cast<const float4 *>(res)[(size_t)t * d4 + j];
            }
            v.x += r.x;
            v.y += r.y;
            v.z += r.z;
            v.w += r.w;
        }
        if (BF16_OUT) {
            uint2 p;
            p.x = f32_to_bf16(v.x) | (f32_to_bf16(v.y) << 16);
            p.y = f32_to_bf16(v.z) | (f32_to_bf16(v.w) << 16);
            reinterpret_cast<uint2 *>(y)[(size_t)t * d4 + j] = p;
        } else {
            reinterpret_cast<float4 *>(y)[(size_t)t * d4 + j] = v;
        }
    }
}

template <bool BF16_OUT>
hipError_t launch_combine_t(const moe_shape_t &s, dim3 grid, const float4 *o, const int32_t *pos,
                            const float *w, int d4, int chunk4, const void *res, void *y,
                            int parts, size_t ps4, const int *parts_dev, hipStream_t stream) {
    const dim3 block(256);
    switch (s.top_k) {
    case 1:
        hipLaunchKernelGGL((combine_kernel<BF16_OUT, 1>), grid, block, 0, stream, o, pos, w, s.T,
                           d4, chunk4, res, y, parts, ps4, parts_dev);
        break;
    case 2:
        hipLaunchKernelGGL((combine_kernel<BF16_OUT, 2>), grid, block, 0, stream, o, pos, w, s.T,
                           d4, chunk4, res, y, parts, ps4, parts_dev);
        break;
    case 3:
        hipLaunchKernelGGL((combine_kernel<BF16_OUT, 3>), grid, block, 0, stream, o, pos, w, s.T,
                           d4, chunk4, res, y, parts, ps4, parts_dev);
        break;
    case 4:
        hipLaunchKernelGGL((combine_kernel<BF16_OUT, 4>), grid, block, 0, stream, o, pos, w, s.T,
                           d4, chunk4, res, y, parts, ps4, parts_dev);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const moe_shape_t &s, const float *o, const int32_t *pos,
                          const float *w, void *y, hipStream_t stream, const void *res,
                          int parts, const int *parts_dev) {
    if (s.T == 0) return hipSuccess;
    const int d4 = s.d_model / 4;
    // Column chunks of whole 64-vector passes, enough for ~512 workgroups.
    const int tok_groups = (s.T + 3) / 4;
    const int passes = (d4 + 63) / 64;
    const int nch = std::max(1, std::min(passes, 512 / tok_groups));
    const int chunk4 = (passes + nch - 1) / nch * 64;
    const dim3 grid(tok_groups, (d4 + chunk4 - 1) / chunk4);
    const float4 *o4 = reinterpret_cast<const float4 *>(o);
    const size_t ps4 = (size_t)routed_rows(s) * d4;
    if (s.dtype == MOE_BF16)
        return launch_combine_t<true>(s, grid, o4, pos, w, d4, chunk4, res, y, parts, ps4,
                                      parts_dev, stream);
    return launch_combine_t<false>(s, grid, o4, pos, w, d4, chunk4, res, y, parts, ps4,
                                   parts_dev, stream);
}

}  // namespace moe
