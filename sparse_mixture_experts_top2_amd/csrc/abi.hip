// C interface of libmoe: argument checks, workspace planning and the launch
// sequence of the layer (route -> dispatch -> experts -> combine), all
// enqueued on the caller's stream with no host synchronisation.  The
// contract of every entry point is stated in include/moe.h.
#include <math.h>
#include <string.h>

#include <atomic>

#include "moe_internal.h"

namespace moe {

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

Layout plan_workspace(const moe_shape_t &s) {
    Layout L{};
    const size_t T = (size_t)s.T, d = (size_t)s.d_model, f = (size_t)s.d_ff;
    const size_t E = (size_t)s.n_experts, eb = elem_bytes(s.dtype);
    const size_t rows = (size_t)s.top_k * T;      // routed rows
    size_t off = 0;
    L.idx = off;     off += align256(rows * sizeof(int32_t));
    L.w = off;       off += align256(rows * sizeof(float));
    L.counts = off;  off += align256(E * sizeof(int32_t));
    L.offsets = off; off += align256((E + 1) * sizeof(int32_t));
    L.pos = off;     off += align256(rows * sizeof(int32_t));
    L.src = off;     off += align256(rows * sizeof(int32_t));
    L.xn = off;      off += align256(T * d * eb);
    L.xp = off;      off += align256(rows * d * eb);
    L.h = off;       off += align256(rows * f * eb);
    // o: at decode sizes room for the int8 path's K-slice partial sums, at
    // bf16 prefill sizes for the down product's K parts
    const size_t o_parts = T <= (size_t)kDecodeMaxT ? (size_t)kDownParts
                           : s.dtype == MOE_BF16    ? (size_t)kMaxDownSplit
                                                    : 1;
    L.o = off;       off += align256(o_parts * rows * d * sizeof(float));
    L.parts = off;   off += align256(sizeof(int32_t));
    // gpart: partial sums of the decode gate/up units cut in K halves
    const bool dec16 = T <= (size_t)kDecodeMaxT && s.dtype == MOE_BF16;
    L.gpart = off;   off += dec16 ? align256(kDecodeTailBytes) : 0;
    L.total = off;
    return L;
}

hipError_t launch_gateup(const moe_shape_t &s, const void *xp, const int32_t *counts,
                         const int32_t *offsets, const void *w1, const void *w3, void *h,
                         hipStream_t stream) {
    if (s.T == 0) return hipSuccess;
    if (s.dtype == MOE_F32)
        return launch_gateup_f32(s, static_cast<const float *>(xp), counts, offsets,
                                 static_cast<const float *>(w1), static_cast<const float *>(w3),
                                 static_cast<float *>(h), stream);
    return launch_gateup_bf16(s, static_cast<const uint16_t *>(xp), counts, offsets,
                              static_cast<const uint16_t *>(w1),
                              static_cast<const uint16_t *>(w3), static_cast<uint16_t *>(h),
                              stream);
}

hipError_t launch_down(const moe_shape_t &s, const void *h, const int32_t *counts,
                       const int32_t *offsets, const void *w2, float *o, hipStream_t stream,
                       float *gpart) {
    if (s.T == 0) return hipSuccess;
    if (s.dtype == MOE_F32)
        return launch_down_f32(s, static_cast<const float *>(h), counts, offsets,
                               static_cast<const float *>(w2), o, stream);
    return launch_down_bf16(s, static_cast<const uint16_t *>(h), counts, offsets,
                            static_cast<const uint16_t *>(w2), o, stream, gpart);
}

}  // namespace moe

using namespace moe;

namespace {

int check_shape(const moe_shape_t *s) {
    if (!s) return MOE_ERR_NULL;
    if (s->dtype != MOE_F32 && s->dtype != MOE_BF16) return MOE_ERR_DTYPE;
    if (s->n_experts < 2 || s->n_experts > kMaxExperts) return MOE_ERR_UNSUPPORTED;
    if (s->top_k < 1 || s->top_k > kMaxTopK || s->top_k > s->n_experts)
        return MOE_ERR_UNSUPPORTED;
    if (s->T < 0 || s->d_model < 8 || s->d_ff < 8) return MOE_ERR_SHAPE;
    if (s->d_model % 8 != 0 || s->d_ff % 8 != 0) return MOE_ERR_SHAPE;
    // Keep every element index of the largest array inside 2^31 * 16 bytes
    // of address arithmetic done in size_t, and row counts inside int32.
    if ((int64_t)s->T * s->top_k > (1 << 29)) return MOE_ERR_SHAPE;
    return MOE_OK;
}

bool misaligned(const void *p) { return ((uintptr_t)p & 15u) != 0; }

bool overlap(const void *a, size_t na, const void *b, size_t nb) {
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// A caller buffer: its start and the bytes a call reads or writes there.
struct Buf {
    const void *p;
    size_t n;
};

// Whether an output overlaps an input, another output or the workspace, or
// the workspace overlaps an input.  NULL or empty buffers overlap nothing;
// inputs may overlap one another.
template <size_t NI, size_t NO>
bool aliased(const Buf (&in)[NI], const Buf (&out)[NO], Buf ws = Buf{nullptr, 0}) {
    auto hit = [](Buf a, Buf b) { return a.p && b.p && a.n && b.n && overlap(a.p, a.n, b.p, b.n); };
    for (size_t i = 0; i < NO; ++i) {
        for (size_t j = 0; j < NI; ++j)
            if (hit(out[i], in[j])) return true;
        for (size_t j = i + 1; j < NO; ++j)
            if (hit(out[i], out[j])) return true;
        if (hit(out[i], ws)) return true;
    }
    for (size_t j = 0; j < NI; ++j)
        if (hit(ws, in[j])) return true;
    return false;
}

// Byte sizes of a layer's arrays.
struct Sizes {
    size_t act, wg, w13, w2, topk, rows_d, rows_f, o, cnt, off;
    explicit Sizes(const moe_shape_t &s) {
        const size_t eb = elem_bytes(s.dtype), T = (size_t)s.T, d = (size_t)s.d_model;
        const size_t f = (size_t)s.d_ff, E = (size_t)s.n_experts, R = T * s.top_k;
        act = T * d * eb;          // x, y
        wg = d * E * eb;           // w_gate
        w13 = E * d * f * eb;      // w1, w3
        w2 = E * f * d * eb;       // w2
        topk = R * 4;              // topk_idx, topk_w, pos
        rows_d = R * d * eb;       // xp
        rows_f = R * f * eb;       // h
        o = R * d * 4;             // o
        cnt = E * 4;               // counts
        off = (E + 1) * 4;         // offsets
    }
};

// Overlap that is not an exact alias (same start, same size).
bool partial_overlap(const void *a, const void *b, size_t n) {
    return a != b && overlap(a, n, b, n);
}

// The layer's launch sequence.  With g (RMSNorm weight) the router first
// normalises x into the workspace and every later step reads the normalised
// rows; with res the combine adds the residual.
hipError_t run_layer(const moe_shape_t &s, const void *x, const void *g, float eps,
                     const void *w_gate, const void *w1, const void *w3, const void *w2,
                     void *y, const void *res, int32_t *idx, float *w, const Layout &L,
                     char *base, hipStream_t str) {
    int32_t *counts = reinterpret_cast<int32_t *>(base + L.counts);
    int32_t *offsets = reinterpret_cast<int32_t *>(base + L.offsets);
    int32_t *pos = reinterpret_cast<int32_t *>(base + L.pos);
    void *xp = base + L.xp;
    void *h = base + L.h;
    float *o = reinterpret_cast<float *>(base + L.o);

    const bool dec = s.dtype == MOE_BF16 && s.T <= kDecodeMaxT;
    hipError_t e;
    const void *xin = x;
    if (g) {
        xin = base + L.xn;
        e = launch_route_norm(s, x, g, eps, w_gate, base + L.xn, idx, w, str);
    } else {
        e = launch_route(s, x, w_gate, idx, w, str);
    }
    if (dec) {
        // Few tokens: the gate/up kernel gathers its rows straight from the
        // layer input through the row -> token table, so no xp copy is made.
        // The ranking runs inside the gate/up kernel (no launch of its own).
        int32_t *src = reinterpret_cast<int32_t *>(base + L.src);
        const DecodeRank rk{idx, routed_rows(s), s.top_k, counts, offsets, pos, src};
        if (e == hipSuccess)
            e = launch_gateup_bf16(s, static_cast<const uint16_t *>(xin), counts, offsets,
                                   static_cast<const uint16_t *>(w1),
                                   static_cast<const uint16_t *>(w3),
                                   static_cast<uint16_t *>(h), str, src,
                                   reinterpret_cast<float *>(base + L.gpart), &rk);
    } else {
        if (e == hipSuccess) e = launch_dispatch(s, xin, idx, counts, offsets, pos, xp, str);
        if (e == hipSuccess) e = launch_gateup(s, xp, counts, offsets, w1, w3, h, str);
    }
    // bf16 prefill: the down product may be cut into K parts (the kernel
    // picks the count from the expert counts); the combine adds them.
    const int *parts_dev = nullptr;
    if (e == hipSuccess && s.dtype == MOE_BF16 && s.T > kDecodeMaxT) {
        int *pd = reinterpret_cast<int *>(base + L.parts);
        const hipError_t de = launch_down_split_bf16(
            routed_rows(s), s.n_experts, static_cast<const uint16_t *>(h), counts, offsets,
            static_cast<const uint16_t *>(w2), s.d_ff, s.d_model, 0,
            (size_t)routed_rows(s) * s.d_model, o, pd, str);
        if (de == hipSuccess) parts_dev = pd;
        else if (de != hipErrorNotSupported) e = de;
    }
    // bf16 decode: the down product may cut its last round like gate/up,
    // reusing the partial-sum region (the gate/up finish has read it by then)
    float *dpart = dec ? reinterpret_cast<float *>(base + L.gpart) : nullptr;
    if (e == hipSuccess && !parts_dev)
        e = launch_down(s, h, counts, offsets, w2, o, str, dpart);
    if (e == hipSuccess) e = launch_combine(s, o, pos, w, y, str, res, 1, parts_dev);
    return e;
}

// The int8-weight expert calls: bf16 activations, decode sizes only.
int check_w8(const moe_shape_t *s) {
    int st = check_shape(s);
    if (st) return st;
    if (s->dtype != MOE_BF16 || s->T > kDecodeMaxT) return MOE_ERR_UNSUPPORTED;
    // the decode kernel addresses one expert's codes with 32-bit offsets
    if ((int64_t)s->d_model * s->d_ff >= ((int64_t)1 << 31)) return MOE_ERR_SHAPE;
    return MOE_OK;
}

// moe_forward_noalloc's workspace: one copy per device, in the library's
// own device memory.  Host code never passes `scratch` itself (its host
// name is only a stand-in for the symbol); it uses the device address that
// scratch_ptr() looks up once per device.
static __device__ __align__(256) char scratch[MOE_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxScratchDevices];

// Device address of the current device's `scratch`, looked up on the
// first call on that device (nullptr if the lookup fails).  Two threads
// racing on the first call both store the same address.
void *scratch_ptr() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return nullptr;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) return p;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
    return p;
}

}  // namespace

extern "C" {

const char *moe_status_str(int status) {
    switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_NULL: return "MOE_ERR_NULL: a required pointer is NULL";
    case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE: T < 0, d_model / d_ff not a positive multiple of 8, or a size past a documented limit";
    case MOE_ERR_DTYPE: return "MOE_ERR_DTYPE: dtype must be MOE_F32 or MOE_BF16";
    case MOE_ERR_ALIGN: return "MOE_ERR_ALIGN: device pointers must be 16-byte aligned";
    case MOE_ERR_ALIAS: return "MOE_ERR_ALIAS: an output overlaps an input";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing or smaller than moe_workspace_bytes";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: n_experts must be in [2, 64] and top_k in [1, min(4, n_experts)]; the int8-weight calls take bf16 layers with T <= 32";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: a HIP kernel launch failed";
    case MOE_ERR_SCRATCH: return "MOE_ERR_SCRATCH: the shape needs more workspace than the library's fixed scratch array (MOE_SCRATCH_BYTES)";
    default: return "unknown moe status";
    }
}

size_t moe_workspace_bytes(const moe_shape_t *s) {
    if (check_shape(s) != MOE_OK) return 0;
    return plan_workspace(*s).total;
}

int moe_route(const moe_shape_t *s, const void *x, const void *w_gate, int32_t *topk_idx,
              float *topk_w, void *stream) {
    int st = check_shape(s);
    if (st) return st;
    if (s->T == 0) return MOE_OK;  // nothing to read or write
    if (!x || !w_gate || !topk_idx || !topk_w) return MOE_ERR_NULL;
    if (misaligned(x) || misaligned(w_gate) || misaligned(topk_idx) || misaligned(topk_w))
        return MOE_ERR_ALIGN;
    const Sizes z(*s);
    if (aliased({Buf{x, z.act}, Buf{w_gate, z.wg}}, {Buf{topk_idx, z.topk}, Buf{topk_w, z.topk}}))
        return MOE_ERR_ALIAS;
    return hip_status(launch_route(*s, x, w_gate, topk_idx, topk_w, (hipStream_t)stream));
}

int moe_route_probs(const moe_shape_t *s, const void *x, const void *w_gate, float *probs_opt,
                    int32_t *topk_idx, float *topk_w, void *stream) {
    int st = check_shape(s);
    if (st) return st;
    if (s->T == 0) return MOE_OK;  // nothing to read or write
    if (!x || !w_gate || !topk_idx || !topk_w) return MOE_ERR_NULL;
    if (misaligned(x) || misaligned(w_gate) || misaligned(topk_idx) || misaligned(topk_w) ||
        misaligned(probs_opt))
        return MOE_ERR_ALIGN;
    const Sizes z(*s);
    const size_t pb = (size_t)s->T * s->n_experts * 4;
    if (aliased({Buf{x, z.act}, Buf{w_gate, z.wg}},
                {Buf{probs_opt, pb}, Buf{topk_idx, z.topk}, Buf{topk_w, z.topk}}))
        return MOE_ERR_ALIAS;
    return hip_status(
        launch_route_probs(*s, x, w_gate, probs_opt, topk_idx, topk_w, (hipStream_t)stream));
}

int moe_dispatch(const moe_shape_t *s, const void *x, const int32_t *topk_idx, int32_t *counts,
                 int32_t *offsets, int32_t *pos, void *xp, void *stream) {
    int st = check_shape(s);
    if (st) return st;
    if (s->T == 0) return MOE_OK;  // nothing to read or write
    if (!x || !topk_idx || !counts || !offsets || !pos || !xp) return MOE_ERR_NULL;
    if (misaligned(x) || misaligned(topk_idx) || misaligned(counts) || misaligned(offsets) ||
        misaligned(pos) || misaligned(xp))
        return MOE_ERR_ALIGN;
    const Sizes z(*s);
    if (aliased({Buf{x, z.act}, Buf{topk_idx, z.topk}},
                {Buf{counts, z.cnt}, Buf{offsets, z.off}, Buf{pos, z.topk}, Buf{xp, z.rows_d}}))
        return MOE_ERR_ALIAS;
    return hip_status(
        launch_dispatch(*s, x, topk_idx, counts, offsets, pos, xp, (hipStream_t)stream));
}

int moe_expert_gateup(const moe_shape_t *s, const void *xp, const int32_t *counts,
                      const int32_t *offsets, const void *w1, const void *w3, void *h,
                      void *stream) {
    int st = check_shape(s);
    if (st) return st;
    if (s->T == 0) return MOE_OK;  // nothing to read or write
    if (!xp || !counts || !offsets || !w1 || !w3 || !h) return MOE_ERR_NULL;
    if (misaligned(xp) || misaligned(counts) || misaligned(offsets) || misaligned(w1) ||
        misaligned(w3) || misaligned(h))
        return MOE_ERR_ALIGN;
    const Sizes z(*s);
    if (aliased({Buf{xp, z.rows_d}, Buf{counts, z.cnt}, Buf{offsets, z.off}, Buf{w1, z.w13},
                 Buf{w3, z.w13}},
                {Buf{h, z.rows_f}}))
        return MOE_ERR_ALIAS;
    return hip_status(launch_gateup(*s, xp, counts, offsets, w1, w3, h, (hipStream_t)stream));
}

int moe_expert_gateup_ws(const moe_shape_t *s, const void *xp, const int32_t *counts,
                         const int32_t *offsets, const void *w1, const void *w3, void *h,
                         void *ws, size_t ws_bytes, void *stream) {
    int st = check_shape(s);
    if (st) return st;
    if (s->T == 0) return MOE_OK;  // nothing to read or write
    if (!xp || !counts || !offsets || !w1 || !w3 || !h || !ws) return MOE_ERR_NULL;
    if (misaligned(xp) || misaligned(counts) || misaligned(offsets) || misaligned(w1) ||
        misaligned(w3) || misaligned(h) || misaligned(ws))
        return MOE_ERR_ALIGN;
    const Layout L = plan_workspace(*s);
    if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    // the only workspace region written: the decode kernel's partial sums
    const bool dec = s->dtype == MOE_BF16 && s->T <= kDecodeMaxT;
    char *gp = static_cast<char *>(ws) + L.gpart;
    const Sizes z(*s);
    if (aliased({Buf{xp, z.rows_d}, Buf{counts, z.cnt}, Buf{offsets, z.off}, Buf{w1, z.w13},
                 Buf{w3, z.w13}},
                {Buf{h, z.rows_f}}, Buf{dec ? gp : nullptr, kDecodeTailBytes}))
        return MOE_ERR_ALIAS;
    if (!dec)
        return hip_status(launch_gateup(*s, xp, counts, offsets, w1, w3, h, (hipStream_t)stream));
    return hip_status(launch_gateup_bf16(*s, static_cast<const uint16_t *>(xp), counts, offsets,
                                         static_cast<const uint16_t *>(w1),
                                         static_cast<const uint16_t *>(w3),
                                         static_cast<uint16_t *>(h), (hipStream_t)stream, nullptr,
                                         reinterpret_cast<float *>(gp)));
}

int moe_expert_down(const moe_shape_t *s, const void *h, const int32_t *counts,
                    const int32_t *offsets, const void *w2, float *o, void *stream) {
    int st = check_shape(s);
    if (st) return st;
    if (s->T == 0) return MOE_OK;  // nothing to read or write
    if (!h || !counts || !offsets || !w2 || !o) return MOE_ERR_NULL;
    if (misaligned(h) || misaligned(counts) || misaligned(offsets) || misaligned(w2) ||
        misaligned(o))
        return MOE_ERR_ALIGN;
    const Sizes z(*s);
    if (aliased({Buf{h, z.rows_f}, Buf{counts, z.cnt}, Buf{offsets, z.off}, Buf{w2, z.w2}},
                {Buf{o, z.o}}))
        return MOE_ERR_ALIAS;
    return hip_status(launch_down(*s, h, counts, offsets, w2, o, (hipStream_t)stream));
}

int moe_experts(const moe_shape_t *s, const void *xp, const int32_t *counts,
                const int32_t *offsets, const void *w1, const void *w3, const void *w2, float *o,
                void *ws, size_t ws_bytes, void *stream) {
    int st = check_shape(s);
    if (st) return st;
    if (s->T == 0) return MOE_OK;  // nothing to read or write
    if (!xp || !counts || !offsets || !w1 || !w3 || !w2 || !o) return MOE_ERR_NULL;
    if (misaligned(xp) || misaligned(counts) || misaligned(offsets) || misaligned(w1) ||
        misaligned(w3) || misaligned(w2) || misaligned(o))
        return MOE_ERR_ALIGN;
    const Layout L = plan_workspace(*s);
    if (!ws || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    if (misaligned(ws)) return MOE_ERR_ALIGN;
    const Sizes z(*s);
    if (aliased({Buf{xp, z.rows_d}, Buf{counts, z.cnt}, Buf{offsets, z.off}, Buf{w1, z.w13},
                 Buf{w3, z.w13}, Buf{w2, z.w2}},
                {Buf{o, z.o}}, Buf{ws, L.total}))
        return MOE_ERR_ALIAS;
    void *h = static_cast<char *>(ws) + L.h;
    hipStream_t str = (hipStream_t)stream;
    hipError_t e = launch_gateup(*s, xp, counts, offsets, w1, w3, h, str);
    if (e == hipSuccess) e = launch_down(*s, h, counts, offsets, w2, o, str);
    return hip_status(e);
}

int moe_combine(const moe_shape_t *s, const float *o, const int32_t *pos, const float *topk_w,
                void *y, void *stream) {
    int st = check_shape(s);
    if (st) return st;
    if (s->T == 0) return MOE_OK;  // nothing to read or write
    if (!o || !pos || !topk_w || !y) return MOE_ERR_NULL;
    if (misaligned(o) || misaligned(pos) || misaligned(topk_w) || misaligned(y))
        return MOE_ERR_ALIGN;
    const Sizes z(*s);
    if (aliased({Buf{o, z.o}, Buf{pos, z.topk}, Buf{topk_w, z.topk}}, {Buf{y, z.act}}))
        return MOE_ERR_ALIAS;
    return hip_status(launch_combine(*s, o, pos, topk_w, y, (hipStream_t)stream));
}

int moe_forward(const moe_shape_t *s, const void *x, const void *w_gate, const void *w1,
                const void *w3, const void *w2, void *y, int32_t *topk_idx_opt,
                float *topk_w_opt, void *ws, size_t ws_bytes, void *stream) {
    int st = check_shape(s);
    if (st) return st;
    if (s->T == 0) return MOE_OK;  // nothing to read or write
    if (!x || !w_gate || !w1 || !w3 || !w2 || !y) return MOE_ERR_NULL;
    if (misaligned(x) || misaligned(w_gate) || misaligned(w1) || misaligned(w3) ||
        misaligned(w2) || misaligned(y) || misaligned(topk_idx_opt) || misaligned(topk_w_opt))
        return MOE_ERR_ALIGN;
    const Layout L = plan_workspace(*s);
    if (!ws || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    if (misaligned(ws)) return MOE_ERR_ALIGN;
    const Sizes z(*s);
    if (aliased({Buf{x, z.act}, Buf{w_gate, z.wg}, Buf{w1, z.w13}, Buf{w3, z.w13},
                 Buf{w2, z.w2}},
                {Buf{y, z.act}, Buf{topk_idx_opt, z.topk}, Buf{topk_w_opt, z.topk}},
                Buf{ws, L.total}))
        return MOE_ERR_ALIAS;

    char *base = static_cast<char *>(ws);
    int32_t *idx = topk_idx_opt ? topk_idx_opt : reinterpret_cast<int32_t *>(base + L.idx);
    float *w = topk_w_opt ? topk_w_opt : reinterpret_cast<float *>(base + L.w);
    return hip_status(run_layer(*s, x, nullptr, 0.0f, w_gate, w1, w3, w2, y, nullptr, idx, w, L,
                                base, (hipStream_t)stream));
}

int moe_forward_noalloc(const moe_shape_t *s, const void *x, const void *w_gate,
                        const void *w1, const void *w3, const void *w2, void *y,
                        int32_t *topk_idx_opt, float *topk_w_opt, void *stream) {
    int st = check_shape(s);
    if (st) return st;
    if (s->T == 0) return MOE_OK;  // nothing to read or write
    if (!x || !w_gate || !w1 || !w3 || !w2 || !y) return MOE_ERR_NULL;
    if (misaligned(x) || misaligned(w_gate) || misaligned(w1) || misaligned(w3) ||
        misaligned(w2) || misaligned(y) || misaligned(topk_idx_opt) || misaligned(topk_w_opt))
        return MOE_ERR_ALIGN;
    const Layout L = plan_workspace(*s);
    if (L.total > MOE_SCRATCH_BYTES) return MOE_ERR_SCRATCH;
    const Sizes z(*s);
    if (aliased({Buf{x, z.act}, Buf{w_gate, z.wg}, Buf{w1, z.w13}, Buf{w3, z.w13},
                 Buf{w2, z.w2}},
                {Buf{y, z.act}, Buf{topk_idx_opt, z.topk}, Buf{topk_w_opt, z.topk}}))
        return MOE_ERR_ALIAS;
    char *base = static_cast<char *>(scratch_ptr());
    if (!base) return MOE_ERR_HIP;
    int32_t *idx = topk_idx_opt ? topk_idx_opt : reinterpret_cast<int32_t *>(base + L.idx);
    float *w = topk_w_opt ? topk_w_opt : reinterpret_cast<float *>(base + L.w);
    return hip_status(run_layer(*s, x, nullptr, 0.0f, w_gate, w1, w3, w2, y, nullptr, idx, w, L,
                                base, (hipStream_t)stream));
}

int moe_rmsnorm_route(const moe_shape_t *s, const void *h, const void *rms_weight, float eps,
                      const void *w_gate, void *xn, int32_t *topk_idx, float *topk_w,
                      void *stream) {
    int st = check_shape(s);
    if (st) return st;
    if (!(eps >= 0.0f) || eps == INFINITY) return MOE_ERR_SHAPE;
    if (s->T == 0) return MOE_OK;  // nothing to read or write
    if (!h || !rms_weight || !w_gate || !xn || !topk_idx || !topk_w) return MOE_ERR_NULL;
    if (misaligned(h) || misaligned(rms_weight) || misaligned(w_gate) || misaligned(xn) ||
        misaligned(topk_idx) || misaligned(topk_w))
        return MOE_ERR_ALIGN;
    const Sizes z(*s);
    const size_t gb = (size_t)s->d_model * elem_bytes(s->dtype);
    if (aliased({Buf{h, z.act}, Buf{rms_weight, gb}, Buf{w_gate, z.wg}},
                {Buf{xn, z.act}, Buf{topk_idx, z.topk}, Buf{topk_w, z.topk}}))
        return MOE_ERR_ALIAS;
    return hip_status(launch_route_norm(*s, h, rms_weight, eps, w_gate, xn, topk_idx, topk_w,
                                        (hipStream_t)stream));
}

int moe_block_forward(const moe_shape_t *s, const void *h, const void *rms_weight, float eps,
                      const void *residual, const void *w_gate, const void *w1, const void *w3,
                      const void *w2, void *out, int32_t *topk_idx_opt, float *topk_w_opt,
                      void *ws, size_t ws_bytes, void *stream) {
    int st = check_shape(s);
    if (st) return st;
    if (!(eps >= 0.0f) || eps == INFINITY) return MOE_ERR_SHAPE;
    if (s->T == 0) return MOE_OK;  // nothing to read or write
    if (!h || !rms_weight || !w_gate || !w1 || !w3 || !w2 || !out) return MOE_ERR_NULL;
    if (misaligned(h) || misaligned(rms_weight) || misaligned(residual) || misaligned(w_gate) ||
        misaligned(w1) || misaligned(w3) || misaligned(w2) || misaligned(out) ||
        misaligned(topk_idx_opt) || misaligned(topk_w_opt))
        return MOE_ERR_ALIGN;
    const Layout L = plan_workspace(*s);
    if (!ws || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    if (misaligned(ws)) return MOE_ERR_ALIGN;
    // out may be h or the residual itself (an in-place block update): h is
    // read only by the first kernel, and the combine reads each residual
    // element before writing it.  Partial overlaps are refused.
    // Every other overlap is refused as in moe_forward.
    const Sizes z(*s);
    const size_t gb = (size_t)s->d_model * elem_bytes(s->dtype);
    if (partial_overlap(out, h, z.act) || (residual && partial_overlap(out, residual, z.act)))
        return MOE_ERR_ALIAS;
    const Buf wts[] = {Buf{rms_weight, gb}, Buf{w_gate, z.wg}, Buf{w1, z.w13}, Buf{w3, z.w13},
                       Buf{w2, z.w2}};
    if (aliased({Buf{h, z.act}, Buf{residual, z.act}, wts[0], wts[1], wts[2], wts[3], wts[4]},
                {Buf{topk_idx_opt, z.topk}, Buf{topk_w_opt, z.topk}}, Buf{ws, L.total}) ||
        aliased({wts[0], wts[1], wts[2], wts[3], wts[4], Buf{topk_idx_opt, z.topk},
                 Buf{topk_w_opt, z.topk}},
                {Buf{out, z.act}}, Buf{ws, L.total}))
        return MOE_ERR_ALIAS;

    char *base = static_cast<char *>(ws);
    int32_t *idx = topk_idx_opt ? topk_idx_opt : reinterpret_cast<int32_t *>(base + L.idx);
    float *w = topk_w_opt ? topk_w_opt : reinterpret_cast<float *>(base + L.w);
    return hip_status(run_layer(*s, h, rms_weight, eps, w_gate, w1, w3, w2, out, residual, idx,
                                w, L, base, (hipStream_t)stream));
}

// ---- Weight-only int8 expert weights -------------------------------------

int moe_quantize_int8(int n_mat, int K, int N, int dtype, const void *w, int8_t *q,
                      float *scale, void *stream) {
    if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_DTYPE;
    if (n_mat < 1 || n_mat > 65535 || K < 2 || K % 2 != 0 || N < 8 || N % 8 != 0)
        return MOE_ERR_SHAPE;
    if (!w || !q || !scale) return MOE_ERR_NULL;
    if (misaligned(w) || misaligned(q) || misaligned(scale)) return MOE_ERR_ALIGN;
    const size_t n = (size_t)n_mat * K * N;
    const size_t wb = n * elem_bytes(dtype), sb = (size_t)n_mat * N * sizeof(float);
    if (overlap(q, n, w, wb) || overlap(scale, sb, w, wb) || overlap(q, n, scale, sb))
        return MOE_ERR_ALIAS;
    return hip_status(launch_quantize_int8(n_mat, K, N, dtype, w, q, scale, (hipStream_t)stream));
}

int moe_expert_gateup_w8(const moe_shape_t *s, const void *xp, const int32_t *counts,
                         const int32_t *offsets, const int8_t *q1, const float *s1,
                         const int8_t *q3, const float *s3, void *h, void *stream) {
    int st = check_w8(s);
    if (st) return st;
    if (s->T == 0) return MOE_OK;  // nothing to read or write
    if (!xp || !counts || !offsets || !q1 || !s1 || !q3 || !s3 || !h) return MOE_ERR_NULL;
    if (misaligned(xp) || misaligned(counts) || misaligned(offsets) || misaligned(q1) ||
        misaligned(s1) || misaligned(q3) || misaligned(s3) || misaligned(h))
        return MOE_ERR_ALIGN;
    const Sizes z(*s);
    const size_t qb = z.w13 / 2, sb = (size_t)s->n_experts * s->d_ff * 4;
    if (aliased({Buf{xp, z.rows_d}, Buf{counts, z.cnt}, Buf{offsets, z.off}, Buf{q1, qb},
                 Buf{s1, sb}, Buf{q3, qb}, Buf{s3, sb}},
                {Buf{h, z.rows_f}}))
        return MOE_ERR_ALIAS;
    return hip_status(launch_gateup_w8(*s, static_cast<const uint16_t *>(xp), counts, offsets,
                                       q1, s1, q3, s3, static_cast<uint16_t *>(h),
                                       (hipStream_t)stream));
}

int moe_expert_gateup_w8_ws(const moe_shape_t *s, const void *xp, const int32_t *counts,
                            const int32_t *offsets, const int8_t *q1, const float *s1,
                            const int8_t *q3, const float *s3, void *h, void *ws,
                            size_t ws_bytes, void *stream) {
    int st = check_w8(s);
    if (st) return st;
    if (s->T == 0) return MOE_OK;  // nothing to read or write
    if (!xp || !counts || !offsets || !q1 || !s1 || !q3 || !s3 || !h || !ws) return MOE_ERR_NULL;
    if (misaligned(xp) || misaligned(counts) || misaligned(offsets) || misaligned(q1) ||
        misaligned(s1) || misaligned(q3) || misaligned(s3) || misaligned(h) || misaligned(ws))
        return MOE_ERR_ALIGN;
    const Layout L = plan_workspace(*s);
    if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    // the only workspace region written: the cut slabs' partial sums
    char *gp = static_cast<char *>(ws) + L.gpart;
    const Sizes z(*s);
    const size_t qb = z.w13 / 2, sb = (size_t)s->n_experts * s->d_ff * 4;
    if (aliased({Buf{xp, z.rows_d}, Buf{counts, z.cnt}, Buf{offsets, z.off}, Buf{q1, qb},
                 Buf{s1, sb}, Buf{q3, qb}, Buf{s3, sb}},
                {Buf{h, z.rows_f}}, Buf{gp, kDecodeTailBytes}))
        return MOE_ERR_ALIAS;
    return hip_status(launch_gateup_w8(*s, static_cast<const uint16_t *>(xp), counts, offsets,
                                       q1, s1, q3, s3, static_cast<uint16_t *>(h),
                                       (hipStream_t)stream, nullptr, nullptr,
                                       reinterpret_cast<float *>(gp)));
}

int moe_expert_down_w8(const moe_shape_t *s, const void *h, const int32_t *counts,
                       const int32_t *offsets, const int8_t *q2, const float *s2, float *o,
                       void *stream) {
    int st = check_w8(s);
    if (st) return st;
    if (s->T == 0) return MOE_OK;  // nothing to read or write
    if (!h || !counts || !offsets || !q2 || !s2 || !o) return MOE_ERR_NULL;
    if (misaligned(h) || misaligned(counts) || misaligned(offsets) || misaligned(q2) ||
        misaligned(s2) || misaligned(o))
        return MOE_ERR_ALIGN;
    const Sizes z(*s);
    const size_t qb = z.w2 / 2, sb = (size_t)s->n_experts * s->d_model * 4;
    if (aliased({Buf{h, z.rows_f}, Buf{counts, z.cnt}, Buf{offsets, z.off}, Buf{q2, qb},
                 Buf{s2, sb}},
                {Buf{o, z.o}}))
        return MOE_ERR_ALIAS;
    return hip_status(launch_down_w8(*s, static_cast<const uint16_t *>(h), counts, offsets, q2,
                                     s2, o, 1, (hipStream_t)stream));
}

int moe_forward_w8(const moe_shape_t *s, const void *x, const void *w_gate, const int8_t *q1,
                   const float *s1, const int8_t *q3, const float *s3, const int8_t *q2,
                   const float *s2, void *y, int32_t *topk_idx_opt, float *topk_w_opt, void *ws,
                   size_t ws_bytes, void *stream) {
    int st = check_w8(s);
    if (st) return st;
    if (s->T == 0) return MOE_OK;  // nothing to read or write
    if (!x || !w_gate || !q1 || !s1 || !q3 || !s3 || !q2 || !s2 || !y) return MOE_ERR_NULL;
    if (misaligned(x) || misaligned(w_gate) || misaligned(q1) || misaligned(s1) ||
        misaligned(q3) || misaligned(s3) || misaligned(q2) || misaligned(s2) || misaligned(y) ||
        misaligned(topk_idx_opt) || misaligned(topk_w_opt))
        return MOE_ERR_ALIGN;
    const Layout L = plan_workspace(*s);
    if (!ws || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    if (misaligned(ws)) return MOE_ERR_ALIGN;
    const Sizes z(*s);
    const size_t q13 = z.w13 / 2, q2b = z.w2 / 2;
    const size_t s13 = (size_t)s->n_experts * s->d_ff * 4, s2b = (size_t)s->n_experts * s->d_model * 4;
    if (aliased({Buf{x, z.act}, Buf{w_gate, z.wg}, Buf{q1, q13}, Buf{s1, s13}, Buf{q3, q13},
                 Buf{s3, s13}, Buf{q2, q2b}, Buf{s2, s2b}},
                {Buf{y, z.act}, Buf{topk_idx_opt, z.topk}, Buf{topk_w_opt, z.topk}},
                Buf{ws, L.total}))
        return MOE_ERR_ALIAS;

    char *base = static_cast<char *>(ws);
    int32_t *idx = topk_idx_opt ? topk_idx_opt : reinterpret_cast<int32_t *>(base + L.idx);
    float *w = topk_w_opt ? topk_w_opt : reinterpret_cast<float *>(base + L.w);
    int32_t *counts = reinterpret_cast<int32_t *>(base + L.counts);
    int32_t *offsets = reinterpret_cast<int32_t *>(base + L.offsets);
    int32_t *pos = reinterpret_cast<int32_t *>(base + L.pos);
    int32_t *src = reinterpret_cast<int32_t *>(base + L.src);
    uint16_t *h = reinterpret_cast<uint16_t *>(base + L.h);
    float *o = reinterpret_cast<float *>(base + L.o);
    const hipStream_t str = (hipStream_t)stream;
    // Route; gate/up ranks the picks itself (with the row -> token table)
    // and gathers its rows from x; down in kDownParts K slices; the combine
    // adds the slices.
    hipError_t e = launch_route(*s, x, w_gate, idx, w, str);
    const DecodeRank rk{idx, routed_rows(*s), s->top_k, counts, offsets, pos, src};
    if (e == hipSuccess)
        e = launch_gateup_w8(*s, static_cast<const uint16_t *>(x), counts, offsets, q1, s1, q3,
                             s3, h, str, src, &rk, reinterpret_cast<float *>(base + L.gpart));
    if (e == hipSuccess) e = launch_down_w8(*s, h, counts, offsets, q2, s2, o, kDownParts, str);
    if (e == hipSuccess) e = launch_combine(*s, o, pos, w, y, str, nullptr, kDownParts);
    return hip_status(e);
}

// ---- Backward --------------------------------------------------------------

size_t moe_backward_workspace_bytes(const moe_shape_t *s) {
    if (check_shape(s) != MOE_OK) return 0;
    return plan_backward(*s).total;
}

int moe_backward(const moe_shape_t *s, const void *x, const void *w_gate, const void *w1,
                 const void *w3, const void *w2, const void *dy, void *dx, float *dw_gate,
                 float *dw1, float *dw3, float *dw2, void *ws, size_t ws_bytes, void *stream) {
    int st = check_shape(s);
    if (st) return st;
    // With T = 0, x, dy and dx hold nothing and may be NULL; the weight
    // gradients are still written (as zeros).
    if (!w_gate || !w1 || !w3 || !w2 || !dw_gate || !dw1 || !dw3 || !dw2) return MOE_ERR_NULL;
    if (s->T > 0 && (!x || !dy || !dx)) return MOE_ERR_NULL;
    const void *ptrs[] = {x, w_gate, w1, w3, w2, dy, dx, dw_gate, dw1, dw3, dw2};
    for (const void *p : ptrs)
        if (misaligned(p)) return MOE_ERR_ALIGN;
    const BackwardLayout L = plan_backward(*s);
    if (!ws || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    if (misaligned(ws)) return MOE_ERR_ALIGN;
    const size_t eb = elem_bytes(s->dtype), T = (size_t)s->T, d = (size_t)s->d_model;
    const size_t f = (size_t)s->d_ff, E = (size_t)s->n_experts;
    if (aliased({Buf{x, T * d * eb}, Buf{w_gate, d * E * eb}, Buf{w1, E * d * f * eb},
                 Buf{w3, E * d * f * eb}, Buf{w2, E * f * d * eb}, Buf{dy, T * d * eb}},
                {Buf{dx, T * d * eb}, Buf{dw_gate, d * E * 4}, Buf{dw1, E * d * f * 4},
                 Buf{dw3, E * d * f * 4}, Buf{dw2, E * f * d * 4}},
                Buf{ws, L.total}))
        return MOE_ERR_ALIAS;
    return hip_status(launch_backward(*s, x, w_gate, w1, w3, w2, dy, dx, dw_gate, dw1, dw3, dw2,
                                      L, static_cast<char *>(ws), (hipStream_t)stream));
}

}  // extern "C"
