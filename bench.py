#!/usr/bin/env python3
"""Throughput of the top-2 sparse MoE layer (Mixtral 8x7B shape) on one MI355X.

One step = one ``moe_forward`` call (route, dispatch, gate/up, down,
combine) over one batch of synthetic tokens whose inputs are already in HBM.
The headline workload is the 8x7B decode step (T = 32 tokens); the 8x7B
prefill (T = 4096) is measured in the same run and reported under
``secondary``.  Prints ONE JSON line.

Roofline entries: the dominant kernel of each workload (the gate/up grouped
GEMM: two thirds of the layer's bytes and FLOPs) is timed on its own with
HIP events on the stream it runs on; its algorithmic bytes (decode, HBM
bound: the selected experts' w1/w3 plus xp read and h written) or FLOPs
(prefill, MFMA bound: 2 * 2T * d * 2f) per launch are divided by that time.
``traffic`` is the measured HBM bytes per launch from the committed
rocprofv3 counter summary under profiles/ (null once the kernels' source no
longer matches the one the counters were taken on).

The CPU baseline is the plain oracle (fp64, on the host cores this process
may use, up to 16: one GPU's share of the host) run on the decode tokens
for a bounded time; the line reports the threads used and the host's core
counts.

``block_boundary``: the same workloads through moe_block_forward (RMSNorm
fused into the router, residual add into the combine), with the time the
fused steps add over the plain layer.

``w8``: the decode workload with weight-only int8 expert weights (one
fp32 scale per output column, quantized once before timing): step time,
the layer's bytes (codes and scales of the experts that received tokens,
x, y, router) over HBM peak, and the int8 gate/up kernel alone.

``backward``: moe_backward (gradients of sum(dy * y) for x, the router and
the expert matrices, recomputing the forward pieces it needs) on the
prefill workload: step time and the fraction of bf16 MFMA peak for its
nine grouped GEMMs, 9 * 2 * kT * d * f FLOPs.

``top_k``: the same workloads routed to 1 and to 4 experts per token
(Mixtral uses 2), each with its layer roofline: bytes of the experts that
received tokens for the decode step, 2 k T (3 d f) + 2 T d E FLOPs for the
prefill.

``graph_replay``: the headline step again, captured once as a HIP graph and
replayed per step (the library only enqueues kernels, so the whole call
captures).

``other_configs``: the remaining workloads measured the same way (the tiny
fp32 layer, whose kernels run on the vector ALUs, the skewed-routing 8x7B
prefill, and the larger expert shape at prefill and at decode), step time
and layer roofline each.

``ceilings``: context, not targets: what torch reaches on this GPU for a
plain device copy (bytes read + written per second) and for one bf16
matmul of the prefill's per-step expert shape [8192 x 4096] x [4096 x 14336].

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s (8x7B shape, T=32 & T=4096); % of HBM / MFMA peak"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA, TFLOP/s (256 CUs x 2.4 GHz x 4096 FLOP/clk)
PEAK_FP32_TFLOPS = 157.3       # MI355X fp32 vector ALU, TFLOP/s


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default per workload)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps (default per workload)")
    ap.add_argument("--workload", default="decode_8x7b")
    ap.add_argument("--secondary", default="prefill_8x7b", help="'' to skip")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="wall time budget of the CPU oracle baseline (0 to skip)")
    ap.add_argument("--no-block", dest="block", action="store_false",
                    help="skip the block-boundary (RMSNorm + residual) measurement")
    ap.add_argument("--no-topk", dest="topk", action="store_false",
                    help="skip the top-1 / top-4 measurement")
    ap.add_argument("--no-w8", dest="w8", action="store_false",
                    help="skip the int8-weight decode measurement")
    ap.add_argument("--no-backward", dest="backward", action="store_false",
                    help="skip the backward measurement")
    ap.add_argument("--no-graph", dest="graph", action="store_false",
                    help="skip the headline step replayed as a captured HIP graph")
    ap.add_argument("--no-others", dest="others", action="store_false",
                    help="skip the other workloads and the torch ceilings")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this size (for counter scaling)")
    return ap.parse_args()


def time_region(fn, steps, stream):
    """Mean ms per call of fn() over `steps` calls, with HIP events on `stream`."""
    import torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def measure(wl_name, steps, warmup):
    import torch
    import sparse_mixture_experts_top2_amd as moe
    from sparse_mixture_experts_top2_amd import workloads as W

    wl = W.WORKLOADS[wl_name]
    dev = torch.device("cuda:0")
    log(f"{wl_name}: drawing inputs on the GPU (T={wl.T}, d={wl.d}, f={wl.f}, E={wl.E})")
    inp = W.make_inputs(wl, device="cuda")
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ws = moe.alloc_workspace(wl.T, wl.d, wl.f, wl.E, inp.x.dtype, dev)
    y = torch.empty(wl.T, wl.d, dtype=inp.x.dtype, device=dev)

    def step():
        moe.forward(inp.x, inp.w_gate, inp.w1, inp.w3, inp.w2, workspace=ws, out=y)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms_events = time_region(step, steps, stream)
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    ms = ms_events

    # The dominant step alone: gate/up over the same routed rows, with the
    # layer's workspace so that it runs the layer's kernels.
    idx, w = moe.route(inp.x, inp.w_gate)
    counts, offsets, pos, xp = moe.dispatch(inp.x, idx, wl.E)
    h = torch.empty(2 * wl.T, wl.f, dtype=inp.x.dtype, device=dev)

    def gateup():
        moe.expert_gateup(xp, counts, offsets, inp.w1, inp.w3, out=h, workspace=ws)

    for _ in range(max(2, warmup)):
        gateup()
    k_ms = time_region(gateup, steps, stream)
    c = counts.cpu().tolist()
    active = sum(1 for v in c if v > 0)
    eb = 2 if wl.dtype == W.BF16 else 4
    weight_bytes_gu = active * 2 * wl.d * wl.f * eb
    gu_bytes = weight_bytes_gu + 2 * wl.T * wl.d * eb + 2 * wl.T * wl.f * eb
    gu_flops = 2.0 * (2 * wl.T) * wl.d * (2 * wl.f)
    layer_flops = wl.T * (2.0 * 2 * 3 * wl.d * wl.f + 2.0 * wl.d * wl.E)
    layer_bytes = active * 3 * wl.d * wl.f * eb + 2 * wl.T * wl.d * eb + wl.d * wl.E * eb
    hbm_bound = wl.T <= 32 and wl.dtype == W.BF16
    if wl.dtype == W.F32:
        # fp32 layers run on the vector ALUs (FMA), not the matrix cores
        ach = gu_flops / (k_ms * 1e-3) / 1e12
        roof = {"kernel": "expert gate/up (fp32 LDS-tiled FMA)", "bound": "alu",
                "achieved": round(ach, 3), "peak": PEAK_FP32_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / PEAK_FP32_TFLOPS, 5), "traffic": None,
                "algorithmic_flops_per_launch": gu_flops, "avg_launch_ms": round(k_ms, 5)}
        lay = layer_flops / (ms * 1e-3) / 1e12
        layer = {"bound": "alu", "achieved": round(lay, 3), "peak": PEAK_FP32_TFLOPS,
                 "unit": "TFLOP/s", "frac": round(lay / PEAK_FP32_TFLOPS, 5),
                 "algorithmic_flops_per_step": layer_flops}
    elif hbm_bound:
        ach = gu_bytes / (k_ms * 1e-3) / 1e9
        roof = {"kernel": "expert gate/up (weight-streaming MFMA)", "bound": "hbm",
                "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": counter_traffic(wl_name),
                "algorithmic_bytes_per_launch": gu_bytes, "avg_launch_ms": round(k_ms, 5)}
        lay = layer_bytes / (ms * 1e-3) / 1e9
        layer = {"bound": "hbm", "achieved": round(lay, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                 "frac": round(lay / PEAK_HBM_GBS, 4), "algorithmic_bytes_per_step": layer_bytes}
    else:
        ach = gu_flops / (k_ms * 1e-3) / 1e12
        roof = {"kernel": "expert gate/up (LDS-tiled MFMA grouped GEMM)", "bound": "mfma",
                "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": counter_traffic(wl_name),
                "algorithmic_flops_per_launch": gu_flops, "avg_launch_ms": round(k_ms, 5)}
        lay = layer_flops / (ms * 1e-3) / 1e12
        layer = {"bound": "mfma", "achieved": round(lay, 1), "peak": PEAK_BF16_TFLOPS,
                 "unit": "TFLOP/s", "frac": round(lay / PEAK_BF16_TFLOPS, 4),
                 "algorithmic_flops_per_step": layer_flops}
    log(f"{wl_name}: {ms:.4f} ms/step ({wl.T / ms * 1e3:.0f} tokens/s); gate/up {k_ms:.4f} ms; "
        f"counts {c}")
    return dict(wl=wl, inp=inp, ms=ms, ms_events=ms_events, wall_ms=wall_ms,
                tokens_per_s=wl.T / (ms * 1e-3), roofline=roof, layer_roofline=layer,
                counts=c, active_experts=active)


def measure_graph(res, steps, warmup):
    """The same layer step launched as one captured HIP graph per step (the
    library enqueues kernels only, so the whole call captures): what a
    launch-bound caller such as a decode loop would see."""
    import torch
    import sparse_mixture_experts_top2_amd as moe
    wl, inp = res["wl"], res["inp"]
    dev = torch.device("cuda:0")
    ws = moe.alloc_workspace(wl.T, wl.d, wl.f, wl.E, inp.x.dtype, dev)
    y = torch.empty(wl.T, wl.d, dtype=inp.x.dtype, device=dev)

    def step():
        moe.forward(inp.x, inp.w_gate, inp.w1, inp.w3, inp.w2, workspace=ws, out=y)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(warmup):
        graph.replay()
    ms = time_region(graph.replay, steps, torch.cuda.current_stream(dev))
    log(f"{wl.name} as a HIP graph: {ms:.4f} ms/step ({wl.T / ms * 1e3:.0f} tokens/s)")
    del graph, ws, y
    torch.cuda.empty_cache()
    return {"workload": wl.name, "value": round(wl.T / (ms * 1e-3), 1), "unit": "tokens/s",
            "ms_per_step": round(ms, 5), "steps": steps, "warmup": warmup,
            "launch": "one captured HIP graph replayed per step"}


def measure_block(wl_name, steps, warmup, plain_ms):
    """The block boundary on the same workload: out = x + layer(RMSNorm(x))
    in one moe_block_forward call (norm fused into the router, residual into
    the combine), timed like the plain layer.  Reports its step time and
    the cost of the fused norm and residual over the plain layer."""
    import torch
    import sparse_mixture_experts_top2_amd as moe
    from sparse_mixture_experts_top2_amd import workloads as W

    wl = W.WORKLOADS[wl_name]
    dev = torch.device("cuda:0")
    inp = W.make_inputs(wl, device="cuda")
    g = W.make_norm_weight(wl.d, wl.seed + 500, wl.dtype, device="cuda")
    stream = torch.cuda.current_stream(dev)
    ws = moe.alloc_workspace(wl.T, wl.d, wl.f, wl.E, inp.x.dtype, dev)
    out = torch.empty_like(inp.x)

    def step():
        moe.block_forward(inp.x, g, 1e-5, inp.w_gate, inp.w1, inp.w3, inp.w2, residual=inp.x,
                          workspace=ws, out=out)

    for _ in range(warmup):
        step()
    ms = time_region(step, steps, stream)
    log(f"{wl_name} block: {ms:.4f} ms/step ({wl.T / ms * 1e3:.0f} tokens/s)")
    return {"workload": wl_name, "value": round(wl.T / (ms * 1e-3), 1), "unit": "tokens/s",
            "ms_per_step": round(ms, 5), "steps": steps, "warmup": warmup,
            "fused_norm_residual_ms": round(ms - plain_ms, 5)}


def measure_topk(wl_name, k, steps, warmup):
    """The layer on the same workload shape with top_k = k: step time and
    the layer's roofline fraction (decode: HBM bytes of the experts that
    received tokens plus x and y; prefill: 2 k T (3 d f) + 2 T d E FLOPs)."""
    import torch
    import sparse_mixture_experts_top2_amd as moe
    from sparse_mixture_experts_top2_amd import workloads as W

    wl = W.WORKLOADS[wl_name].with_(top_k=k)
    dev = torch.device("cuda:0")
    inp = W.make_inputs(wl, device="cuda")
    stream = torch.cuda.current_stream(dev)
    ws = moe.alloc_workspace(wl.T, wl.d, wl.f, wl.E, inp.x.dtype, dev, top_k=k)
    y = torch.empty_like(inp.x)

    def step():
        moe.forward(inp.x, inp.w_gate, inp.w1, inp.w3, inp.w2, workspace=ws, out=y, top_k=k)

    for _ in range(warmup):
        step()
    ms = time_region(step, steps, stream)
    idx, _ = moe.route(inp.x, inp.w_gate, top_k=k)
    c = torch.bincount(idx.flatten().long(), minlength=wl.E).cpu().tolist()
    active = sum(1 for v in c if v > 0)
    eb = 2 if wl.dtype == W.BF16 else 4
    if wl.T <= 32:
        nbytes = active * 3 * wl.d * wl.f * eb + 2 * wl.T * wl.d * eb + wl.d * wl.E * eb
        ach = nbytes / (ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4), "algorithmic_bytes_per_step": nbytes}
    else:
        flops = wl.T * (2.0 * k * 3 * wl.d * wl.f + 2.0 * wl.d * wl.E)
        ach = flops / (ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                "algorithmic_flops_per_step": flops}
    log(f"{wl_name} top-{k}: {ms:.4f} ms/step ({wl.T / ms * 1e3:.0f} tokens/s); "
        f"layer {roof['frac'] * 100:.1f}% of {roof['bound']} peak; counts {c}")
    return {"workload": wl_name, "top_k": k, "value": round(wl.T / (ms * 1e-3), 1),
            "unit": "tokens/s", "ms_per_step": round(ms, 5), "steps": steps, "warmup": warmup,
            "layer_roofline": roof, "expert_counts": c}


def measure_w8(wl_name, steps, warmup):
    """The decode layer on int8 expert weights (moe_forward_w8)."""
    import torch
    import sparse_mixture_experts_top2_amd as moe
    from sparse_mixture_experts_top2_amd import workloads as W

    wl = W.WORKLOADS[wl_name]
    dev = torch.device("cuda:0")
    inp = W.make_inputs(wl, device="cuda")
    q1, s1 = moe.quantize_int8(inp.w1)
    q3, s3 = moe.quantize_int8(inp.w3)
    q2, s2 = moe.quantize_int8(inp.w2)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ws = moe.alloc_workspace(wl.T, wl.d, wl.f, wl.E, inp.x.dtype, dev)
    y = torch.empty_like(inp.x)

    def step():
        moe.forward_w8(inp.x, inp.w_gate, q1, s1, q3, s3, q2, s2, workspace=ws, out=y)

    for _ in range(warmup):
        step()
    ms = time_region(step, steps, stream)
    idx, _ = moe.route(inp.x, inp.w_gate)
    counts, offsets, pos, xp = moe.dispatch(inp.x, idx, wl.E)
    h = torch.empty(2 * wl.T, wl.f, dtype=inp.x.dtype, device=dev)

    def gateup():
        moe.expert_gateup_w8(xp, counts, offsets, q1, s1, q3, s3, out=h, workspace=ws)

    for _ in range(max(2, warmup)):
        gateup()
    k_ms = time_region(gateup, steps, stream)
    c = counts.cpu().tolist()
    active = sum(1 for v in c if v > 0)
    gu_bytes = (active * (2 * wl.d * wl.f + 2 * wl.f * 4) + 2 * wl.T * wl.d * 2 +
                2 * wl.T * wl.f * 2)
    layer_bytes = (active * (3 * wl.d * wl.f + (2 * wl.f + wl.d) * 4) + 2 * wl.T * wl.d * 2 +
                   wl.d * wl.E * 2)
    ach = gu_bytes / (k_ms * 1e-3) / 1e9
    lay = layer_bytes / (ms * 1e-3) / 1e9
    log(f"{wl_name} int8 weights: {ms:.4f} ms/step ({wl.T / ms * 1e3:.0f} tokens/s); "
        f"gate/up {k_ms:.4f} ms ({ach:.0f} GB/s); layer {lay:.0f} GB/s")
    return {"workload": wl_name, "weights": "int8, one fp32 scale per output column",
            "value": round(wl.T / (ms * 1e-3), 1), "unit": "tokens/s",
            "ms_per_step": round(ms, 5), "steps": steps, "warmup": warmup,
            "roofline": {"kernel": "expert gate/up on int8 codes (weight-streaming MFMA)",
                         "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                         "traffic": counter_traffic(wl_name, TRAFFIC_PROFILE_W8),
                         "algorithmic_bytes_per_launch": gu_bytes,
                         "avg_launch_ms": round(k_ms, 5)},
            "layer_roofline": {"bound": "hbm", "achieved": round(lay, 1), "peak": PEAK_HBM_GBS,
                               "unit": "GB/s", "frac": round(lay / PEAK_HBM_GBS, 4),
                               "algorithmic_bytes_per_step": layer_bytes},
            "expert_counts": c}


def measure_backward(wl_name, steps, warmup):
    """moe_backward on the workload (synthetic dy ~ N(0, 1))."""
    import torch
    import sparse_mixture_experts_top2_amd as moe
    from sparse_mixture_experts_top2_amd import workloads as W

    wl = W.WORKLOADS[wl_name]
    dev = torch.device("cuda:0")
    inp = W.make_inputs(wl, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(wl.seed + 900)
    dy = torch.randn(wl.T, wl.d, generator=gen, device="cuda").to(inp.x.dtype)
    ws = torch.empty(moe.backward_workspace_bytes(wl.T, wl.d, wl.f, wl.E, inp.x.dtype),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        moe.backward(inp.x, inp.w_gate, inp.w1, inp.w3, inp.w2, dy, workspace=ws)

    for _ in range(warmup):
        step()
    ms = time_region(step, steps, stream)
    # Eight grouped products of 2 kT d f: the recomputed g and u (two),
    # da (one: dy W2^T, from which the routing-weight gradient follows
    # without recomputing o), dXp (two) and dW1, dW3, dW2 (three); plus the
    # router's dx and dW_gate terms.
    R = 2 * wl.T
    flops = 8 * 2.0 * R * wl.d * wl.f + 4.0 * wl.T * wl.d * wl.E
    ach = flops / (ms * 1e-3) / 1e12
    log(f"{wl_name} backward: {ms:.3f} ms/step ({wl.T / ms * 1e3:.0f} tokens/s); "
        f"{ach:.0f} TFLOP/s = {ach / PEAK_BF16_TFLOPS * 100:.1f}% of bf16 peak")
    return {"workload": wl_name, "value": round(wl.T / (ms * 1e-3), 1), "unit": "tokens/s",
            "ms_per_step": round(ms, 4), "steps": steps, "warmup": warmup,
            "roofline": {"bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                         "algorithmic_flops_per_step": flops}}


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "hbm_traffic_gateup_8x7b.md")
TRAFFIC_PROFILE_W8 = os.path.join(ROOT, "profiles", "hbm_traffic_gateup_w8_decode_8x7b.md")


def counter_traffic(wl_name, profile=None):
    """HBM bytes per gate/up launch from the committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE, each scaled by a copy kernel of known
    size), or None when there is no entry for this workload or any source
    file of its kernels has changed since the counters were taken.

    The summary's last fenced block holds `fetch_scale`, `write_scale` and,
    per workload W, `W: fetch_kib=... write_kib=...` and
    `W_sources: path=sha256 path=sha256 ...`."""
    import hashlib
    try:
        text = open(profile or TRAFFIC_PROFILE).read()
    except OSError:
        return None
    block = text.rsplit("```", 2)[-2] if text.count("```") >= 2 else ""
    kv = {}
    for line in block.splitlines():
        if ":" in line:
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    try:
        sources = [f.split("=") for f in kv[wl_name + "_sources"].split()]
        if not sources:
            return None
        for path, sha in sources:
            with open(os.path.join(ROOT, path), "rb") as fh:
                if hashlib.sha256(fh.read()).hexdigest() != sha:
                    return None
        fields = dict(f.split("=") for f in kv[wl_name].split())
        return int(round((float(fields["fetch_kib"]) * float(kv["fetch_scale"]) +
                          float(fields["write_kib"]) * float(kv["write_scale"])) * 1024))
    except (KeyError, ValueError, OSError):
        return None


def cpu_baseline(res, budget_s):
    """The oracle as it stands, on the decode tokens, for about budget_s.
    It runs on every host core this process may use, up to the 16 that
    are this GPU's share of the host; both counts are reported."""
    import oracle
    visible = oracle.default_threads()
    threads = min(16, visible)
    inp = res["inp"]
    log(f"cpu baseline: copying inputs to host, oracle on {threads} threads")
    host = [t.cpu() for t in (inp.x, inp.w_gate, inp.w1, inp.w3, inp.w2)]
    T = inp.wl.T
    chunk = min(T, 16)
    done, t0 = 0, time.perf_counter()
    while True:
        lo = done % T
        rows = slice(lo, min(T, lo + chunk))
        oracle.forward(host[0][rows], *host[1:], threads=threads)
        done += rows.stop - rows.start
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    return {"value": round(done / el, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "host_cores_visible": visible, "host_cpu_count": os.cpu_count(),
            "sample": f"{done} token-evaluations of {inp.wl.name} (its {T} tokens in chunks of "
                      f"{chunk}, repeated) in {el:.1f} s; fp64 per-token loop on {threads} "
                      f"threads ({visible} host cores in this process's affinity set, "
                      f"{os.cpu_count()} on the host; 16 is one GPU's share of the host)"}


def copy_calibration(mib, steps):
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    ms = time_region(lambda: torch.mul(src, 1.0, out=dst), steps, torch.cuda.current_stream())
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "bytes_written": n * 4,
                      "ms": round(ms, 5), "GBps_rw": round(2 * n * 4 / ms / 1e6, 1)}), flush=True)


def measure_other(wl_name, steps, warmup):
    """One more workload measured like the headline one, in brief."""
    import torch
    r = measure(wl_name, steps, warmup)
    wl = r["wl"]
    out = {"workload": wl_name, "value": round(r["tokens_per_s"], 1), "unit": "tokens/s",
           "ms_per_step": round(r["ms"], 5), "steps": steps, "warmup": warmup,
           "dtype": wl.dtype, "config": {"T": wl.T, "d_model": wl.d, "d_ff": wl.f,
                                         "n_experts": wl.E, "top_k": 2},
           "roofline": r["roofline"], "layer_roofline": r["layer_roofline"],
           "expert_counts": r["counts"]}
    del r
    torch.cuda.empty_cache()
    return out


def measure_ceilings():
    """torch on this GPU, for context: a 2 GiB device copy and a bf16 matmul
    of the prefill's expert shape."""
    import torch
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    n = (2 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    ms = time_region(lambda: dst.copy_(src), 20, stream)
    copy_gbs = 2 * n * 4 / (ms * 1e-3) / 1e9
    del src, dst
    gen = torch.Generator(device=dev).manual_seed(7)
    a = torch.randn(8192, 4096, generator=gen, device=dev).to(torch.bfloat16)
    b = (torch.randn(4096, 14336, generator=gen, device=dev) * 0.015).to(torch.bfloat16)
    c = torch.empty(8192, 14336, dtype=torch.bfloat16, device=dev)
    for _ in range(3):
        torch.matmul(a, b, out=c)
    mm_ms = time_region(lambda: torch.matmul(a, b, out=c), 20, stream)
    mm_tf = 2.0 * 8192 * 4096 * 14336 / (mm_ms * 1e-3) / 1e12
    del a, b, c
    torch.cuda.empty_cache()
    log(f"ceilings: copy {copy_gbs:.0f} GB/s (read + write); bf16 matmul {mm_tf:.0f} TFLOP/s")
    return {"device_copy_GBps_read_plus_write": round(copy_gbs, 1),
            "torch_matmul_bf16_8192x4096x14336_TFLOPs": round(mm_tf, 1),
            "note": "context only: torch's own kernels on this GPU, not targets"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the layer has no "
              "multi-GPU path in this library.", flush=True)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU: the layer runs only in HIP kernels", flush=True)
        sys.exit(1)
    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib, args.steps or 20)
        return

    def defaults(name):
        if name.startswith("decode"):
            return (args.steps or 200, args.warmup if args.warmup is not None else 20)
        return (args.steps or 30, args.warmup if args.warmup is not None else 5)

    steps, warmup = defaults(args.workload)
    main_res = measure(args.workload, steps, warmup)
    graph = measure_graph(main_res, steps, warmup) if args.graph else None
    blocks = []
    if args.block:
        blocks.append(measure_block(args.workload, steps, warmup, main_res["ms"]))
    w8 = None
    if args.w8 and main_res["wl"].T <= 32 and main_res["wl"].dtype == "bf16":
        w8 = measure_w8(args.workload, steps, warmup)
        torch.cuda.empty_cache()
    topk = []
    if args.topk:
        for k in (1, 4):
            topk.append(measure_topk(args.workload, k, max(20, steps // 2), warmup))
    sec = None
    bwd = None
    if args.secondary:
        s_steps, s_warm = defaults(args.secondary)
        r = measure(args.secondary, s_steps, s_warm)
        if args.block:
            blocks.append(measure_block(args.secondary, s_steps, s_warm, r["ms"]))
        if args.topk:
            for k in (1, 4):
                topk.append(measure_topk(args.secondary, k, s_steps // 2 or 1, s_warm))
        if args.backward:
            bwd = measure_backward(args.secondary, max(5, s_steps // 3), 2)
        sec = {"workload": r["wl"].name, "value": round(r["tokens_per_s"], 1), "unit": "tokens/s",
               "ms_per_step": round(r["ms"], 5), "steps": s_steps, "warmup": s_warm,
               "config": {"T": r["wl"].T, "d_model": r["wl"].d, "d_ff": r["wl"].f,
                          "n_experts": r["wl"].E, "top_k": 2},
               "roofline": r["roofline"], "layer_roofline": r["layer_roofline"],
               "expert_counts": r["counts"]}
        del r
        torch.cuda.empty_cache()
    others = None
    ceilings = None
    if args.others:
        others = [measure_other("tiny_fp32", 200, 20),
                  measure_other("skewed_8x7b", 10, 3),
                  measure_other("larger_expert", 10, 3),
                  measure_other("larger_expert_decode", 100, 10)]
        ceilings = measure_ceilings()
    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(main_res, args.cpu_seconds)
    wl = main_res["wl"]
    out = {
        "metric": METRIC,
        "value": round(main_res["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(main_res["ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic (seeded torch draws on the GPU: x ~ N(0,1), experts ~ N(0, 1/fan_in), "
                "router std 0.02)",
        "config": {"workload": wl.name, "T": wl.T, "d_model": wl.d, "d_ff": wl.f,
                   "n_experts": wl.E, "top_k": 2},
        "roofline": main_res["roofline"],
        "layer_roofline": main_res["layer_roofline"],
        "expert_counts": main_res["counts"],
        "cpu_baseline": cpu,
        "secondary": sec,
        "graph_replay": graph,
        "block_boundary": blocks or None,
        "top_k": topk or None,
        "w8": w8,
        "backward": bwd,
        "other_configs": others,
        "ceilings": ceilings,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
