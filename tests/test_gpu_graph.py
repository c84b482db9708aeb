"""The layer inside a captured HIP graph: every call only enqueues kernels on
the caller's stream (no allocation, copy, fill or synchronisation inside the
library), so a whole forward can be captured once and replayed.  Each case
captures the call into a graph with fixed input and output buffers, then
replays it several times with new inputs copied into those buffers and
other eager work on the GPU in between, and checks every replay bit for bit
against an eager call on the same inputs (which the parity tests check
against the oracle)."""
import pytest
import torch

import sparse_mixture_experts_top2_amd as moe
from sparse_mixture_experts_top2_amd import workloads as W

from helpers import checked_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
REPLAYS = 3


def announce(msg):
    print(f"[gpu-graph] {msg}", flush=True)


def capture(fn):
    """Warm up on a side stream, then capture fn() into a graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    return graph


def fresh_x(wl, i):
    """A new input batch for replay i, drawn on the CPU like the layer's own
    inputs (the same shape and distribution)."""
    return checked_inputs(wl.with_(seed=wl.seed + 100 + i)).x


GRAPH_CASES = [
    W.small_workload(32, 128, 1024, E=40, seed=71),      # decode kernels, tail cut
    W.small_workload(7, 128, 256, seed=72),               # decode kernels
    W.small_workload(600, 256, 512, E=4, seed=73),        # prefill pipeline, K parts
    W.small_workload(77, 200, 328, seed=74),              # register-staged fallback
    W.small_workload(150, 128, 256, E=16, top_k=3, seed=75),
    W.WORKLOADS["tiny_fp32"],
]


@pytest.mark.parametrize("wl", GRAPH_CASES, ids=lambda w: w.name)
def test_forward_replays_in_a_graph(wl):
    announce(f"forward {wl.name}")
    g = checked_inputs(wl).to(DEV)
    k = wl.top_k
    ws = moe.alloc_workspace(wl.T, wl.d, wl.f, wl.E, g.x.dtype, DEV, top_k=k)
    x = g.x.clone()
    y = torch.empty_like(x)
    graph = capture(lambda: moe.forward(x, g.w_gate, g.w1, g.w3, g.w2, workspace=ws, out=y,
                                        top_k=k))
    other_ws = moe.alloc_workspace(wl.T, wl.d, wl.f, wl.E, g.x.dtype, DEV, top_k=k)
    for i in range(REPLAYS):
        x.copy_(fresh_x(wl, i).to(DEV))
        y.zero_()
        graph.replay()
        torch.cuda.synchronize()
        ref = moe.forward(x, g.w_gate, g.w1, g.w3, g.w2, workspace=other_ws, top_k=k)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.uint8), ref.view(torch.uint8)), (wl.name, i)
        # unrelated eager work between replays
        moe.forward(g.x, g.w_gate, g.w1, g.w3, g.w2, workspace=other_ws, top_k=k)
    announce(f"  {REPLAYS} replays bit-identical to eager calls")


def test_forward_w8_replays_in_a_graph():
    wl = W.small_workload(32, 256, 512, seed=76)
    announce(f"forward_w8 {wl.name}")
    g = checked_inputs(wl).to(DEV)
    qs = []
    for w in (g.w1, g.w3, g.w2):
        qs += list(moe.quantize_int8(w))
    ws = moe.alloc_workspace(wl.T, wl.d, wl.f, wl.E, g.x.dtype, DEV)
    x = g.x.clone()
    y = torch.empty_like(x)
    graph = capture(lambda: moe.forward_w8(x, g.w_gate, *qs, workspace=ws, out=y))
    for i in range(REPLAYS):
        x.copy_(fresh_x(wl, i).to(DEV))
        y.zero_()
        graph.replay()
        torch.cuda.synchronize()
        ref = moe.forward_w8(x, g.w_gate, *qs)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.uint8), ref.view(torch.uint8)), i


def test_block_forward_replays_in_a_graph():
    wl = W.small_workload(600, 256, 512, E=4, seed=77)
    announce(f"block_forward {wl.name}")
    g = checked_inputs(wl).to(DEV)
    gen = torch.Generator().manual_seed(5)
    rms_w = (1.0 + 0.1 * torch.randn(wl.d, generator=gen)).to(g.x.dtype).to(DEV)
    ws = moe.alloc_workspace(wl.T, wl.d, wl.f, wl.E, g.x.dtype, DEV)
    h = g.x.clone()
    res = torch.empty_like(h)
    out = torch.empty_like(h)
    graph = capture(lambda: moe.block_forward(h, rms_w, 1e-5, g.w_gate, g.w1, g.w3, g.w2,
                                              residual=res, workspace=ws, out=out))
    for i in range(REPLAYS):
        h.copy_(fresh_x(wl, i).to(DEV))
        res.copy_(fresh_x(wl, i + 10).to(DEV))
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        ref = moe.block_forward(h, rms_w, 1e-5, g.w_gate, g.w1, g.w3, g.w2, residual=res)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.uint8), ref.view(torch.uint8)), i


@pytest.mark.parametrize("wl", [W.small_workload(600, 256, 512, E=4, seed=78),
                                W.small_workload(40, 128, 256, dtype=W.F32, seed=79)],
                         ids=lambda w: w.name)
def test_backward_replays_in_a_graph(wl):
    announce(f"backward {wl.name}")
    g = checked_inputs(wl).to(DEV)
    gen = torch.Generator().manual_seed(wl.seed + 7)
    dy = torch.randn(wl.T, wl.d, generator=gen).to(g.x.dtype).to(DEV)
    ws = torch.empty(moe.backward_workspace_bytes(wl.T, wl.d, wl.f, wl.E, g.x.dtype),
                     dtype=torch.uint8, device=DEV)
    x = g.x.clone()
    outs = []
    graph = capture(lambda: outs.append(moe.backward(x, g.w_gate, g.w1, g.w3, g.w2, dy,
                                                     workspace=ws)))
    grads = outs[-1]                      # the captured call's outputs, refilled by each replay
    for i in range(REPLAYS):
        x.copy_(fresh_x(wl, i).to(DEV))
        for t in grads:
            t.zero_()
        graph.replay()
        torch.cuda.synchronize()
        ref = moe.backward(x, g.w_gate, g.w1, g.w3, g.w2, dy)
        torch.cuda.synchronize()
        for name, got, want in zip(("dx", "dw_gate", "dw1", "dw3", "dw2"), grads, ref):
            assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), (name, i)
