"""moe_forward_noalloc (the layer with its workspace in the library's fixed
device array, for callers that cannot allocate) against moe_forward, the
entry point with a caller workspace, through the C interface.

Both run the same kernels in the same order, so the outputs and routing
must be bit-identical; one case is also checked against the oracle at the
layer's tolerance.  Each check makes two calls in a row, the second with a
smaller input, so that what the first call left in the shared array cannot
leak into the second."""
import numpy as np
import pytest
import torch

import oracle
import sparse_mixture_experts_top2_amd as moe
from sparse_mixture_experts_top2_amd import workloads as W

from helpers import Y_TOL, checked_inputs, row_max_rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def announce(msg):
    print(f"[gpu-noalloc] {msg}", flush=True)


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def both(g, T, k=2):
    """moe_forward on a fresh workspace, then moe_forward_noalloc, on the
    first T tokens; returns ((y, idx, w) of each)."""
    x = g.x[:T].contiguous()
    y_ref, i_ref, w_ref = moe.forward(x, g.w_gate, g.w1, g.w3, g.w2, return_routing=True,
                                      top_k=k)
    y = torch.full_like(x, float("nan"))
    idx = torch.full((T, k), -1, dtype=torch.int32, device=DEV)
    w = torch.full((T, k), float("nan"), dtype=torch.float32, device=DEV)
    moe.forward_noalloc(x, g.w_gate, g.w1, g.w3, g.w2, out=y, routing_out=(idx, w), top_k=k)
    torch.cuda.synchronize()
    return (y_ref, i_ref, w_ref), (y, idx, w)


def assert_same(ref, got):
    for a, b in zip(ref, got):
        assert torch.equal(bits(a), bits(b))


CASES = [
    # (workload, first T, second T)
    (W.small_workload(32, 1024, 2048, seed=901), 32, 9),     # decode kernels, tail cut
    (W.small_workload(300, 512, 1024, seed=902), 300, 130),  # prefill kernels, K parts
    (W.WORKLOADS["tiny_fp32"], 64, 17),                      # fp32 layer
    (W.small_workload(40, 256, 512, E=16, top_k=3, seed=903), 40, 33),
]


@pytest.mark.parametrize("wl,t1,t2", CASES, ids=[c[0].name for c in CASES])
def test_noalloc_matches_forward(wl, t1, t2):
    announce(f"{wl.name}: T={t1} then T={t2}")
    inp = checked_inputs(wl)
    g = inp.to(DEV)
    for T in (t1, t2):
        ref, got = both(g, T, wl.top_k)
        assert_same(ref, got)
    if wl.name == "tiny_fp32":
        y_o, idx_o, _ = oracle.forward(inp.x[:t2], inp.w_gate, inp.w1, inp.w3, inp.w2)
        np.testing.assert_array_equal(got[1].cpu().numpy(), idx_o)
        assert row_max_rel_err(got[0], y_o) <= Y_TOL[wl.dtype]


def test_noalloc_decode_8x7b_then_smaller():
    """The 8x7B decode step (T = 32, the benchmark's launch configuration),
    then 5 tokens; no device memory is allocated by either call once the
    library's code is loaded."""
    wl = W.WORKLOADS["decode_8x7b"]
    announce("8x7B decode: drawing inputs on the GPU")
    g = W.make_inputs(wl, device="cuda")
    torch.cuda.synchronize()
    for T in (32, 5):
        ref, got = both(g, T)
        assert_same(ref, got)
        x = g.x[:T].contiguous()
        y = torch.empty_like(x)
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info()[0]
        alloc0 = torch.cuda.memory_allocated()
        moe.forward_noalloc(x, g.w_gate, g.w1, g.w3, g.w2, out=y)
        torch.cuda.synchronize()
        assert torch.cuda.mem_get_info()[0] == free0
        assert torch.cuda.memory_allocated() == alloc0
        assert torch.equal(bits(y), bits(ref[0]))
        announce(f"8x7B decode T={T}: bit-identical to moe_forward, nothing allocated")


def test_noalloc_refuses_shapes_past_the_scratch():
    """A shape whose workspace exceeds the fixed array is refused before
    anything is enqueued: y keeps its contents."""
    T, d, f, E = 4096, 1024, 2048, 8
    assert moe.workspace_bytes(T, d, f, E, torch.bfloat16) > moe.SCRATCH_BYTES
    x = torch.zeros(T, d, dtype=torch.bfloat16, device=DEV)
    wg = torch.zeros(d, E, dtype=torch.bfloat16, device=DEV)
    w1 = torch.zeros(E, d, f, dtype=torch.bfloat16, device=DEV)
    w2 = torch.zeros(E, f, d, dtype=torch.bfloat16, device=DEV)
    y = torch.full_like(x, 3.0)
    with pytest.raises(moe.MoeArgumentError, match="MOE_ERR_SCRATCH"):
        moe.forward_noalloc(x, wg, w1, w1, w2, out=y)
    torch.cuda.synchronize()
    assert bool((y == 3.0).all())
