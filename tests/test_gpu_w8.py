"""GPU parity for weight-only int8 expert weights (decode sizes): the HIP
library through its C interface against the CPU oracle.

Bars: the codes and scales of the quantizer bit-exact (an integer decision
taken in fp32 on both sides); the layer within the bf16 layer's tolerance
(row-max-normalised 2e-2), routing indices exact and routing weights within
1e-4; each stage alone as in the bf16 step tests.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_mixture_experts_top2_amd as moe
from sparse_mixture_experts_top2_amd import workloads as W

from helpers import RW_TOL, Y_TOL, checked_inputs, row_max_rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def announce(msg):
    print(f"[gpu-w8] {msg}", flush=True)


def quantized(inp):
    """Codes and scales of w1, w3, w2 from the GPU quantizer, checked
    bit-exact against the oracle's; returned on the GPU (the kernels'
    row-pair layout) and on the host (plain [E, K, N], for the oracle)."""
    dev, host = [], []
    for w in (inp.w1, inp.w3, inp.w2):
        q, sc = moe.quantize_int8(w.to(DEV))
        torch.cuda.synchronize()
        q_o, sc_o = oracle.quantize_int8(w)
        np.testing.assert_array_equal(moe.unpack_int8(q).cpu().numpy(), q_o)
        np.testing.assert_array_equal(sc.cpu().numpy(), sc_o)
        dev += [q, sc]
        host += [q_o, sc_o]
    return dev, host


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
@pytest.mark.parametrize("shape", [(3, 64, 256), (2, 50, 328), (1, 8, 8), (4, 130, 520)])
def test_quantize_matches_oracle(dtype, shape):
    n, K, N = shape
    gen = torch.Generator().manual_seed(K * N + n)
    w = torch.randn(n, K, N, generator=gen) * torch.rand(n, 1, N, generator=gen) * 3
    w[0, :, 3] = 0.0                                   # a zero column: s = 0, q = 0
    w[-1, :, N - 1] = torch.arange(K) - K // 2 + 0.5   # with a maximum of 127, s = 1
    w[-1, 0, N - 1] = 127.0                             # and every code is an exact half
    w = w.to(torch.bfloat16) if dtype == W.BF16 else w.float()
    q, sc = moe.quantize_int8(w.to(DEV))
    torch.cuda.synchronize()
    q_o, sc_o = oracle.quantize_int8(w)
    np.testing.assert_array_equal(moe.unpack_int8(q).cpu().numpy(), q_o)
    np.testing.assert_array_equal(sc.cpu().numpy(), sc_o)
    assert sc_o[0, 3] == 0.0 and not q_o[0, :, 3].any()


sw = W.small_workload
CASES = [
    sw(1, 128, 256, seed=301),
    sw(7, 256, 512, seed=302),
    sw(16, 256, 512, top_k=4, seed=303),
    sw(17, 256, 512, seed=304),
    sw(32, 256, 512, seed=305),
    sw(32, 208, 336, top_k=1, seed=306),     # ragged column slabs on both GEMMs
    sw(32, 200, 328, seed=310),               # rows of 8-column groups (not 16)
    sw(24, 128, 272, E=64, top_k=3, seed=307),
    sw(9, 4096, 336, E=3, top_k=2, seed=309),  # K not a multiple of 32 per wavefront
    sw(20, 512, 1024, E=4, top_k=4, seed=308),
]


def run_w8_parity(inp):
    wl = inp.wl
    (q1, s1, q3, s3, q2, s2), host = quantized(inp)
    g = inp.to(DEV)
    y, idx, w = moe.forward_w8(g.x, g.w_gate, q1, s1, q3, s3, q2, s2, return_routing=True,
                               top_k=wl.top_k)
    torch.cuda.synchronize()
    y_o, idx_o, w_o = oracle.forward_w8(inp.x, inp.w_gate, *host, top_k=wl.top_k)
    np.testing.assert_array_equal(idx.cpu().numpy(), idx_o)
    np.testing.assert_allclose(w.cpu().numpy(), w_o, rtol=0, atol=RW_TOL[wl.dtype])
    err = row_max_rel_err(y, y_o)
    announce(f"{wl.name} row-max-rel err {err:.3e}")
    assert err <= Y_TOL[wl.dtype], err
    return y, y_o


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_forward_w8(wl):
    announce(f"forward_w8 {wl.name}")
    run_w8_parity(checked_inputs(wl))


@pytest.mark.parametrize("wl", [CASES[1], CASES[4], CASES[5]], ids=lambda w: w.name)
def test_each_stage_w8(wl):
    """Gate/up and down on int8 codes, each fed the oracle's previous step."""
    announce(f"stages {wl.name}")
    k = wl.top_k
    inp = checked_inputs(wl)
    (q1, s1, q3, s3, q2, s2), (hq1, hs1, hq3, hs3, hq2, hs2) = quantized(inp)
    idx_o, _ = oracle.route(inp.x, inp.w_gate, top_k=k)
    c_o, off_o, _, src_o = oracle.dispatch(idx_o, wl.E)
    xp_o = inp.x[torch.as_tensor(src_o // k)].contiguous()
    expert_of_row = np.repeat(np.arange(wl.E, dtype=np.int32), c_o)
    c_d = torch.as_tensor(c_o, device=DEV)
    off_d = torch.as_tensor(off_o, device=DEV)
    h = moe.expert_gateup_w8(xp_o.to(DEV), c_d, off_d, q1, s1, q3, s3, top_k=k)
    h_ref = oracle.expert_hidden_w8(xp_o, expert_of_row, hq1, hs1, hq3, hs3)
    err = row_max_rel_err(h, h_ref)
    announce(f"  gate/up row-max-rel err {err:.3e}")
    assert err <= 1e-2, err
    h_in = torch.from_numpy(h_ref).to(torch.bfloat16)
    o = moe.expert_down_w8(h_in.to(DEV), c_d, off_d, q2, s2, top_k=k)
    o_ref = oracle.expert_down_w8(h_in, expert_of_row, hq2, hs2)
    err = row_max_rel_err(o, o_ref)
    announce(f"  down row-max-rel err {err:.3e}")
    assert err <= 1e-4, err


def w8_tail_plan(units, cus):
    """How the int8 decode gate/up fills its last round of workgroups
    (mirrors the launcher): (whole slabs, column-half slabs, quarter slabs)
    or None when every slab runs whole."""
    if units <= cus or units % cus == 0:
        return None
    rem = units % cus
    if 4 * rem <= cus:
        plan = (units - rem, 0, rem)
    elif 2 * rem <= cus:
        plan = (units - rem, rem, 0)
    elif 4 * rem <= 3 * cus:
        plan = (units - rem, cus // 2, rem - cus // 2)
    else:
        return None
    return plan if 2 * plan[2] <= 256 else None


@pytest.mark.parametrize("wl,kind", [
    (sw(32, 200, 1928, E=56, seed=350), "halves+quarters"),  # ragged K halves, ragged last slab
    (sw(32, 264, 2048, E=40, top_k=3, seed=351), "quarters"),
    (sw(29, 128, 2048, E=48, seed=352), "halves"),
], ids=lambda v: v if isinstance(v, str) else v.name)
def test_w8_gateup_fills_last_round(wl, kind):
    """Layers whose int8 gate/up slabs (E x ceil(f / 256)) leave the last
    round of CUs part-filled, so that the launcher cuts them into column
    halves and quarters (a quarter's two K halves added by a small kernel):
    every token against the oracle."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    plan = w8_tail_plan(wl.E * ((wl.f + 255) // 256), cus)
    want = {"halves+quarters": lambda p: p[1] > 0 and p[2] > 0,
            "quarters": lambda p: p[1] == 0 and p[2] > 0,
            "halves": lambda p: p[1] > 0 and p[2] == 0}[kind]
    if plan is None or not want(plan):
        pytest.skip(f"{cus} CUs give plan {plan} for this shape, not {kind}")
    announce(f"w8 last-round pieces {wl.name}: plan {plan}")
    run_w8_parity(checked_inputs(wl))


@pytest.mark.parametrize("wl", [sw(32, 200, 1928, E=56, seed=353),
                                sw(16, 136, 2048, E=40, top_k=3, seed=354)],
                         ids=lambda w: w.name)
def test_gateup_w8_stage_with_workspace(wl):
    """moe_expert_gateup_w8_ws (the layer's gate/up kernels: whole slabs,
    column halves and quarters, the quarters' K halves added by a finishing
    kernel) against the oracle's h, fed the oracle's dispatch; the stage
    without a workspace (every slab whole) the same way."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    plan = w8_tail_plan(wl.E * ((wl.f + 255) // 256), cus)
    if plan is None or plan[2] == 0:
        pytest.skip(f"{cus} CUs give plan {plan}: no quarters to add")
    announce(f"gate/up stage with workspace {wl.name}: plan {plan}")
    k = wl.top_k
    inp = checked_inputs(wl)
    (q1, s1, q3, s3, _, _), (hq1, hs1, hq3, hs3, _, _) = quantized(inp)
    idx_o, _ = oracle.route(inp.x, inp.w_gate, top_k=k)
    c_o, off_o, _, src_o = oracle.dispatch(idx_o, wl.E)
    xp_o = inp.x[torch.as_tensor(src_o // k)].contiguous()
    expert_of_row = np.repeat(np.arange(wl.E, dtype=np.int32), c_o)
    h_ref = oracle.expert_hidden_w8(xp_o, expert_of_row, hq1, hs1, hq3, hs3)
    c_d = torch.as_tensor(c_o, device=DEV)
    off_d = torch.as_tensor(off_o, device=DEV)
    ws = moe.alloc_workspace(wl.T, wl.d, wl.f, wl.E, torch.bfloat16, DEV, top_k=k)
    ws.fill_(0xFF)   # the stage must not depend on the workspace's contents
    h_ws = moe.expert_gateup_w8(xp_o.to(DEV), c_d, off_d, q1, s1, q3, s3, top_k=k, workspace=ws)
    h = moe.expert_gateup_w8(xp_o.to(DEV), c_d, off_d, q1, s1, q3, s3, top_k=k)
    torch.cuda.synchronize()
    for name, got in (("with workspace", h_ws), ("without", h)):
        err = row_max_rel_err(got, h_ref)
        announce(f"  {name}: row-max-rel err {err:.3e}")
        assert err <= 1e-2, (name, err)


def test_int8_layer_stays_near_the_bf16_layer():
    """Per-column int8 codes change the layer by the quantization error
    only: the int8 layer's output is close to the bf16 layer's."""
    wl = sw(32, 512, 1024, seed=320)
    inp = checked_inputs(wl)
    (q1, s1, q3, s3, q2, s2), _ = quantized(inp)
    g = inp.to(DEV)
    y8 = moe.forward_w8(g.x, g.w_gate, q1, s1, q3, s3, q2, s2)
    y16 = moe.forward(g.x, g.w_gate, g.w1, g.w3, g.w2)
    err = row_max_rel_err(y8, y16.float())
    announce(f"int8 vs bf16 layer row-max-rel {err:.3e}")
    assert err <= 5e-2, err


def test_w8_reruns_are_bit_identical_and_share_a_workspace():
    wl = sw(32, 256, 512, seed=330)
    inp = checked_inputs(wl)
    (q1, s1, q3, s3, q2, s2), _ = quantized(inp)
    g = inp.to(DEV)
    ws = moe.alloc_workspace(wl.T, wl.d, wl.f, wl.E, torch.bfloat16, DEV, top_k=4)
    ys = [moe.forward_w8(g.x, g.w_gate, q1, s1, q3, s3, q2, s2, workspace=ws) for _ in range(3)]
    y4 = moe.forward_w8(g.x, g.w_gate, q1, s1, q3, s3, q2, s2, workspace=ws, top_k=4)
    y_own = moe.forward_w8(g.x, g.w_gate, q1, s1, q3, s3, q2, s2)
    torch.cuda.synchronize()
    for y in ys[1:] + [y_own]:
        assert torch.equal(y.view(torch.int16), ys[0].view(torch.int16))
    assert not torch.equal(y4.view(torch.int16), ys[0].view(torch.int16))


def test_w8_refuses_prefill_sizes_and_fp32():
    wl = sw(33, 128, 256, seed=340)
    g = W.make_inputs(wl).to(DEV)
    qs = []
    for w in (g.w1, g.w3, g.w2):
        qs += list(moe.quantize_int8(w))
    with pytest.raises(moe.MoeArgumentError, match="UNSUPPORTED"):
        moe.forward_w8(g.x, g.w_gate, *qs)
    y = moe.forward_w8(g.x[:32].contiguous(), g.w_gate, *qs)
    assert y.shape == (32, 128)
    with pytest.raises(TypeError):
        moe.forward_w8(g.x[:32].float().contiguous(), g.w_gate.float(), *qs)


@pytest.mark.slow
@pytest.mark.parametrize("name", ["decode_8x7b", "larger_expert_decode"])
def test_full_size_decode_w8(name):
    """A decode step (T = 32) at a full layer shape (the 8x7B one, in the
    launch configuration the benchmark times, and the larger expert shape):
    every code and scale of every matrix bit-exact against the oracle's
    quantizer, then the whole layer on the GPU's codes against the oracle's
    layer on its own codes, on all 32 tokens."""
    wl = W.WORKLOADS[name]
    announce("full decode w8: drawing inputs")
    inp = checked_inputs(wl)
    dev, host = quantized(inp)
    announce("full decode w8: every code and scale matches the oracle's")
    g = inp.to(DEV)
    y, idx, w = moe.forward_w8(g.x, g.w_gate, *dev, return_routing=True)
    torch.cuda.synchronize()
    announce("full decode w8: oracle on 32 tokens")
    y_o, idx_o, w_o = oracle.forward_w8(inp.x, inp.w_gate, *host)
    np.testing.assert_array_equal(idx.cpu().numpy(), idx_o)
    np.testing.assert_allclose(w.cpu().numpy(), w_o, rtol=0, atol=RW_TOL[wl.dtype])
    err = row_max_rel_err(y, y_o)
    announce(f"full decode w8 row-max-rel err {err:.3e}")
    assert err <= Y_TOL[wl.dtype], err
