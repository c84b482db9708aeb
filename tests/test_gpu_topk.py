"""GPU parity for top-k routing other than 2 (k = 1 .. 4) and expert counts
up to 64: the HIP library through its C interface against the CPU oracle on
the same seeded inputs, to the same bars as the top-2 layer.

The cases cover each router instance (up to 8, 16, 32 and 64 experts; few
and many tokens per workgroup), both weight-streaming expert kernels
(T <= 16 and T <= 32: at most T rows per expert, whatever k is), the
prefill kernels with and without the direct-to-LDS path, fp32 and bf16,
k = E (every token on every expert) and ties among k candidates.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_mixture_experts_top2_amd as moe
from sparse_mixture_experts_top2_amd import workloads as W

from helpers import RW_TOL, Y_TOL, checked_block_inputs, checked_inputs, row_max_rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def announce(msg):
    print(f"[gpu-topk] {msg}", flush=True)


def check_routing(inp, idx_g, w_g):
    wl = inp.wl
    idx_o, w_o = oracle.route(inp.x, inp.w_gate, top_k=wl.top_k)
    assert tuple(idx_g.shape) == (wl.T, wl.top_k)
    np.testing.assert_array_equal(idx_g.cpu().numpy(), idx_o)
    np.testing.assert_allclose(w_g.cpu().numpy(), w_o, rtol=0, atol=RW_TOL[wl.dtype])
    return idx_o, w_o


def run_forward_parity(inp, sample=None):
    wl = inp.wl
    g = inp.to(DEV)
    y, idx, w = moe.forward(g.x, g.w_gate, g.w1, g.w3, g.w2, return_routing=True,
                            top_k=wl.top_k)
    torch.cuda.synchronize()
    idx_o, _ = check_routing(inp, idx, w)
    rows = np.arange(wl.T) if sample is None else np.asarray(sample)
    y_o, idx_s, _ = oracle.forward(inp.x[rows], inp.w_gate, inp.w1, inp.w3, inp.w2,
                                   top_k=wl.top_k)
    np.testing.assert_array_equal(idx_s, idx_o[rows])
    err = row_max_rel_err(y[torch.as_tensor(rows, device=DEV)], y_o)
    announce(f"{wl.name} T={wl.T} rows={len(rows)} row-max-rel err {err:.3e}")
    assert err <= Y_TOL[wl.dtype], err
    return y, idx_o


sw = W.small_workload
CASES = [
    # weight-streaming kernels (bf16, T <= 16 and T <= 32)
    sw(1, 128, 256, top_k=1, seed=101),
    sw(16, 256, 512, top_k=4, seed=102),
    sw(32, 256, 512, top_k=3, seed=103),
    sw(29, 200, 328, top_k=1, seed=104),
    sw(24, 128, 256, E=64, top_k=4, seed=105),
    sw(12, 128, 256, E=48, top_k=3, seed=106),
    # prefill kernels: direct-to-LDS (d % 64 == 0, f % 128 == 0) and generic
    sw(300, 256, 512, top_k=1, seed=107),
    sw(300, 256, 512, top_k=4, seed=108),
    sw(257, 200, 328, E=16, top_k=3, seed=109),
    sw(600, 128, 256, E=12, top_k=4, seed=110),
    sw(500, 128, 256, E=64, top_k=4, seed=111),
    sw(400, 192, 264, E=40, top_k=2, seed=112),
    sw(300, 128, 256, E=32, top_k=3, seed=113),
    # fp32 layers
    sw(50, 72, 40, dtype=W.F32, top_k=1, seed=114),
    sw(150, 128, 256, E=32, dtype=W.F32, top_k=3, seed=115),
    sw(700, 128, 264, E=16, dtype=W.F32, top_k=4, seed=116),
    sw(90, 64, 128, E=64, dtype=W.F32, top_k=4, seed=117),
    # k = E: every token on every expert; the weights are the full softmax
    sw(40, 128, 256, E=4, top_k=4, seed=118),
    sw(300, 128, 256, E=3, dtype=W.F32, top_k=3, seed=119),
    sw(20, 128, 256, E=2, top_k=1, seed=120),
    # expert counts whose router rows are not a multiple of 16 bytes
    sw(70, 128, 256, E=33, top_k=4, seed=121),
    sw(500, 128, 256, E=20, top_k=2, seed=122),
]


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_forward_topk(wl):
    announce(f"forward {wl.name}")
    run_forward_parity(checked_inputs(wl))


STEP_CASES = [CASES[2], CASES[7], CASES[8], CASES[14]]


@pytest.mark.parametrize("wl", STEP_CASES, ids=lambda w: w.name)
def test_each_step_topk(wl):
    """route -> dispatch -> gate/up -> down -> combine with k slots, each
    step fed the oracle's previous step (never a GPU output)."""
    announce(f"steps {wl.name}")
    k = wl.top_k
    inp = checked_inputs(wl)
    g = inp.to(DEV)
    tdt = g.x.dtype
    idx, w = moe.route(g.x, g.w_gate, top_k=k)
    idx_o, w_o = check_routing(inp, idx, w)
    counts, offsets, pos, xp = moe.dispatch(g.x, torch.as_tensor(idx_o, device=DEV), wl.E)
    c_o, off_o, pos_o, src_o = oracle.dispatch(idx_o, wl.E)
    assert int(off_o[-1]) == k * wl.T
    np.testing.assert_array_equal(counts.cpu().numpy(), c_o)
    np.testing.assert_array_equal(offsets.cpu().numpy(), off_o)
    np.testing.assert_array_equal(pos.cpu().numpy(), pos_o)
    xp_o = inp.x[torch.as_tensor(src_o // k)].contiguous()
    if tdt == torch.bfloat16:
        assert torch.equal(xp.cpu().view(torch.int16), xp_o.view(torch.int16))
    else:
        assert torch.equal(xp.cpu(), xp_o)
    expert_of_row = np.repeat(np.arange(wl.E, dtype=np.int32), c_o)
    c_d = torch.as_tensor(c_o, device=DEV)
    off_d = torch.as_tensor(off_o, device=DEV)
    h = moe.expert_gateup(xp_o.to(DEV), c_d, off_d, g.w1, g.w3, top_k=k)
    h_ref = oracle.expert_hidden(xp_o, expert_of_row, inp.w1, inp.w3)
    err = row_max_rel_err(h, h_ref)
    announce(f"  gate/up row-max-rel err {err:.3e}")
    assert err <= (1e-5 if wl.dtype == W.F32 else 1e-2), err
    h_in = torch.from_numpy(h_ref).to(tdt)
    o = moe.expert_down(h_in.to(DEV), c_d, off_d, g.w2, top_k=k)
    o_ref = oracle.expert_down(h_in, expert_of_row, inp.w2)
    err = row_max_rel_err(o, o_ref)
    announce(f"  down row-max-rel err {err:.3e}")
    assert err <= (1e-5 if wl.dtype == W.F32 else 1e-4), err
    o2 = moe.experts(xp_o.to(DEV), c_d, off_d, g.w1, g.w3, g.w2, top_k=k)
    o2_ref = oracle.expert_rows(xp_o, expert_of_row, inp.w1, inp.w3, inp.w2)
    assert row_max_rel_err(o2, o2_ref) <= Y_TOL[wl.dtype]
    o_in = torch.from_numpy(o2_ref).float()
    w_in = torch.from_numpy(w_o).float()
    y = moe.combine(o_in.to(DEV), torch.as_tensor(pos_o, device=DEV), w_in.to(DEV), tdt)
    o64 = o_in.double().numpy()
    ref = oracle.combine(np.stack([o64[pos_o[:, s]] for s in range(k)], axis=1),
                         w_in.double().numpy())
    err = row_max_rel_err(y, ref)
    assert err <= (2 ** -8 if wl.dtype == W.BF16 else 1e-6), err


def _biased(wl, bias_col, screen=True):
    bias = [0.0] * wl.E
    for e, b in bias_col.items():
        bias[e] = b
    wl = wl.with_(bias=tuple(bias))
    return checked_inputs(wl) if screen else W.make_inputs(wl)


@pytest.mark.parametrize("T", [16, 32, 300])
def test_every_token_on_the_same_four_experts(T):
    """Four experts take every token (the weight-streaming kernels then see
    their largest row count, T), the other four none."""
    wl = sw(T, 128, 256, top_k=4, seed=130 + T)
    inp = _biased(wl, {6: 80.0, 2: 70.0, 7: 60.0, 0: 50.0}, screen=False)
    y, idx_o = run_forward_parity(inp)
    assert np.all(idx_o == np.array([6, 2, 7, 0], np.int32))


@pytest.mark.parametrize("dtype", [W.F32, W.BF16])
def test_three_way_tie_takes_the_lower_indices(dtype):
    """Three identical router columns: slots take them in index order and
    the weights are exactly 1/3 each (k = 3)."""
    wl = sw(40, 128, 256, E=16, dtype=dtype, top_k=3, seed=141)
    inp = _biased(wl, {9: 50.0, 4: 50.0, 13: 50.0}, screen=False)
    inp.w_gate[:, 9] = inp.w_gate[:, 4]
    inp.w_gate[:, 13] = inp.w_gate[:, 4]
    g = inp.to(DEV)
    idx, w = moe.route(g.x, g.w_gate, top_k=3)
    assert torch.all(idx == torch.tensor([4, 9, 13], dtype=torch.int32, device=DEV))
    third = torch.tensor(1.0, dtype=torch.float32) / 3
    assert torch.all(w.cpu() == third)
    run_forward_parity(inp)


def test_top1_is_the_picked_expert_exactly():
    """k = 1: the weight is exactly 1, so y is the picked expert's output
    rounded once; it must match a plain k = 1 reading of the oracle."""
    wl = sw(64, 128, 256, dtype=W.F32, top_k=1, seed=150)
    inp = checked_inputs(wl)
    g = inp.to(DEV)
    y, idx, w = moe.forward(g.x, g.w_gate, g.w1, g.w3, g.w2, return_routing=True, top_k=1)
    assert torch.all(w == 1.0)
    counts, offsets, pos, xp = moe.dispatch(g.x, idx, wl.E)
    o = moe.experts(xp, counts, offsets, g.w1, g.w3, g.w2, top_k=1)
    assert torch.equal(y, o[pos[:, 0].long()])


@pytest.mark.parametrize("wl", [sw(24, 256, 512, top_k=3, seed=160),
                                sw(300, 256, 512, E=16, top_k=4, seed=161)],
                         ids=lambda w: w.name)
def test_block_forward_topk(wl):
    """The fused block boundary with top-k routing."""
    announce(f"block {wl.name}")
    eps = 1e-5
    gw = W.make_norm_weight(wl.d, wl.seed + 7, wl.dtype)
    inp = checked_block_inputs(wl, gw, eps)
    res = W.make_norm_weight(wl.T * wl.d, wl.seed + 8, wl.dtype).view(wl.T, wl.d)
    g = inp.to(DEV)
    out, idx, w = moe.block_forward(g.x, gw.to(DEV), eps, g.w_gate, g.w1, g.w3, g.w2,
                                    residual=res.to(DEV), return_routing=True, top_k=wl.top_k)
    torch.cuda.synchronize()
    ref, idx_o, w_o, _ = oracle.block_forward(inp.x, gw, eps, inp.w_gate, inp.w1, inp.w3,
                                              inp.w2, residual=res, top_k=wl.top_k)
    np.testing.assert_array_equal(idx.cpu().numpy(), idx_o)
    np.testing.assert_allclose(w.cpu().numpy(), w_o, rtol=0, atol=RW_TOL[wl.dtype])
    err = row_max_rel_err(out, ref)
    announce(f"  block row-max-rel err {err:.3e}")
    assert err <= Y_TOL[wl.dtype], err


def test_workspace_shared_across_k():
    """One workspace sized for k = 4 serves calls with k = 1, 2, 4 in turn;
    each result is bit-identical to a call with its own workspace."""
    base = sw(200, 256, 512, seed=170)
    ws = moe.alloc_workspace(base.T, base.d, base.f, base.E, torch.bfloat16, DEV, top_k=4)
    inp = checked_inputs(base.with_(top_k=4))
    g = inp.to(DEV)
    for k in (4, 1, 2, 4):
        y_shared = moe.forward(g.x, g.w_gate, g.w1, g.w3, g.w2, workspace=ws, top_k=k)
        y_own = moe.forward(g.x, g.w_gate, g.w1, g.w3, g.w2, top_k=k)
        torch.cuda.synchronize()
        assert torch.equal(y_shared.view(torch.int16), y_own.view(torch.int16)), k


def test_binding_checks_k_against_shapes():
    wl = sw(10, 128, 256, seed=180)
    g = W.make_inputs(wl).to(DEV)
    idx = torch.zeros(10, 3, dtype=torch.int32, device=DEV)
    idx[:, 1] = 1
    idx[:, 2] = 2
    counts, offsets, pos, xp = moe.dispatch(g.x, idx, wl.E)
    assert tuple(pos.shape) == (10, 3) and tuple(xp.shape) == (30, 128)
    with pytest.raises(ValueError):
        moe.experts(xp, counts, offsets, g.w1, g.w3, g.w2, top_k=4)
    with pytest.raises(moe.MoeArgumentError):
        moe.route(g.x, g.w_gate, top_k=5)


PROBS_CASES = [
    sw(40, 128, 256, seed=190),
    sw(300, 256, 512, top_k=4, seed=191),
    sw(100, 128, 256, E=64, top_k=3, seed=192),
    sw(600, 128, 256, E=12, dtype=W.F32, top_k=1, seed=193),
    sw(70, 128, 256, E=33, top_k=4, seed=194),
    sw(500, 128, 256, E=20, top_k=2, seed=195),
    sw(500, 128, 256, E=20, dtype=W.F32, top_k=3, seed=196),
    sw(30, 64, 128, E=4, top_k=4, seed=197),
]


@pytest.mark.parametrize("wl", PROBS_CASES, ids=lambda w: w.name)
def test_route_probs_page_form(wl):
    """The page's order of steps (softmax over all experts, top-k of the
    probabilities, renormalised) against the oracle's; the picks also equal
    the default router's and the weights agree with it to fp32 rounding."""
    announce(f"route_probs {wl.name}")
    k = wl.top_k
    inp = checked_inputs(wl)
    g = inp.to(DEV)
    probs, idx, w = moe.route_probs(g.x, g.w_gate, top_k=k)
    torch.cuda.synchronize()
    p_o, idx_o, w_o = oracle.route_probs(inp.x, inp.w_gate, top_k=k)
    np.testing.assert_array_equal(idx.cpu().numpy(), idx_o)
    np.testing.assert_allclose(w.cpu().numpy(), w_o, rtol=0, atol=RW_TOL[wl.dtype])
    np.testing.assert_allclose(probs.cpu().numpy(), p_o, rtol=0, atol=RW_TOL[wl.dtype])
    err = float(np.abs(probs.cpu().numpy() - p_o).max())
    announce(f"  probs max abs err {err:.3e}")
    idx_d, w_d = moe.route(g.x, g.w_gate, top_k=k)
    assert torch.equal(idx_d, idx)
    assert float((w_d - w).abs().max()) <= 2e-6
    _, idx2, w2 = moe.route_probs(g.x, g.w_gate, top_k=k, return_probs=False)
    assert torch.equal(idx2, idx) and torch.equal(w2, w)
