"""GPU parity: the HIP library (through its C interface) against the CPU
oracle on the same seeded inputs.

Bars: routing indices and every integer output bit-exact; routing weights
within 1e-5 (fp32) / 1e-4 (bf16) absolute; layer outputs within a
row-max-normalised error of 1e-5 (fp32) / 2e-2 (bf16 I/O, fp32 accumulation).
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_mixture_experts_top2_amd as moe
from sparse_mixture_experts_top2_amd import workloads as W

from helpers import (RW_TOL, Y_TOL, checked_inputs, down_split_parts, row_max_rel_err,
                     tile_sample, to_f64)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def announce(msg):
    print(f"[gpu-parity] {msg}", flush=True)


def check_routing(inp, idx_g, w_g, dtype):
    idx_o, w_o = oracle.route(inp.x, inp.w_gate)
    np.testing.assert_array_equal(idx_g.cpu().numpy(), idx_o)
    np.testing.assert_allclose(w_g.cpu().numpy(), w_o, rtol=0, atol=RW_TOL[dtype])
    return idx_o, w_o


def run_forward_parity(inp, sample=None):
    wl = inp.wl
    g = inp.to(DEV)
    y, idx, w = moe.forward(g.x, g.w_gate, g.w1, g.w3, g.w2, return_routing=True)
    torch.cuda.synchronize()
    idx_o, _ = check_routing(inp, idx, w, wl.dtype)
    rows = np.arange(wl.T) if sample is None else np.asarray(sample)
    y_o, idx_s, _ = oracle.forward(inp.x[rows], inp.w_gate, inp.w1, inp.w3, inp.w2)
    np.testing.assert_array_equal(idx_s, idx_o[rows])
    err = row_max_rel_err(y[torch.as_tensor(rows, device=DEV)], y_o)
    announce(f"{wl.name} T={wl.T} rows={len(rows)} row-max-rel err {err:.3e}")
    assert err <= Y_TOL[wl.dtype], err
    return y, idx_o


SMALL = [
    W.WORKLOADS["tiny_fp32"],
    W.small_workload(50, 72, 40, dtype=W.F32, seed=3),
    W.small_workload(1, 128, 256, seed=4),
    W.small_workload(7, 128, 256, seed=5),
    W.small_workload(16, 256, 512, seed=6),
    W.small_workload(32, 256, 512, seed=7),
    W.small_workload(20, 200, 328, seed=8),
    W.small_workload(33, 256, 512, seed=9),
    W.small_workload(77, 192, 264, seed=10),
    W.small_workload(300, 256, 512, seed=11),
    W.small_workload(700, 256, 384, seed=12),
    W.small_workload(100, 200, 328, seed=13),
    W.small_workload(200, 128, 256, E=2, seed=14),
    W.small_workload(200, 128, 256, E=4, seed=15),
    W.small_workload(150, 128, 256, E=16, seed=16),
    W.small_workload(150, 128, 256, E=32, seed=17),
    W.small_workload(24, 128, 256, E=32, seed=18),
]


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_forward_small(wl):
    announce(f"forward {wl.name}")
    run_forward_parity(checked_inputs(wl))


STEP_CASES = [SMALL[0], SMALL[1], SMALL[5], SMALL[6], SMALL[9], SMALL[11], SMALL[15]]


@pytest.mark.parametrize("wl", STEP_CASES, ids=lambda w: w.name)
def test_each_step(wl):
    """route -> dispatch -> gate/up -> down -> combine, each step on its own
    against the oracle.  Every step's inputs come from the generator or from
    the oracle's previous step, never from a GPU output."""
    announce(f"steps {wl.name}")
    inp = checked_inputs(wl)
    g = inp.to(DEV)
    tdt = g.x.dtype
    # route
    idx, w = moe.route(g.x, g.w_gate)
    idx_o, w_o = check_routing(inp, idx, w, wl.dtype)
    # dispatch
    counts, offsets, pos, xp = moe.dispatch(g.x, torch.as_tensor(idx_o, device=DEV), wl.E)
    c_o, off_o, pos_o, src_o = oracle.dispatch(idx_o, wl.E)
    np.testing.assert_array_equal(counts.cpu().numpy(), c_o)
    np.testing.assert_array_equal(offsets.cpu().numpy(), off_o)
    np.testing.assert_array_equal(pos.cpu().numpy(), pos_o)
    xp_o = inp.x[torch.as_tensor(src_o // 2)].contiguous()
    assert torch.equal(xp.cpu().view(torch.int16) if tdt == torch.bfloat16 else xp.cpu(),
                       xp_o.view(torch.int16) if tdt == torch.bfloat16 else xp_o)
    expert_of_row = np.repeat(np.arange(wl.E, dtype=np.int32), c_o)
    c_d = torch.as_tensor(c_o, device=DEV)
    off_d = torch.as_tensor(off_o, device=DEV)
    # gate/up + SwiGLU epilogue
    h = moe.expert_gateup(xp_o.to(DEV), c_d, off_d, g.w1, g.w3)
    h_ref = oracle.expert_hidden(xp_o, expert_of_row, inp.w1, inp.w3)
    err = row_max_rel_err(h, h_ref)
    announce(f"  gate/up row-max-rel err {err:.3e}")
    assert err <= (1e-5 if wl.dtype == W.F32 else 1e-2), err
    # down, fed the oracle's hidden activation rounded to the layer dtype
    h_in = torch.from_numpy(h_ref).to(tdt)
    o = moe.expert_down(h_in.to(DEV), c_d, off_d, g.w2)
    o_ref = oracle.expert_down(h_in, expert_of_row, inp.w2)
    err = row_max_rel_err(o, o_ref)
    announce(f"  down row-max-rel err {err:.3e}")
    assert err <= (1e-5 if wl.dtype == W.F32 else 1e-4), err
    # the two halves together
    o2 = moe.experts(xp_o.to(DEV), c_d, off_d, g.w1, g.w3, g.w2)
    o2_ref = oracle.expert_rows(xp_o, expert_of_row, inp.w1, inp.w3, inp.w2)
    assert row_max_rel_err(o2, o2_ref) <= Y_TOL[wl.dtype]
    # combine, fed the oracle's expert outputs as fp32 and its weights
    o_in = torch.from_numpy(o2_ref).float()
    w_in = torch.from_numpy(w_o).float()
    y = moe.combine(o_in.to(DEV), torch.as_tensor(pos_o, device=DEV), w_in.to(DEV), tdt)
    o64 = o_in.double().numpy()
    ref = oracle.combine(np.stack([o64[pos_o[:, 0]], o64[pos_o[:, 1]]], axis=1),
                         w_in.double().numpy())
    err = row_max_rel_err(y, ref)
    assert err <= (2 ** -8 if wl.dtype == W.BF16 else 1e-6), err


# Decode shapes whose gate/up cuts its last round of (expert, 128-column)
# units in two K halves on a 256-CU device: 40 experts x 8 column blocks =
# 320 units, 64 past the first full round.
TAIL_CASES = [
    W.small_workload(32, 128, 1024, E=40, seed=21),
    W.small_workload(12, 256, 1024, E=40, seed=22),
    W.small_workload(32, 200, 1016, E=40, seed=23),            # ragged last column block
]


def tail_cut_applies(wl) -> bool:
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    units = wl.E * ((wl.f + 127) // 128)
    rem = units % cus
    return units > cus and 0 < rem and 2 * rem <= cus


@pytest.mark.parametrize("wl", TAIL_CASES, ids=lambda w: w.name)
def test_decode_tail_cut(wl):
    """The layer and the gate/up stage with a workspace (which cut the last
    round's units in K halves) against the oracle."""
    if not tail_cut_applies(wl):
        pytest.skip("this device's CU count does not cut these units")
    announce(f"decode tail cut {wl.name}")
    inp = checked_inputs(wl)
    run_forward_parity(inp)
    k = wl.top_k
    g = inp.to(DEV)
    idx_o, _ = oracle.route(inp.x, inp.w_gate, top_k=k)
    c_o, off_o, _, src_o = oracle.dispatch(idx_o, wl.E)
    xp_o = inp.x[torch.as_tensor(src_o // k)].contiguous()
    expert_of_row = np.repeat(np.arange(wl.E, dtype=np.int32), c_o)
    c_d = torch.as_tensor(c_o, device=DEV)
    off_d = torch.as_tensor(off_o, device=DEV)
    ws = moe.alloc_workspace(wl.T, wl.d, wl.f, wl.E, g.x.dtype, DEV, top_k=k)
    h_ws = moe.expert_gateup(xp_o.to(DEV), c_d, off_d, g.w1, g.w3, top_k=k, workspace=ws)
    h = moe.expert_gateup(xp_o.to(DEV), c_d, off_d, g.w1, g.w3, top_k=k)
    h_ref = oracle.expert_hidden(xp_o, expert_of_row, inp.w1, inp.w3)
    for name, got in (("with workspace", h_ws), ("without", h)):
        err = row_max_rel_err(got, h_ref)
        announce(f"  gate/up {name} row-max-rel err {err:.3e}")
        assert err <= 1e-2, (name, err)


# Decode shapes whose down product cuts its last round the same way: 40
# experts x ceil(d / 128) = 8 column blocks of the output.
DOWN_TAIL_CASES = [
    W.small_workload(32, 1024, 256, E=40, seed=25),            # down cut only
    W.small_workload(16, 1016, 256, E=40, seed=26),            # one row block, ragged d
    W.small_workload(32, 1024, 1024, E=40, seed=27),           # gate/up and down both cut
]


@pytest.mark.parametrize("wl", DOWN_TAIL_CASES, ids=lambda w: w.name)
def test_decode_down_tail_cut(wl):
    """The layer whose decode down product cuts its last round's units in K
    halves (and adds them in a finishing kernel) against the oracle, every
    token."""
    down = wl.with_(f=(wl.d + 127) // 128 * 128)   # units of the down product: E x ceil(d/128)
    if not tail_cut_applies(down):
        pytest.skip("this device's CU count does not cut these units")
    announce(f"decode down tail cut {wl.name} (gate/up cut too: {tail_cut_applies(wl)})")
    run_forward_parity(checked_inputs(wl))


@pytest.mark.parametrize("wl", [SMALL[9], SMALL[1]], ids=lambda w: w.name)
def test_gateup_with_workspace_off_decode_sizes(wl):
    """Above decode sizes (and for fp32) the gate/up stage with a workspace
    runs the same kernels as without one: bit-identical h."""
    inp = checked_inputs(wl)
    g = inp.to(DEV)
    idx, _ = moe.route(g.x, g.w_gate)
    counts, offsets, _, xp = moe.dispatch(g.x, idx, wl.E)
    ws = moe.alloc_workspace(wl.T, wl.d, wl.f, wl.E, g.x.dtype, DEV)
    h_ws = moe.expert_gateup(xp, counts, offsets, g.w1, g.w3, workspace=ws)
    h = moe.expert_gateup(xp, counts, offsets, g.w1, g.w3)
    torch.cuda.synchronize()
    as_bits = (lambda t: t.view(torch.int16)) if g.x.dtype == torch.bfloat16 else (lambda t: t)
    assert torch.equal(as_bits(h_ws), as_bits(h))


def test_prefill_down_in_one_part():
    """A prefill layer whose down tiles fill the CUs' rounds exactly (8
    experts x 8 row tiles x 4 column tiles = 256 tiles), so the down kernel
    keeps its reduction whole and the combine reads one part: every token
    against the oracle."""
    wl = W.small_workload(7680, 1024, 512, seed=24)
    inp = checked_inputs(wl)
    idx_o, _ = oracle.route(inp.x, inp.w_gate)
    c_o, _, _, _ = oracle.dispatch(idx_o, wl.E)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if down_split_parts(c_o, wl.d // 256, cus, wl.f // 64) != 1:
        pytest.skip(f"counts {list(c_o)} on {cus} CUs pick more than one part")
    announce(f"down in one part {wl.name} counts {list(c_o)}")
    run_forward_parity(inp)


def _biased(wl, bias_col, screen=True):
    """A constant input column with router weights `bias_col` on it (folded
    in by the generator, before any near-tie screening)."""
    bias = [0.0] * wl.E
    for e, b in bias_col.items():
        bias[e] = b
    wl = wl.with_(bias=tuple(bias))
    return checked_inputs(wl) if screen else W.make_inputs(wl)


@pytest.mark.parametrize("T", [1, 32, 300])
def test_expert_with_no_tokens(T):
    wl = W.small_workload(T, 128, 256, seed=20 + T)
    inp = _biased(wl, {3: -1000.0, 6: -1000.0})
    assert not oracle.near_tie_tokens(inp.x, inp.w_gate).any()
    y, idx_o = run_forward_parity(inp)
    assert not np.isin(idx_o, [3, 6]).any()


@pytest.mark.parametrize("T", [16, 32, 257])
def test_every_token_on_the_same_two_experts(T):
    wl = W.small_workload(T, 128, 256, seed=30 + T)
    inp = _biased(wl, {4: 60.0, 1: 50.0}, screen=False)
    y, idx_o = run_forward_parity(inp)
    assert np.all(idx_o[:, 0] == 4) and np.all(idx_o[:, 1] == 1)


@pytest.mark.parametrize("dtype", [W.F32, W.BF16])
def test_exact_tie_takes_the_lower_index(dtype):
    """Duplicate router columns give bit-identical logits on both sides;
    the lower expert index must take slot 0 and the weights are 1/2."""
    wl = W.small_workload(40, 128, 256, dtype=dtype, seed=41)
    inp = _biased(wl, {2: 50.0, 5: 50.0}, screen=False)
    inp.w_gate[:, 5] = inp.w_gate[:, 2]
    g = inp.to(DEV)
    idx, w = moe.route(g.x, g.w_gate)
    assert torch.all(idx[:, 0] == 2) and torch.all(idx[:, 1] == 5)
    assert torch.all(w == 0.5)
    run_forward_parity(inp)


def test_zero_tokens():
    wl = W.small_workload(4, 128, 256)
    g = W.make_inputs(wl).to(DEV)
    y = moe.forward(g.x[:0], g.w_gate, g.w1, g.w3, g.w2)
    assert y.shape == (0, 128)


def test_bit_identical_reruns_and_token_permutation():
    wl = W.small_workload(300, 256, 512, seed=50)
    inp = checked_inputs(wl)
    g = inp.to(DEV)
    y1 = moe.forward(g.x, g.w_gate, g.w1, g.w3, g.w2)
    y2 = moe.forward(g.x, g.w_gate, g.w1, g.w3, g.w2)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    # Each row's value does not depend on which other tokens share the call
    # except through the grouped order, so a permutation keeps rows close.
    perm = torch.randperm(wl.T, generator=torch.Generator().manual_seed(0)).to(DEV)
    y3 = moe.forward(g.x[perm].contiguous(), g.w_gate, g.w1, g.w3, g.w2)
    assert row_max_rel_err(y3, y1[perm]) <= Y_TOL[wl.dtype]


# Many-token shapes whose tile counts fall on either side of the CU count:
#   40 tokens, f=2048: far fewer 256x256 tiles than CUs;
#   1500 tokens, f=3968: between one and two tiles per CU (f not a multiple
#       of 256, so gate/up's column tiles straddle the split of 2 x 128);
#   3000 tokens: about three tiles per CU, ragged row tiles per expert.
MANY_TOKENS = [
    W.small_workload(40, 1024, 2048, seed=60),
    W.small_workload(1500, 1024, 3968, seed=61),
    W.small_workload(3000, 1024, 3968, seed=62),
]


@pytest.mark.parametrize("wl", MANY_TOKENS, ids=lambda w: w.name)
def test_many_tokens_shared_workspace(wl):
    """Parity, and bit-identical results over three calls that share one
    workspace (nothing a call leaves in the workspace may leak into the
    next)."""
    announce(f"many tokens {wl.name}")
    inp = checked_inputs(wl)
    g = inp.to(DEV)
    ws = moe.alloc_workspace(wl.T, wl.d, wl.f, wl.E, g.x.dtype, DEV)
    ys = [moe.forward(g.x, g.w_gate, g.w1, g.w3, g.w2, workspace=ws) for _ in range(3)]
    torch.cuda.synchronize()
    for y in ys[1:]:
        assert torch.equal(y.view(torch.int16), ys[0].view(torch.int16))
    rng = np.random.default_rng(wl.seed)
    rows = np.arange(wl.T) if wl.T <= 256 else np.sort(rng.choice(wl.T, 192, replace=False))
    idx_o, _ = oracle.route(inp.x, inp.w_gate)
    y_o, idx_s, _ = oracle.forward(inp.x[rows], inp.w_gate, inp.w1, inp.w3, inp.w2)
    np.testing.assert_array_equal(idx_s, idx_o[rows])
    err = row_max_rel_err(ys[0][torch.as_tensor(rows, device=DEV)], y_o)
    announce(f"{wl.name} rows={len(rows)} row-max-rel err {err:.3e}")
    assert err <= Y_TOL[wl.dtype], err


def test_power_of_two_scaling_is_exact():
    wl = W.small_workload(64, 128, 256, dtype=W.F32, seed=60)
    g = checked_inputs(wl).to(DEV)
    y1 = moe.forward(g.x, g.w_gate, g.w1, g.w3, g.w2)
    y2 = moe.forward(g.x, g.w_gate, g.w1, g.w3, (2 * g.w2).contiguous())
    assert torch.equal(y2, 2 * y1)


# ---------------------------------------------------------------------------
# The full layer shapes, in the launch configuration the benchmark times.
# The oracle runs on a sample of tokens (each token is independent); routing
# is checked for every token.

FULL = [("decode_8x7b", False), ("prefill_8x7b", True), ("skewed_8x7b", True),
        ("larger_expert", True)]


@pytest.mark.slow
def test_decode_at_the_larger_expert_shape():
    """A 32-token decode step on the larger expert shape (d = 6144, f =
    16384): the decode kernels with 128 gate/up units per expert (4 full
    rounds, no tail cut) and 48 down units per expert.  Every token against
    the oracle."""
    wl = W.WORKLOADS["larger_expert_decode"]
    announce("larger-expert decode: drawing inputs")
    y, idx_o = run_forward_parity(checked_inputs(wl))
    announce(f"larger-expert decode: counts {np.bincount(idx_o.ravel(), minlength=wl.E).tolist()}")


@pytest.mark.slow
@pytest.mark.parametrize("name,sampled", FULL, ids=[f[0] for f in FULL])
def test_full_size(name, sampled):
    """Every token's routing and dispatch integers, and the output of a
    token sample chosen from the oracle's grouped order so that it reaches
    into every 256-row tile of every expert, its ragged last tile included
    (for the skewed shape: expert 0's 64 tiles and the three ~3% experts).
    The decode shape checks all 32 tokens."""
    wl = W.WORKLOADS[name]
    announce(f"full {name}: drawing inputs")
    inp = checked_inputs(wl)
    announce(f"full {name}: {inp.redrawn_rows} rows redrawn; running")
    sample = None
    if sampled:
        idx_all, _ = oracle.route(inp.x, inp.w_gate)
        sample = tile_sample(idx_all, wl.E, seed=wl.seed)
        announce(f"full {name}: {len(sample)} tokens cover every expert's row tiles")
    y, idx_o = run_forward_parity(inp, sample)
    # dispatch integers over every token
    g_idx = torch.as_tensor(idx_o, device=DEV)
    counts, offsets, pos, _ = moe.dispatch(inp.x.to(DEV), g_idx, wl.E)
    c_o, off_o, pos_o, _ = oracle.dispatch(idx_o, wl.E)
    np.testing.assert_array_equal(counts.cpu().numpy(), c_o)
    np.testing.assert_array_equal(pos.cpu().numpy(), pos_o)
    announce(f"full {name}: counts {c_o.tolist()}")
    # the same call again is bit-identical
    g = inp.to(DEV)
    y2 = moe.forward(g.x, g.w_gate, g.w1, g.w3, g.w2)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
