"""The seeded generator: determinism, value recipe, near-tie rejection and
the skewed-routing bias column.  CPU only."""
import math

import numpy as np
import pytest
import torch

import oracle
from sparse_mixture_experts_top2_amd import workloads as W


def test_same_seed_same_bytes():
    wl = W.small_workload(50, 64, 96, dtype=W.BF16, seed=3)
    a, b = W.make_inputs(wl), W.make_inputs(wl)
    for u, v in zip((a.x, a.w_gate, a.w1, a.w3, a.w2), (b.x, b.w_gate, b.w1, b.w3, b.w2)):
        assert torch.equal(u.view(torch.int16), v.view(torch.int16))
    c = W.make_inputs(wl, seed=4)
    assert not torch.equal(a.x, c.x)


def test_router_only_draw_is_a_prefix_of_the_full_draw():
    wl = W.small_workload(40, 32, 48, seed=9)
    full, head = W.make_inputs(wl), W.make_inputs(wl, experts=False)
    assert torch.equal(full.x, head.x) and torch.equal(full.w_gate, head.w_gate)


def test_value_recipe():
    wl = W.WORKLOADS["tiny_fp32"]
    inp = W.make_inputs(wl)
    assert inp.x.dtype == torch.float32 and inp.x.shape == (64, 128)
    assert inp.w1.shape == (8, 128, 256) and inp.w2.shape == (8, 256, 128)
    # std within a few percent of the recipe: x 1, w1/w3/w_gate 1/sqrt(128), w2 1/sqrt(256)
    assert abs(inp.x.std().item() - 1.0) < 0.05
    assert abs(inp.w1.std().item() * math.sqrt(128) - 1.0) < 0.03
    assert abs(inp.w2.std().item() * math.sqrt(256) - 1.0) < 0.03
    assert abs(inp.w_gate.std().item() * math.sqrt(128) - 1.0) < 0.15


def test_bf16_values_are_rne_of_the_fp32_draw():
    wl = W.small_workload(8, 16, 16, dtype=W.BF16, seed=1)
    gen = torch.Generator().manual_seed(wl.seed)
    x32 = torch.randn(wl.T, wl.d, generator=gen)
    inp = W.make_inputs(wl)
    assert torch.equal(inp.x, x32.to(torch.bfloat16))


def test_near_tie_rejection_leaves_clear_gaps():
    wl = W.small_workload(2000, 32, 16, dtype=W.BF16, seed=5)
    raw = W.make_inputs(wl, experts=False)
    clean = W.make_inputs(wl, experts=False, gap_fn=oracle.near_tie_tokens)
    assert not oracle.near_tie_tokens(clean.x, clean.w_gate).any()
    n_bad = int(oracle.near_tie_tokens(raw.x, raw.w_gate).sum())
    assert n_bad >= 1 and clean.redrawn_rows >= n_bad
    kept = ~oracle.near_tie_tokens(raw.x, raw.w_gate)
    assert torch.equal(clean.x[kept], raw.x[kept])


def test_skew_bias_column_fractions():
    wl = W.WORKLOADS["skewed_8x7b"]
    inp = W.make_inputs(wl, experts=False)
    assert torch.all(inp.x[:, -1] == 1.0)
    idx, _ = oracle.route(inp.x, inp.w_gate)
    frac = np.bincount(idx.reshape(-1), minlength=8) / idx.size
    assert 0.47 < frac[0] < 0.50
    assert np.all((frac[1:5] > 0.09) & (frac[1:5] < 0.12))
    assert np.all((frac[5:] > 0.02) & (frac[5:] < 0.04))


def test_uniform_routing_at_decode_shape():
    wl = W.WORKLOADS["prefill_8x7b"]
    inp = W.make_inputs(wl, experts=False)
    idx, _ = oracle.route(inp.x, inp.w_gate)
    frac = np.bincount(idx.reshape(-1), minlength=8) / idx.size
    assert np.all((frac > 0.09) & (frac < 0.16))
