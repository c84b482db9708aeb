"""A bounded, derandomized sweep of layer shapes (hypothesis draws T, d,
d_ff, E, top_k, the dtype and the seed; the same examples on every run):
the layer and its backward from the HIP library against the oracle, to the
bars of the fixed-shape parity tests.  Sizes stay where the oracle takes
well under a second per example."""
import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
import sparse_mixture_experts_top2_amd as moe
from sparse_mixture_experts_top2_amd import workloads as W

from helpers import RW_TOL, Y_TOL, checked_inputs, row_max_rel_err, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GRAD_TOL = {W.F32: 1e-5, W.BF16: 2e-2}


def announce(msg):
    print(f"[gpu-sweep] {msg}", flush=True)


@st.composite
def layer_shapes(draw, max_T, max_d8, max_f8):
    E = draw(st.integers(2, 16))
    return W.small_workload(draw(st.integers(1, max_T)), 8 * draw(st.integers(1, max_d8)),
                            8 * draw(st.integers(1, max_f8)), E=E,
                            dtype=draw(st.sampled_from([W.BF16, W.F32])),
                            seed=draw(st.integers(0, 10 ** 6)),
                            top_k=draw(st.integers(1, min(4, E))))


SETTINGS = dict(deadline=None, derandomize=True, database=None,
                suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])


@settings(max_examples=50, **SETTINGS)
@given(wl=layer_shapes(320, 64, 80))
def test_forward_sweep(wl):
    announce(f"forward {wl.name}")
    inp = checked_inputs(wl)
    g = inp.to(DEV)
    y, idx, w = moe.forward(g.x, g.w_gate, g.w1, g.w3, g.w2, return_routing=True, top_k=wl.top_k)
    torch.cuda.synchronize()
    y_o, idx_o, w_o = oracle.forward(inp.x, inp.w_gate, inp.w1, inp.w3, inp.w2, top_k=wl.top_k)
    np.testing.assert_array_equal(idx.cpu().numpy(), idx_o)
    np.testing.assert_allclose(w.cpu().numpy(), w_o, rtol=0, atol=RW_TOL[wl.dtype])
    err = row_max_rel_err(y, y_o)
    assert err <= Y_TOL[wl.dtype], (wl.name, err)


@settings(max_examples=25, **SETTINGS)
@given(wl=layer_shapes(160, 32, 48))
def test_backward_sweep(wl):
    announce(f"backward {wl.name}")
    inp = checked_inputs(wl)
    gen = torch.Generator().manual_seed(wl.seed + 3)
    dy = torch.randn(wl.T, wl.d, generator=gen).to(inp.x.dtype)
    g = inp.to(DEV)
    got = moe.backward(g.x, g.w_gate, g.w1, g.w3, g.w2, dy.to(DEV), top_k=wl.top_k)
    torch.cuda.synchronize()
    ref = oracle.backward(inp.x, inp.w_gate, inp.w1, inp.w3, inp.w2, dy, top_k=wl.top_k)
    for name, t in zip(("dx", "dw_gate", "dw1", "dw3", "dw2"), got):
        r = ref[name]
        if name == "dx":
            err = row_max_rel_err(t, r)
        else:
            err = float(np.abs(to_f64(t) - r).max() / max(np.abs(r).max(), 1e-30))
        assert err <= GRAD_TOL[wl.dtype], (wl.name, name, err)
