"""GPU parity of the prefill grouped GEMMs on crafted expert row counts,
through the stage calls of the C interface (moe_expert_gateup,
moe_expert_down) against the oracle's expert stages.

The counts are chosen, not routed, so that every kind of row tile the
kernels schedule occurs: full 256-row tiles, last tiles of more than 128
rows (8 row blocks of 32), of 65..128 rows (4 blocks) and of 1..64 rows
(2 blocks), the boundary sizes 64, 65, 128, 129, 255, 256 and 257, and
experts with no rows.  The K depths cover the pipeline's 6-stage unrolled
body and its remainder.  Inputs come from the seeded generator; the down
product is fed the oracle's hidden activation rounded to bf16.

Bars: gate/up row-max-normalised error <= 1e-2 (h is rounded to bf16 on
the GPU, the oracle keeps fp64), down <= 1e-4 (fp32 output)."""
import numpy as np
import pytest
import torch

import oracle
import sparse_mixture_experts_top2_amd as moe
from sparse_mixture_experts_top2_amd import workloads as W

from helpers import row_max_rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

COUNTS = [
    [300, 70, 0, 128, 129, 64, 65, 1, 256, 513, 2, 40],      # all three tile kinds
    [255, 257, 0, 0, 511, 767],                             # around the tile size
    [64, 128, 32, 96],                                      # short experts only
]
SHAPES = [(512, 768), (384, 1024), (1024, 512)]            # (d, f)


def announce(msg):
    print(f"[gpu-gemm] {msg}", flush=True)


def crafted(counts, d, f, seed):
    E = len(counts)
    R = int(sum(counts))
    assert R % 2 == 0
    wl = W.small_workload(R // 2, d, f, E=E, seed=seed)
    inp = W.make_inputs(wl)
    gen = torch.Generator().manual_seed(seed + 1)
    xp = torch.randn(R, d, generator=gen).to(torch.bfloat16)
    c = np.asarray(counts, np.int32)
    off = np.concatenate([[0], np.cumsum(c)]).astype(np.int32)
    expert_of_row = np.repeat(np.arange(E, dtype=np.int32), c)
    return inp, xp, c, off, expert_of_row


@pytest.mark.parametrize("ci", range(len(COUNTS)))
@pytest.mark.parametrize("si", range(len(SHAPES)))
def test_grouped_gemm_tile_kinds(ci, si):
    counts = COUNTS[ci]
    d, f = SHAPES[si]
    announce(f"counts {counts} d={d} f={f}")
    inp, xp, c, off, ex = crafted(counts, d, f, seed=500 + 10 * ci + si)
    cd = torch.as_tensor(c, device=DEV)
    od = torch.as_tensor(off, device=DEV)
    h = moe.expert_gateup(xp.to(DEV), cd, od, inp.w1.to(DEV), inp.w3.to(DEV))
    torch.cuda.synchronize()
    h_ref = oracle.expert_hidden(xp, ex, inp.w1, inp.w3)
    err = row_max_rel_err(h, h_ref)
    announce(f"  gate/up row-max-rel err {err:.3e}")
    assert err <= 1e-2, err
    h_in = torch.from_numpy(h_ref).to(torch.bfloat16)
    o = moe.expert_down(h_in.to(DEV), cd, od, inp.w2.to(DEV))
    torch.cuda.synchronize()
    o_ref = oracle.expert_down(h_in, ex, inp.w2)
    err = row_max_rel_err(o, o_ref)
    announce(f"  down row-max-rel err {err:.3e}")
    assert err <= 1e-4, err
