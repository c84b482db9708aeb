"""Seeded synthetic workloads for the top-2 sparse MoE feed-forward layer.

This module only draws numbers.  It holds none of the layer's arithmetic (no
router product, no softmax, no expert evaluation), so both sides of a parity
check -- the HIP library and the CPU oracle -- can take their inputs from it
without sharing any of the method.  Where a caller wants near-tied routing
decisions removed, it passes in a ``gap_fn`` that computes them; this module
only redraws the rows that function flags.

Shapes follow the Mixtral 8x7B configuration given on "Mixtral 8x7B -- The
Evolving Transformer" (section 00 CONFIG: d_model 4096, d_ff 14336 per expert,
8 experts, top-2) and the KerasFormers Mixtral API table (embed_dim 4096,
mlp_dim 14336, num_experts 8, num_experts_per_tok 2).  Weight layouts are the
dense row-major ones the library takes: x [T, d], w_gate [d, E],
w1 / w3 [E, d, f] (gate / up), w2 [E, f, d] (down).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Callable, Optional, Sequence

import torch

F32 = "f32"
BF16 = "bf16"


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic layer configuration.

    ``router_std`` is the standard deviation of w_gate's entries.  Expert
    matrices are drawn with variance 1/fan_in (fan_in = d for w1 and w3,
    f for w2).  ``bias`` (length E), when set, is folded into the data as a
    constant input column: x[:, d-1] = 1 and w_gate[d-1, :] = bias, so the
    router stays bias-free as on the pages while routing becomes skewed.
    """

    name: str
    T: int
    d: int
    f: int
    E: int = 8
    top_k: int = 2
    dtype: str = BF16
    router_std: float = 0.02
    bias: Optional[Sequence[float]] = None
    seed: int = 1000
    note: str = ""

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The layer shapes this library is measured and checked on.
WORKLOADS = {
    "tiny_fp32": Workload(
        "tiny_fp32", T=64, d=128, f=256, dtype=F32,
        router_std=1.0 / math.sqrt(128), seed=1000,
        note="tiny fp32 layer, parity case the oracle finishes in well under a second"),
    "decode_8x7b": Workload(
        "decode_8x7b", T=32, d=4096, f=14336, dtype=BF16, router_std=0.02,
        seed=1001, note="Mixtral 8x7B layer, one decode step of 32 tokens (HBM-bound)"),
    "prefill_8x7b": Workload(
        "prefill_8x7b", T=4096, d=4096, f=14336, dtype=BF16, router_std=0.02,
        seed=1002, note="Mixtral 8x7B layer, prefill of batch 2 x seq 2048 (MFMA-bound)"),
    "skewed_8x7b": Workload(
        "skewed_8x7b", T=16384, d=4096, f=14336, dtype=BF16, router_std=0.02,
        bias=(4.0, 0.0, 0.0, 0.0, 0.0, -1.0, -1.0, -1.0), seed=1003,
        note="8x7B shape with a router bias column: expert 0 takes ~half of all assignments"),
    "larger_expert": Workload(
        "larger_expert", T=8192, d=6144, f=16384, dtype=BF16,
        router_std=1.0 / math.sqrt(6144), seed=1004,
        note="8x22B-sized expert tiles, ~4.8 GB of expert weights"),
    "larger_expert_decode": Workload(
        "larger_expert_decode", T=32, d=6144, f=16384, dtype=BF16,
        router_std=1.0 / math.sqrt(6144), seed=1005,
        note="one decode step of 32 tokens on the larger expert shape (HBM-bound)"),
}


@dataclasses.dataclass
class LayerInputs:
    """Inputs of one layer call.  Tensors hold the values both sides use:
    fp32 for f32 workloads, bfloat16 for bf16 workloads."""

    wl: Workload
    x: torch.Tensor        # [T, d]
    w_gate: torch.Tensor   # [d, E]
    w1: torch.Tensor       # [E, d, f]  gate projection
    w3: torch.Tensor       # [E, d, f]  up projection
    w2: torch.Tensor       # [E, f, d]  down projection
    redrawn_rows: int = 0

    def to(self, device) -> "LayerInputs":
        return LayerInputs(self.wl, self.x.to(device), self.w_gate.to(device),
                           self.w1.to(device), self.w3.to(device),
                           self.w2.to(device), self.redrawn_rows)


def torch_dtype(dtype: str) -> torch.dtype:
    return {F32: torch.float32, BF16: torch.bfloat16}[dtype]


def _cast(t: torch.Tensor, dtype: str) -> torch.Tensor:
    # fp32 -> bf16 through torch's round-to-nearest-even conversion.
    return t.to(torch_dtype(dtype)).contiguous()


def _draw_x_rows(gen: torch.Generator, n: int, wl: Workload, device) -> torch.Tensor:
    x = torch.randn(n, wl.d, generator=gen, device=device)
    if wl.bias is not None:
        x[:, wl.d - 1] = 1.0
    return x


def _draw_experts(gen: torch.Generator, wl: Workload, device):
    tdt = torch_dtype(wl.dtype)
    w1 = torch.empty(wl.E, wl.d, wl.f, dtype=tdt, device=device)
    w3 = torch.empty(wl.E, wl.d, wl.f, dtype=tdt, device=device)
    w2 = torch.empty(wl.E, wl.f, wl.d, dtype=tdt, device=device)
    s_in, s_ff = 1.0 / math.sqrt(wl.d), 1.0 / math.sqrt(wl.f)
    for e in range(wl.E):
        w1[e] = (torch.randn(wl.d, wl.f, generator=gen, device=device) * s_in).to(tdt)
        w3[e] = (torch.randn(wl.d, wl.f, generator=gen, device=device) * s_in).to(tdt)
        w2[e] = (torch.randn(wl.f, wl.d, generator=gen, device=device) * s_ff).to(tdt)
    return w1, w3, w2


def make_inputs(wl: Workload, seed: Optional[int] = None, *,
                gap_fn: Optional[Callable[[torch.Tensor, torch.Tensor], torch.Tensor]] = None,
                device: str = "cpu", max_redraw_rounds: int = 64,
                experts: bool = True) -> LayerInputs:
    """Draw one seeded layer input.

    Draw order from ``torch.Generator(device).manual_seed(seed)``: x, w_gate,
    then w1[e], w3[e], w2[e] for e = 0..E-1 (one expert's matrix at a time,
    which bounds host memory for the large shapes), each as standard normals
    scaled by its standard deviation, then rounded to the workload dtype.

    ``gap_fn(x, w_gate)`` returns a bool tensor [T] marking tokens whose
    routing decision is too close to call.  Those rows of x are redrawn, in
    token order, from a second generator seeded ``seed + 1`` until none is
    flagged.  Without ``gap_fn`` nothing is redrawn.  ``experts=False`` stops
    after w_gate (w1, w3, w2 are then empty [E, 0, 0] tensors); x and w_gate
    are the same as in the full draw, since they come first in the stream.
    """
    seed = wl.seed if seed is None else seed
    gen = torch.Generator(device=device).manual_seed(seed)
    x = _draw_x_rows(gen, wl.T, wl, device)
    w_gate = torch.randn(wl.d, wl.E, generator=gen, device=device) * wl.router_std
    if wl.bias is not None:
        w_gate[wl.d - 1, :] = torch.tensor(list(wl.bias), dtype=torch.float32, device=device)
    tdt = torch_dtype(wl.dtype)
    if not experts:
        w1 = w3 = w2 = torch.empty(wl.E, 0, 0, dtype=tdt, device=device)
    else:
        w1, w3, w2 = _draw_experts(gen, wl, device)
    x = _cast(x, wl.dtype)
    w_gate = _cast(w_gate, wl.dtype)

    redrawn = 0
    if gap_fn is not None:
        gen2 = torch.Generator(device=device).manual_seed(seed + 1)
        for _ in range(max_redraw_rounds):
            bad = gap_fn(x, w_gate)
            rows = torch.nonzero(bad.to(device), as_tuple=False).flatten()
            if rows.numel() == 0:
                break
            x[rows] = _cast(_draw_x_rows(gen2, rows.numel(), wl, device), wl.dtype)
            redrawn += rows.numel()
        else:
            raise RuntimeError(f"{wl.name}: near-tie rows persist after "
                               f"{max_redraw_rounds} redraw rounds")
    return LayerInputs(wl, x, w_gate, w1, w3, w2, redrawn)


def small_workload(T: int, d: int, f: int, E: int = 8, dtype: str = BF16,
                   seed: int = 7, bias=None, router_std: Optional[float] = None,
                   top_k: int = 2) -> Workload:
    """A parity-sized workload with the same value distributions as the
    8x7B decode/prefill recipe (router std 1/sqrt(d) unless given, so that
    logits stay O(1) at small d)."""
    rs = router_std if router_std is not None else 1.0 / math.sqrt(d)
    kname = "" if top_k == 2 else f"_k{top_k}"
    return Workload(f"small_T{T}_d{d}_f{f}_E{E}{kname}_{dtype}", T=T, d=d, f=f, E=E,
                    top_k=top_k, dtype=dtype, router_std=rs, bias=bias, seed=seed)


def make_norm_weight(d: int, seed: int, dtype: str, device: str = "cpu") -> torch.Tensor:
    """Channel weights of the RMSNorm in front of the layer: 1 + 0.1 * N(0, 1)
    from ``torch.Generator(device).manual_seed(seed)``, rounded to ``dtype``
    (synthetic stand-ins for trained rms_2 weights, which sit near 1)."""
    gen = torch.Generator(device=device).manual_seed(seed)
    g = 1.0 + 0.1 * torch.randn(d, generator=gen, device=device)
    return _cast(g, dtype)

