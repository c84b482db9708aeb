"""Canary runs of the layer, the block, the int8 layer and the backward:
every output, routing buffer and workspace sits between guard regions, and
all of it (guards, outputs, workspace) starts filled with 0xFF bytes, a NaN
in bf16 and fp32 and -1 as an integer.  After the call through the C
interface:

* every guard byte is still 0xFF (nothing is written outside its buffer);
* every output is finite and bit-identical to the same call made on freshly
  allocated buffers (so nothing read an output or workspace location that
  the call did not write first: a NaN or a -1 would have reached it);
* the routing indices lie in [0, E).

Shapes are ragged (rows, columns and K not multiples of the tiles) and
cover the generic, the 256x256-tile and the decode paths."""
import ctypes

import pytest
import torch

import sparse_mixture_experts_top2_amd as moe
from sparse_mixture_experts_top2_amd import workloads as W

from helpers import checked_block_inputs, checked_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GUARD = 1 << 16          # bytes on each side of every buffer
EPS = 1e-5


def announce(msg):
    print(f"[gpu-canary] {msg}", flush=True)


class Guarded:
    """nbytes of device memory with GUARD bytes on each side, all 0xFF."""

    def __init__(self, nbytes):
        self.n = int(nbytes)
        self.buf = torch.full((self.n + 2 * GUARD,), 0xFF, dtype=torch.uint8, device=DEV)
        self.inner = self.buf[GUARD:GUARD + self.n]

    def view(self, dtype, *shape):
        return self.inner.view(dtype).view(*shape)

    @property
    def ptr(self):
        return ctypes.c_void_p(self.inner.data_ptr())

    def guards_intact(self):
        return bool((self.buf[:GUARD] == 0xFF).all()) and bool((self.buf[GUARD + self.n:] == 0xFF).all())


def esize(dtype):
    return torch.empty(0, dtype=dtype).element_size()


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def check(name, guarded, got, ref):
    for gb in guarded:
        assert gb.guards_intact(), f"{name}: a guard byte changed"
    for g, r in zip(got, ref):
        assert torch.isfinite(g.float()).all(), f"{name}: non-finite output"
        assert torch.equal(bits(g), bits(r)), f"{name}: differs from the plain call"


P = ctypes.c_void_p


def ptr(t):
    return P(t.data_ptr())


def stream():
    return P(torch.cuda.current_stream().cuda_stream)


sw = W.small_workload
FWD = [sw(77, 200, 328, seed=501), sw(300, 256, 512, seed=502), sw(13, 256, 512, seed=503),
       sw(150, 128, 256, E=16, top_k=3, seed=504), sw(5, 200, 328, dtype=W.F32, seed=505)]


def routing(T, k):
    gi, gw = Guarded(T * k * 4), Guarded(T * k * 4)
    return gi, gw, gi.view(torch.int32, T, k), gw.view(torch.float32, T, k)


@pytest.mark.parametrize("wl", FWD, ids=lambda w: w.name)
def test_forward_canary(wl):
    announce(f"forward {wl.name}")
    g = checked_inputs(wl).to(DEV)
    T, d, f, E, k = wl.T, wl.d, wl.f, wl.E, wl.top_k
    dt = g.x.dtype
    ref_y, ref_i, ref_w = moe.forward(g.x, g.w_gate, g.w1, g.w3, g.w2, return_routing=True,
                                      top_k=k)
    gy = Guarded(T * d * esize(dt))
    gi, gw, idx, w = routing(T, k)
    ws = Guarded(moe.workspace_bytes(T, d, f, E, dt, k))
    shape = moe.make_shape(T, d, f, E, dt, k)
    st = moe.load_library().moe_forward(ctypes.byref(shape), ptr(g.x), ptr(g.w_gate), ptr(g.w1),
                                        ptr(g.w3), ptr(g.w2), gy.ptr, gi.ptr, gw.ptr, ws.ptr,
                                        ws.n, stream())
    assert st == 0, moe.status_str(st)
    torch.cuda.synchronize()
    check("moe_forward", (gy, gi, gw, ws), (gy.view(dt, T, d), idx, w), (ref_y, ref_i, ref_w))
    assert int(idx.min()) >= 0 and int(idx.max()) < E


@pytest.mark.parametrize("wl", FWD[:4], ids=lambda w: w.name)
def test_block_forward_canary(wl):
    announce(f"block_forward {wl.name}")
    gn = W.make_norm_weight(wl.d, 91, wl.dtype)
    inp = checked_block_inputs(wl, gn, EPS)
    g = inp.to(DEV)
    gn = gn.to(DEV)
    T, d, f, E, k = wl.T, wl.d, wl.f, wl.E, wl.top_k
    dt = g.x.dtype
    ref = moe.block_forward(g.x, gn, EPS, g.w_gate, g.w1, g.w3, g.w2, residual=g.x,
                            return_routing=True, top_k=k)
    gy = Guarded(T * d * esize(dt))
    gi, gw, idx, w = routing(T, k)
    ws = Guarded(moe.workspace_bytes(T, d, f, E, dt, k))
    shape = moe.make_shape(T, d, f, E, dt, k)
    st = moe.load_library().moe_block_forward(ctypes.byref(shape), ptr(g.x), ptr(gn), float(EPS),
                                              ptr(g.x), ptr(g.w_gate), ptr(g.w1), ptr(g.w3),
                                              ptr(g.w2), gy.ptr, gi.ptr, gw.ptr, ws.ptr, ws.n,
                                              stream())
    assert st == 0, moe.status_str(st)
    torch.cuda.synchronize()
    check("moe_block_forward", (gy, gi, gw, ws), (gy.view(dt, T, d), idx, w), ref)


@pytest.mark.parametrize("wl", [sw(17, 256, 512, seed=511), sw(32, 200, 328, seed=512),
                                sw(9, 4096, 336, E=3, seed=513)], ids=lambda w: w.name)
def test_forward_w8_canary(wl):
    announce(f"forward_w8 {wl.name}")
    g = checked_inputs(wl).to(DEV)
    T, d, f, E, k = wl.T, wl.d, wl.f, wl.E, wl.top_k
    qs = []
    for m in (g.w1, g.w3, g.w2):
        qs += list(moe.quantize_int8(m))
    ref = moe.forward_w8(g.x, g.w_gate, *qs, return_routing=True, top_k=k)
    gy = Guarded(T * d * 2)
    gi, gw, idx, w = routing(T, k)
    ws = Guarded(moe.workspace_bytes(T, d, f, E, torch.bfloat16, k))
    shape = moe.make_shape(T, d, f, E, torch.bfloat16, k)
    st = moe.load_library().moe_forward_w8(ctypes.byref(shape), ptr(g.x), ptr(g.w_gate),
                                           *[ptr(q) for q in qs], gy.ptr, gi.ptr, gw.ptr, ws.ptr,
                                           ws.n, stream())
    assert st == 0, moe.status_str(st)
    torch.cuda.synchronize()
    check("moe_forward_w8", (gy, gi, gw, ws), (gy.view(torch.bfloat16, T, d), idx, w), ref)


@pytest.mark.parametrize("wl", [sw(77, 200, 328, seed=521), sw(300, 256, 512, seed=522),
                                sw(16, 256, 512, seed=523), sw(40, 128, 256, dtype=W.F32,
                                                                seed=524)],
                         ids=lambda w: w.name)
def test_backward_canary(wl):
    announce(f"backward {wl.name}")
    g = checked_inputs(wl).to(DEV)
    T, d, f, E, k = wl.T, wl.d, wl.f, wl.E, wl.top_k
    dt = g.x.dtype
    gen = torch.Generator().manual_seed(wl.seed + 1)
    dy = torch.randn(T, d, generator=gen).to(dt).to(DEV)
    ref = moe.backward(g.x, g.w_gate, g.w1, g.w3, g.w2, dy, top_k=k)
    outs = [Guarded(T * d * esize(dt)), Guarded(d * E * 4), Guarded(E * d * f * 4),
            Guarded(E * d * f * 4), Guarded(E * f * d * 4)]
    ws = Guarded(moe.backward_workspace_bytes(T, d, f, E, dt, k))
    shape = moe.make_shape(T, d, f, E, dt, k)
    st = moe.load_library().moe_backward(ctypes.byref(shape), ptr(g.x), ptr(g.w_gate), ptr(g.w1),
                                         ptr(g.w3), ptr(g.w2), ptr(dy), *[o.ptr for o in outs],
                                         ws.ptr, ws.n, stream())
    assert st == 0, moe.status_str(st)
    torch.cuda.synchronize()
    views = (outs[0].view(dt, T, d), outs[1].view(torch.float32, d, E),
             outs[2].view(torch.float32, E, d, f), outs[3].view(torch.float32, E, d, f),
             outs[4].view(torch.float32, E, f, d))
    check("moe_backward", outs + [ws], views, ref)
