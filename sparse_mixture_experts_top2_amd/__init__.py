"""Top-2 sparse mixture-of-experts feed-forward layer for AMD Instinct MI355X.

Thin Python binding over ``libmoe.so`` (the C interface declared in
``include/moe.h``).  This module only checks tensors, allocates outputs and
workspace with torch, and passes device pointers and the current HIP stream
to the library; every step of the layer runs in the library's HIP kernels.
There is no CPU or PyTorch fallback: if the library is missing, calls raise.

Functions mirror the C entry points: ``route``, ``dispatch``,
``expert_gateup``, ``expert_down``, ``experts``, ``combine``, ``forward`` and
``workspace_bytes``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# MOE_LIB names another build of the same sources (the sanitizer build of
# the host code, for the CPU tests); there is no other library and no fallback.
LIB_PATH = os.environ.get("MOE_LIB") or os.path.join(_PKG, "libmoe.so")

MOE_F32, MOE_BF16 = 0, 1
MOE_OK = 0
STATUS_NAMES = ["MOE_OK", "MOE_ERR_NULL", "MOE_ERR_SHAPE", "MOE_ERR_DTYPE", "MOE_ERR_ALIGN",
                "MOE_ERR_ALIAS", "MOE_ERR_WORKSPACE", "MOE_ERR_UNSUPPORTED", "MOE_ERR_HIP",
                "MOE_ERR_SCRATCH"]
SCRATCH_BYTES = 64 << 20      # MOE_SCRATCH_BYTES: moe_forward_noalloc's fixed workspace
EXPORTED = ["moe_status_str", "moe_workspace_bytes", "moe_route", "moe_route_probs",
            "moe_dispatch",
            "moe_expert_gateup", "moe_expert_gateup_ws", "moe_expert_down", "moe_experts",
            "moe_combine",
            "moe_forward", "moe_rmsnorm_route", "moe_block_forward", "moe_quantize_int8",
            "moe_expert_gateup_w8", "moe_expert_gateup_w8_ws", "moe_expert_down_w8",
            "moe_forward_w8",
            "moe_backward_workspace_bytes", "moe_backward", "moe_forward_noalloc"]


class MoeShape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


_lib = None


def load_library(path: Optional[str] = None):
    """Load libmoe.so (raises if it is missing: there is no fallback)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"libmoe.so not found at {p}; build it with "
                           "`python -m sparse_mixture_experts_top2_amd.build`")
    lib = ctypes.CDLL(p)
    P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    S = ctypes.POINTER(MoeShape)
    lib.moe_status_str.argtypes = [I]
    lib.moe_status_str.restype = ctypes.c_char_p
    lib.moe_workspace_bytes.argtypes = [S]
    lib.moe_workspace_bytes.restype = Z
    lib.moe_route.argtypes = [S, P, P, P, P, P]
    lib.moe_route.restype = I
    lib.moe_route_probs.argtypes = [S, P, P, P, P, P, P]
    lib.moe_route_probs.restype = I
    lib.moe_dispatch.argtypes = [S, P, P, P, P, P, P, P]
    lib.moe_dispatch.restype = I
    lib.moe_expert_gateup.argtypes = [S, P, P, P, P, P, P, P]
    lib.moe_expert_gateup.restype = I
    lib.moe_expert_gateup_ws.argtypes = [S, P, P, P, P, P, P, P, Z, P]
    lib.moe_expert_gateup_ws.restype = I
    lib.moe_expert_down.argtypes = [S, P, P, P, P, P, P]
    lib.moe_expert_down.restype = I
    lib.moe_experts.argtypes = [S, P, P, P, P, P, P, P, P, Z, P]
    lib.moe_experts.restype = I
    lib.moe_combine.argtypes = [S, P, P, P, P, P]
    lib.moe_combine.restype = I
    lib.moe_forward.argtypes = [S, P, P, P, P, P, P, P, P, P, Z, P]
    lib.moe_forward.restype = I
    lib.moe_forward_noalloc.argtypes = [S, P, P, P, P, P, P, P, P, P]
    lib.moe_forward_noalloc.restype = I
    F = ctypes.c_float
    lib.moe_rmsnorm_route.argtypes = [S, P, P, F, P, P, P, P, P]
    lib.moe_rmsnorm_route.restype = I
    lib.moe_block_forward.argtypes = [S, P, P, F, P, P, P, P, P, P, P, P, P, Z, P]
    lib.moe_block_forward.restype = I
    lib.moe_quantize_int8.argtypes = [I, I, I, I, P, P, P, P]
    lib.moe_quantize_int8.restype = I
    lib.moe_expert_gateup_w8.argtypes = [S, P, P, P, P, P, P, P, P, P]
    lib.moe_expert_gateup_w8.restype = I
    lib.moe_expert_gateup_w8_ws.argtypes = [S, P, P, P, P, P, P, P, P, P, Z, P]
    lib.moe_expert_gateup_w8_ws.restype = I
    lib.moe_expert_down_w8.argtypes = [S, P, P, P, P, P, P, P]
    lib.moe_expert_down_w8.restype = I
    lib.moe_forward_w8.argtypes = [S, P, P, P, P, P, P, P, P, P, P, P, P, Z, P]
    lib.moe_forward_w8.restype = I
    lib.moe_backward_workspace_bytes.argtypes = [S]
    lib.moe_backward_workspace_bytes.restype = Z
    lib.moe_backward.argtypes = [S, P, P, P, P, P, P, P, P, P, P, P, P, Z, P]
    lib.moe_backward.restype = I
    if path is None:
        _lib = lib
    return lib


def status_str(status: int) -> str:
    return load_library().moe_status_str(status).decode()


class MoeArgumentError(ValueError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def _check(status: int, what: str):
    """Argument errors raise MoeArgumentError (a ValueError); a failed HIP
    launch raises MoeError (a RuntimeError)."""
    if status == MOE_OK:
        return
    msg = f"{what}: {status_str(status)}"
    if status == 8:
        raise MoeError(status, msg)
    raise MoeArgumentError(status, msg)


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return MOE_BF16
    if t == torch.float32:
        return MOE_F32
    raise TypeError(f"unsupported dtype {t}; the layer takes float32 or bfloat16")


def make_shape(T: int, d: int, f: int, E: int, dtype, top_k: int = 2) -> MoeShape:
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    return MoeShape(T, d, f, E, top_k, code)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype=None, device=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (the layer runs only in HIP kernels)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (dense row-major)")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def workspace_bytes(T: int, d: int, f: int, E: int, dtype, top_k: int = 2) -> int:
    shape = make_shape(T, d, f, E, dtype, top_k)
    return int(load_library().moe_workspace_bytes(ctypes.byref(shape)))


def alloc_workspace(T: int, d: int, f: int, E: int, dtype, device,
                    top_k: int = 2) -> torch.Tensor:
    n = workspace_bytes(T, d, f, E, dtype, top_k)
    if n == 0:
        raise ValueError("invalid layer shape")
    return torch.empty(n, dtype=torch.uint8, device=device)


def _routing_out(T: int, k: int, device):
    return (torch.empty(T, k, dtype=torch.int32, device=device),
            torch.empty(T, k, dtype=torch.float32, device=device))


def _routed_tokens(rows: int, top_k: int, what: str) -> int:
    if top_k < 1 or rows % top_k:
        raise ValueError(f"{what} must have top_k * T rows (top_k = {top_k}, {rows} rows)")
    return rows // top_k


def route(x: torch.Tensor, w_gate: torch.Tensor,
          top_k: int = 2) -> Tuple[torch.Tensor, torch.Tensor]:
    """Router: returns (topk_idx int32 [T,k], topk_w fp32 [T,k])."""
    _need(x, "x")
    T, d = x.shape
    _need(w_gate, "w_gate", x.dtype, x.device)
    E = w_gate.shape[1]
    _need(w_gate, "w_gate", shape=(d, E))
    idx, w = _routing_out(T, top_k, x.device)
    shape = make_shape(T, d, 8, E, x.dtype, top_k)
    st = load_library().moe_route(ctypes.byref(shape), _ptr(x), _ptr(w_gate), _ptr(idx), _ptr(w),
                                  _stream(x.device))
    _check(st, "moe_route")
    return idx, w


def route_probs(x: torch.Tensor, w_gate: torch.Tensor, top_k: int = 2,
                return_probs: bool = True):
    """Router in the page's order of steps (softmax over all experts, top-k
    of the probabilities, renormalised).  Returns (probs fp32 [T,E] or None,
    topk_idx int32 [T,k], topk_w fp32 [T,k])."""
    _need(x, "x")
    T, d = x.shape
    _need(w_gate, "w_gate", x.dtype, x.device)
    E = w_gate.shape[1]
    _need(w_gate, "w_gate", shape=(d, E))
    idx, w = _routing_out(T, top_k, x.device)
    probs = torch.empty(T, E, dtype=torch.float32, device=x.device) if return_probs else None
    shape = make_shape(T, d, 8, E, x.dtype, top_k)
    st = load_library().moe_route_probs(ctypes.byref(shape), _ptr(x), _ptr(w_gate), _ptr(probs),
                                        _ptr(idx), _ptr(w), _stream(x.device))
    _check(st, "moe_route_probs")
    return probs, idx, w


def dispatch(x: torch.Tensor, topk_idx: torch.Tensor, n_experts: int):
    """Stable grouping by expert: returns (counts [E], offsets [E+1],
    pos [T,k], xp [kT,d]); k is topk_idx's second dimension."""
    _need(x, "x")
    T, d = x.shape
    _need(topk_idx, "topk_idx", torch.int32, x.device)
    if topk_idx.dim() != 2 or topk_idx.shape[0] != T:
        raise ValueError(f"topk_idx must be [T, k] with T = {T}, got {tuple(topk_idx.shape)}")
    k = topk_idx.shape[1]
    dev = x.device
    counts = torch.empty(n_experts, dtype=torch.int32, device=dev)
    offsets = torch.empty(n_experts + 1, dtype=torch.int32, device=dev)
    pos = torch.empty(T, k, dtype=torch.int32, device=dev)
    xp = torch.empty(k * T, d, dtype=x.dtype, device=dev)
    shape = make_shape(T, d, 8, n_experts, x.dtype, k)
    st = load_library().moe_dispatch(ctypes.byref(shape), _ptr(x), _ptr(topk_idx), _ptr(counts),
                                     _ptr(offsets), _ptr(pos), _ptr(xp), _stream(dev))
    _check(st, "moe_dispatch")
    return counts, offsets, pos, xp


def _expert_args(xp, counts, offsets, w, w_name, top_k):
    _need(xp, "xp")
    R, k_in = xp.shape
    T = _routed_tokens(R, top_k, "xp / h")
    _need(w, w_name, xp.dtype, xp.device)
    E = w.shape[0]
    _need(counts, "counts", torch.int32, xp.device, (E,))
    _need(offsets, "offsets", torch.int32, xp.device, (E + 1,))
    return T, k_in, E


def expert_gateup(xp: torch.Tensor, counts: torch.Tensor, offsets: torch.Tensor,
                  w1: torch.Tensor, w3: torch.Tensor, out: Optional[torch.Tensor] = None,
                  top_k: int = 2, workspace: Optional[torch.Tensor] = None):
    """h = silu(xp w1[e]) * (xp w3[e]) per expert row group; [kT, f].  With
    a workspace (alloc_workspace) the call runs exactly the layer's kernels
    for this step (moe_expert_gateup_ws)."""
    T, d, E = _expert_args(xp, counts, offsets, w1, "w1", top_k)
    R = xp.shape[0]
    f = w1.shape[2]
    _need(w1, "w1", shape=(E, d, f))
    _need(w3, "w3", xp.dtype, xp.device, (E, d, f))
    h = out if out is not None else torch.empty(R, f, dtype=xp.dtype, device=xp.device)
    _need(h, "h", xp.dtype, xp.device, (R, f))
    shape = make_shape(T, d, f, E, xp.dtype, top_k)
    lib = load_library()
    if workspace is None:
        st = lib.moe_expert_gateup(ctypes.byref(shape), _ptr(xp), _ptr(counts), _ptr(offsets),
                                   _ptr(w1), _ptr(w3), _ptr(h), _stream(xp.device))
        _check(st, "moe_expert_gateup")
    else:
        _need(workspace, "workspace", torch.uint8, xp.device)
        st = lib.moe_expert_gateup_ws(ctypes.byref(shape), _ptr(xp), _ptr(counts),
                                      _ptr(offsets), _ptr(w1), _ptr(w3), _ptr(h),
                                      _ptr(workspace), workspace.numel(), _stream(xp.device))
        _check(st, "moe_expert_gateup_ws")
    return h


def expert_down(h: torch.Tensor, counts: torch.Tensor, offsets: torch.Tensor, w2: torch.Tensor,
                out: Optional[torch.Tensor] = None, top_k: int = 2):
    """o = h w2[e] per expert row group; fp32 [kT, d]."""
    T, f, E = _expert_args(h, counts, offsets, w2, "w2", top_k)
    R = h.shape[0]
    d = w2.shape[2]
    _need(w2, "w2", shape=(E, f, d))
    o = out if out is not None else torch.empty(R, d, dtype=torch.float32, device=h.device)
    _need(o, "o", torch.float32, h.device, (R, d))
    shape = make_shape(T, d, f, E, h.dtype, top_k)
    st = load_library().moe_expert_down(ctypes.byref(shape), _ptr(h), _ptr(counts), _ptr(offsets),
                                        _ptr(w2), _ptr(o), _stream(h.device))
    _check(st, "moe_expert_down")
    return o


def experts(xp: torch.Tensor, counts: torch.Tensor, offsets: torch.Tensor, w1: torch.Tensor,
            w3: torch.Tensor, w2: torch.Tensor, workspace: Optional[torch.Tensor] = None,
            top_k: int = 2):
    """Grouped SwiGLU over expert-sorted rows: returns o fp32 [kT, d]."""
    _need(xp, "xp")
    R, d = xp.shape
    T = _routed_tokens(R, top_k, "xp")
    _need(w1, "w1", xp.dtype, xp.device)
    E, _, f = w1.shape
    _need(w1, "w1", shape=(E, d, f))
    _need(w3, "w3", xp.dtype, xp.device, (E, d, f))
    _need(w2, "w2", xp.dtype, xp.device, (E, f, d))
    _need(counts, "counts", torch.int32, xp.device, (E,))
    _need(offsets, "offsets", torch.int32, xp.device, (E + 1,))
    ws = workspace if workspace is not None else alloc_workspace(T, d, f, E, xp.dtype, xp.device,
                                                                 top_k)
    o = torch.empty(R, d, dtype=torch.float32, device=xp.device)
    shape = make_shape(T, d, f, E, xp.dtype, top_k)
    st = load_library().moe_experts(ctypes.byref(shape), _ptr(xp), _ptr(counts), _ptr(offsets),
                                    _ptr(w1), _ptr(w3), _ptr(w2), _ptr(o), _ptr(ws),
                                    ws.numel(), _stream(xp.device))
    _check(st, "moe_experts")
    return o


def combine(o: torch.Tensor, pos: torch.Tensor, topk_w: torch.Tensor, dtype) -> torch.Tensor:
    """y[t] = sum_s w[t,s] o[pos[t,s]] over the k slots, as ``dtype``; k is
    pos's second dimension."""
    _need(o, "o", torch.float32)
    R, d = o.shape
    _need(pos, "pos", torch.int32, o.device)
    if pos.dim() != 2:
        raise ValueError(f"pos must be [T, k], got {tuple(pos.shape)}")
    T, k = pos.shape
    if R != k * T:
        raise ValueError(f"o must have k * T = {k * T} rows, got {R}")
    _need(topk_w, "topk_w", torch.float32, o.device, (T, k))
    y = torch.empty(T, d, dtype=dtype, device=o.device)
    shape = make_shape(T, d, 8, max(2, k), dtype, k)
    st = load_library().moe_combine(ctypes.byref(shape), _ptr(o), _ptr(pos), _ptr(topk_w), _ptr(y),
                                    _stream(o.device))
    _check(st, "moe_combine")
    return y


def forward(x: torch.Tensor, w_gate: torch.Tensor, w1: torch.Tensor, w3: torch.Tensor,
            w2: torch.Tensor, workspace: Optional[torch.Tensor] = None,
            return_routing: bool = False, out: Optional[torch.Tensor] = None,
            top_k: int = 2):
    """The whole layer.  Returns y [T, d] (and (topk_idx, topk_w), each
    [T, top_k], when ``return_routing``)."""
    _need(x, "x")
    T, d = x.shape
    _need(w_gate, "w_gate", x.dtype, x.device)
    E = w_gate.shape[1]
    _need(w_gate, "w_gate", shape=(d, E))
    _need(w1, "w1", x.dtype, x.device)
    f = w1.shape[2]
    _need(w1, "w1", shape=(E, d, f))
    _need(w3, "w3", x.dtype, x.device, (E, d, f))
    _need(w2, "w2", x.dtype, x.device, (E, f, d))
    ws = workspace if workspace is not None else alloc_workspace(T, d, f, E, x.dtype, x.device,
                                                                 top_k)
    y = out if out is not None else torch.empty(T, d, dtype=x.dtype, device=x.device)
    _need(y, "out", x.dtype, x.device, (T, d))
    idx = w = None
    if return_routing:
        idx, w = _routing_out(T, top_k, x.device)
    shape = make_shape(T, d, f, E, x.dtype, top_k)
    st = load_library().moe_forward(ctypes.byref(shape), _ptr(x), _ptr(w_gate), _ptr(w1), _ptr(w3),
                                    _ptr(w2), _ptr(y), _ptr(idx), _ptr(w), _ptr(ws), ws.numel(),
                                    _stream(x.device))
    _check(st, "moe_forward")
    return (y, idx, w) if return_routing else y


def forward_noalloc(x: torch.Tensor, w_gate: torch.Tensor, w1: torch.Tensor, w3: torch.Tensor,
                    w2: torch.Tensor, out: Optional[torch.Tensor] = None,
                    routing_out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None,
                    top_k: int = 2):
    """The whole layer through moe_forward_noalloc: no workspace argument
    (the library's fixed device array, SCRATCH_BYTES, serves as one).
    Returns y [T, d].  Pass ``out`` (and ``routing_out`` = (topk_idx int32
    [T, k], topk_w fp32 [T, k]) to receive the routing) so that the call
    allocates nothing, not even in this wrapper."""
    _need(x, "x")
    T, d = x.shape
    _need(w_gate, "w_gate", x.dtype, x.device)
    E = w_gate.shape[1]
    _need(w_gate, "w_gate", shape=(d, E))
    _need(w1, "w1", x.dtype, x.device)
    f = w1.shape[2]
    _need(w1, "w1", shape=(E, d, f))
    _need(w3, "w3", x.dtype, x.device, (E, d, f))
    _need(w2, "w2", x.dtype, x.device, (E, f, d))
    y = out if out is not None else torch.empty(T, d, dtype=x.dtype, device=x.device)
    _need(y, "out", x.dtype, x.device, (T, d))
    idx = w = None
    if routing_out is not None:
        idx, w = routing_out
        _need(idx, "topk_idx", torch.int32, x.device, (T, top_k))
        _need(w, "topk_w", torch.float32, x.device, (T, top_k))
    shape = make_shape(T, d, f, E, x.dtype, top_k)
    st = load_library().moe_forward_noalloc(ctypes.byref(shape), _ptr(x), _ptr(w_gate),
                                            _ptr(w1), _ptr(w3), _ptr(w2), _ptr(y), _ptr(idx),
                                            _ptr(w), _stream(x.device))
    _check(st, "moe_forward_noalloc")
    return y


def rmsnorm_route(h: torch.Tensor, rms_weight: torch.Tensor, eps: float, w_gate: torch.Tensor,
                  xn: Optional[torch.Tensor] = None, top_k: int = 2):
    """Router on RMSNorm(h).  Returns (xn [T, d], topk_idx int32 [T, k],
    topk_w fp32 [T, k])."""
    _need(h, "h")
    T, d = h.shape
    _need(rms_weight, "rms_weight", h.dtype, h.device, (d,))
    _need(w_gate, "w_gate", h.dtype, h.device)
    E = w_gate.shape[1]
    _need(w_gate, "w_gate", shape=(d, E))
    xn = xn if xn is not None else torch.empty_like(h)
    _need(xn, "xn", h.dtype, h.device, (T, d))
    idx, w = _routing_out(T, top_k, h.device)
    shape = make_shape(T, d, 8, E, h.dtype, top_k)
    st = load_library().moe_rmsnorm_route(ctypes.byref(shape), _ptr(h), _ptr(rms_weight),
                                          float(eps), _ptr(w_gate), _ptr(xn), _ptr(idx), _ptr(w),
                                          _stream(h.device))
    _check(st, "moe_rmsnorm_route")
    return xn, idx, w


def block_forward(h: torch.Tensor, rms_weight: torch.Tensor, eps: float, w_gate: torch.Tensor,
                  w1: torch.Tensor, w3: torch.Tensor, w2: torch.Tensor,
                  residual: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, return_routing: bool = False,
                  out: Optional[torch.Tensor] = None, top_k: int = 2):
    """out = residual + layer(RMSNorm(h)) (no add when residual is None).
    Returns out [T, d] (and (topk_idx, topk_w) when ``return_routing``)."""
    _need(h, "h")
    T, d = h.shape
    _need(rms_weight, "rms_weight", h.dtype, h.device, (d,))
    _need(w_gate, "w_gate", h.dtype, h.device)
    E = w_gate.shape[1]
    _need(w_gate, "w_gate", shape=(d, E))
    _need(w1, "w1", h.dtype, h.device)
    f = w1.shape[2]
    _need(w1, "w1", shape=(E, d, f))
    _need(w3, "w3", h.dtype, h.device, (E, d, f))
    _need(w2, "w2", h.dtype, h.device, (E, f, d))
    if residual is not None:
        _need(residual, "residual", h.dtype, h.device, (T, d))
    ws = workspace if workspace is not None else alloc_workspace(T, d, f, E, h.dtype, h.device,
                                                                 top_k)
    y = out if out is not None else torch.empty(T, d, dtype=h.dtype, device=h.device)
    _need(y, "out", h.dtype, h.device, (T, d))
    idx = w = None
    if return_routing:
        idx, w = _routing_out(T, top_k, h.device)
    shape = make_shape(T, d, f, E, h.dtype, top_k)
    st = load_library().moe_block_forward(ctypes.byref(shape), _ptr(h), _ptr(rms_weight),
                                          float(eps), _ptr(residual), _ptr(w_gate), _ptr(w1),
                                          _ptr(w3), _ptr(w2), _ptr(y), _ptr(idx), _ptr(w), _ptr(ws),
                                          ws.numel(), _stream(h.device))
    _check(st, "moe_block_forward")
    return (y, idx, w) if return_routing else y



# ---------------------------------------------------------------------------
# Weight-only int8 expert weights (decode sizes: bf16 layers, T <= 32).

def quantize_int8(w: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """W [n, K, N] (bf16 or fp32) -> (codes, scales fp32 [n, N]): one
    symmetric scale per output column, s = max|W| / 127, q = rint(W / s)
    clamped to [-127, 127].  The codes come in the kernels' row-pair layout,
    int8 [n, K/2, N/8, 2, 8] (element [m, j//2, c//8, j%2, c%8] is the code
    of W[m, j, c]); unpack_int8 gives them as [n, K, N]."""
    _need(w, "w")
    if w.dim() != 3:
        raise ValueError(f"w must be [n, K, N], got {tuple(w.shape)}")
    n, K, N = w.shape
    if K % 2 or N % 8:
        raise ValueError(f"K must be even and N a multiple of 8, got K={K}, N={N}")
    q = torch.empty(n, K // 2, N // 8, 2, 8, dtype=torch.int8, device=w.device)
    sc = torch.empty(n, N, dtype=torch.float32, device=w.device)
    st = load_library().moe_quantize_int8(n, K, N, _dtype_code(w.dtype), _ptr(w), _ptr(q),
                                          _ptr(sc), _stream(w.device))
    _check(st, "moe_quantize_int8")
    return q, sc


def unpack_int8(q: torch.Tensor) -> torch.Tensor:
    """Codes in the row-pair layout [n, K/2, N/8, 2, 8] -> [n, K, N]."""
    n, kh, ng, two, eight = q.shape
    if (two, eight) != (2, 8):
        raise ValueError(f"not row-pair codes: {tuple(q.shape)}")
    return q.permute(0, 1, 3, 2, 4).reshape(n, 2 * kh, 8 * ng)


def _w8_dims(q: torch.Tensor, name: str):
    """(E, K, N) of row-pair codes."""
    if q.dim() != 5 or tuple(q.shape[3:]) != (2, 8):
        raise ValueError(f"q{name} must be row-pair codes [E, K/2, N/8, 2, 8] "
                         f"(quantize_int8), got {tuple(q.shape)}")
    return q.shape[0], 2 * q.shape[1], 8 * q.shape[2]


def _need_w8(q, sc, name, device, E, K, N):
    _need(q, f"q{name}", torch.int8, device, (E, K // 2, N // 8, 2, 8))
    _need(sc, f"s{name}", torch.float32, device, (E, N))


def expert_gateup_w8(xp: torch.Tensor, counts: torch.Tensor, offsets: torch.Tensor,
                     q1: torch.Tensor, s1: torch.Tensor, q3: torch.Tensor, s3: torch.Tensor,
                     top_k: int = 2, out: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None):
    """h = silu(s1 * (xp q1[e])) * (s3 * (xp q3[e])) per expert row group.
    With the layer's workspace it runs exactly the kernels the layer runs
    for this step (moe_expert_gateup_w8_ws)."""
    _need(xp, "xp", torch.bfloat16)
    R, d = xp.shape
    T = _routed_tokens(R, top_k, "xp")
    E, _, f = _w8_dims(q1, "1")
    _need_w8(q1, s1, "1", xp.device, E, d, f)
    _need_w8(q3, s3, "3", xp.device, E, d, f)
    _need(counts, "counts", torch.int32, xp.device, (E,))
    _need(offsets, "offsets", torch.int32, xp.device, (E + 1,))
    h = out if out is not None else torch.empty(R, f, dtype=torch.bfloat16, device=xp.device)
    _need(h, "h", torch.bfloat16, xp.device, (R, f))
    shape = make_shape(T, d, f, E, torch.bfloat16, top_k)
    if workspace is None:
        st = load_library().moe_expert_gateup_w8(ctypes.byref(shape), _ptr(xp), _ptr(counts),
                                                 _ptr(offsets), _ptr(q1), _ptr(s1), _ptr(q3),
                                                 _ptr(s3), _ptr(h), _stream(xp.device))
        _check(st, "moe_expert_gateup_w8")
    else:
        _need(workspace, "workspace", torch.uint8, xp.device)
        st = load_library().moe_expert_gateup_w8_ws(ctypes.byref(shape), _ptr(xp), _ptr(counts),
                                                    _ptr(offsets), _ptr(q1), _ptr(s1), _ptr(q3),
                                                    _ptr(s3), _ptr(h), _ptr(workspace),
                                                    workspace.numel(), _stream(xp.device))
        _check(st, "moe_expert_gateup_w8_ws")
    return h


def expert_down_w8(h: torch.Tensor, counts: torch.Tensor, offsets: torch.Tensor,
                   q2: torch.Tensor, s2: torch.Tensor, top_k: int = 2,
                   out: Optional[torch.Tensor] = None):
    """o = s2 * (h q2[e]) per expert row group; fp32 [kT, d]."""
    _need(h, "h", torch.bfloat16)
    R, f = h.shape
    T = _routed_tokens(R, top_k, "h")
    E, _, d = _w8_dims(q2, "2")
    _need_w8(q2, s2, "2", h.device, E, f, d)
    _need(counts, "counts", torch.int32, h.device, (E,))
    _need(offsets, "offsets", torch.int32, h.device, (E + 1,))
    o = out if out is not None else torch.empty(R, d, dtype=torch.float32, device=h.device)
    _need(o, "o", torch.float32, h.device, (R, d))
    shape = make_shape(T, d, f, E, torch.bfloat16, top_k)
    st = load_library().moe_expert_down_w8(ctypes.byref(shape), _ptr(h), _ptr(counts),
                                           _ptr(offsets), _ptr(q2), _ptr(s2), _ptr(o),
                                           _stream(h.device))
    _check(st, "moe_expert_down_w8")
    return o


def forward_w8(x: torch.Tensor, w_gate: torch.Tensor, q1: torch.Tensor, s1: torch.Tensor,
               q3: torch.Tensor, s3: torch.Tensor, q2: torch.Tensor, s2: torch.Tensor,
               workspace: Optional[torch.Tensor] = None, return_routing: bool = False,
               out: Optional[torch.Tensor] = None, top_k: int = 2):
    """The layer with int8 expert weights (bf16 x, T <= 32).  Returns y
    [T, d] (and (topk_idx, topk_w) when ``return_routing``)."""
    _need(x, "x", torch.bfloat16)
    T, d = x.shape
    _need(w_gate, "w_gate", x.dtype, x.device)
    E = w_gate.shape[1]
    _need(w_gate, "w_gate", shape=(d, E))
    f = _w8_dims(q1, "1")[2]
    _need_w8(q1, s1, "1", x.device, E, d, f)
    _need_w8(q3, s3, "3", x.device, E, d, f)
    _need_w8(q2, s2, "2", x.device, E, f, d)
    ws = workspace if workspace is not None else alloc_workspace(T, d, f, E, x.dtype, x.device,
                                                                 top_k)
    y = out if out is not None else torch.empty(T, d, dtype=x.dtype, device=x.device)
    _need(y, "out", x.dtype, x.device, (T, d))
    idx = w = None
    if return_routing:
        idx, w = _routing_out(T, top_k, x.device)
    shape = make_shape(T, d, f, E, x.dtype, top_k)
    st = load_library().moe_forward_w8(ctypes.byref(shape), _ptr(x), _ptr(w_gate), _ptr(q1),
                                       _ptr(s1), _ptr(q3), _ptr(s3), _ptr(q2), _ptr(s2), _ptr(y),
                                       _ptr(idx), _ptr(w), _ptr(ws), ws.numel(),
                                       _stream(x.device))
    _check(st, "moe_forward_w8")
    return (y, idx, w) if return_routing else y


# ---------------------------------------------------------------------------
# Backward.

def backward_workspace_bytes(T: int, d: int, f: int, E: int, dtype, top_k: int = 2) -> int:
    shape = make_shape(T, d, f, E, dtype, top_k)
    return int(load_library().moe_backward_workspace_bytes(ctypes.byref(shape)))


def backward(x: torch.Tensor, w_gate: torch.Tensor, w1: torch.Tensor, w3: torch.Tensor,
             w2: torch.Tensor, dy: torch.Tensor, top_k: int = 2,
             workspace: Optional[torch.Tensor] = None):
    """Gradients of sum(dy * forward(x, ...)): returns (dx [T, d] in x's
    dtype, dw_gate [d, E], dw1 [E, d, f], dw3 [E, d, f], dw2 [E, f, d], all
    fp32)."""
    _need(x, "x")
    T, d = x.shape
    _need(w_gate, "w_gate", x.dtype, x.device)
    E = w_gate.shape[1]
    _need(w_gate, "w_gate", shape=(d, E))
    _need(w1, "w1", x.dtype, x.device)
    f = w1.shape[2]
    _need(w1, "w1", shape=(E, d, f))
    _need(w3, "w3", x.dtype, x.device, (E, d, f))
    _need(w2, "w2", x.dtype, x.device, (E, f, d))
    _need(dy, "dy", x.dtype, x.device, (T, d))
    n = backward_workspace_bytes(T, d, f, E, x.dtype, top_k)
    if n == 0:
        raise ValueError("invalid layer shape")
    ws = workspace if workspace is not None else torch.empty(n, dtype=torch.uint8,
                                                             device=x.device)
    dev = x.device
    dx = torch.empty_like(x)
    dwg = torch.empty(d, E, dtype=torch.float32, device=dev)
    dw1 = torch.empty(E, d, f, dtype=torch.float32, device=dev)
    dw3 = torch.empty(E, d, f, dtype=torch.float32, device=dev)
    dw2 = torch.empty(E, f, d, dtype=torch.float32, device=dev)
    shape = make_shape(T, d, f, E, x.dtype, top_k)
    st = load_library().moe_backward(ctypes.byref(shape), _ptr(x), _ptr(w_gate), _ptr(w1),
                                     _ptr(w3), _ptr(w2), _ptr(dy), _ptr(dx), _ptr(dwg), _ptr(dw1),
                                     _ptr(dw3), _ptr(dw2), _ptr(ws), ws.numel(), _stream(dev))
    _check(st, "moe_backward")
    return dx, dwg, dw1, dw3, dw2
