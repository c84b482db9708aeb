"""CPU oracle for the top-2 sparse MoE feed-forward layer.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The library's product
path never calls it, and it shares no code with the HIP library: the
arithmetic lives in ``moe_oracle.c`` (plain C, fp64), built by ``build()``
with gcc, and the integer bookkeeping below is plain Python.

Functions, each following "Mixtral 8x7B -- The Evolving Transformer",
section 05 (MOE ROUTER + MOE), and section 04 (SWIGLU):

* ``route``        router logits, top-k (Mixtral: top-2) with lowest-index
                   ties, softmax over the selected logits (MoERouter; formula
                   of section 05)
* ``route_probs``  the same router in the page's order of steps: softmax
                   over all experts, top-k of the probabilities, renormalise
* ``dispatch``     stable grouping of (token, slot) assignments by expert:
                   the per-expert token batches that section 05 says
                   production stacks form instead of looping with masks
* ``expert_rows``  one SwiGLU expert applied to given rows (section 04),
                   and its two halves ``expert_hidden`` (silu(x W1) * (x W3))
                   and ``expert_down`` (h W2)
* ``combine``      y[t] = w[t,0] o[t,0] + w[t,1] o[t,1] (formula of section 05)
* ``forward``      the whole layer, token by token
* ``quantize_int8``, ``forward_w8``  weight-only int8 expert weights (one
                   scale per output channel) and the layer on them
* ``backward``     gradients of sum(dy * y) for x, the router and the three
                   expert matrices (top-k picks held fixed)

Parity status: every function is pinned by tests/test_oracle.py against
closed forms, brute force, library routines (numpy fp64) and invariants.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")
_lib = None

ORC_F32, ORC_BF16 = 0, 1


def build(verbose: bool = False) -> str:
    """Compile the oracle with gcc: IEEE semantics (no fast-math, no FMA
    contraction), so each sum is evaluated in the order the source states."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
           "-ffp-contract=off", "-fno-fast-math", _SRC, "-lm", "-o", _LIB_PATH + ".tmp"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _bind(path: str):
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I = ctypes.c_int
    lib.oracle_route.argtypes = [I, I, I, I, P, P, I, P, P, P, I]
    lib.oracle_route.restype = I
    lib.oracle_expert_rows.argtypes = [I, I, I, I, P, P, P, P, P, I, P, I]
    lib.oracle_expert_rows.restype = I
    lib.oracle_forward.argtypes = [I, I, I, I, I, P, P, P, P, P, I, P, P, P, P, I]
    lib.oracle_forward.restype = I
    lib.oracle_expert_hidden.argtypes = [I, I, I, I, P, P, P, P, I, P, I]
    lib.oracle_expert_hidden.restype = I
    lib.oracle_expert_down.argtypes = [I, I, I, I, P, P, P, I, P, I]
    lib.oracle_expert_down.restype = I
    lib.oracle_route_probs.argtypes = [I, I, I, I, P, P, I, P, P, P, I]
    lib.oracle_route_probs.restype = I
    lib.oracle_quantize_int8.argtypes = [I, I, I, P, I, P, P, I]
    lib.oracle_quantize_int8.restype = I
    lib.oracle_forward_w8.argtypes = [I, I, I, I, I, P, P, I, P, P, P, P, P, P, P, P, P, I]
    lib.oracle_forward_w8.restype = I
    lib.oracle_expert_stage_w8.argtypes = [I, I, I, I, I, P, P, I, P, P, P, P, P, P, P, I]
    lib.oracle_expert_stage_w8.restype = I
    lib.oracle_backward.argtypes = [I, I, I, I, I, P, P, P, P, P, I, P, P, P, P, P, P, P, P, I]
    lib.oracle_backward.restype = I
    lib.oracle_rmsnorm.argtypes = [I, I, P, P, ctypes.c_double, I, P, P, I]
    lib.oracle_rmsnorm.restype = I
    return lib


def build_sanitized(out_path: str, cc: str) -> str:
    """The same source built with AddressSanitizer and UndefinedBehaviorSanitizer
    (``cc``: a clang whose runtime the test process preloads), for the
    sanitizer run of the CPU tests; loaded in place of the plain build when
    the environment names it in MOE_ORACLE_LIB."""
    cmd = [cc, "-O1", "-g", "-fno-omit-frame-pointer", "-std=c11", "-fPIC", "-shared",
           "-pthread", "-ffp-contract=off", "-fno-fast-math",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-shared-libasan",
           _SRC, "-lm", "-o", out_path]
    subprocess.run(cmd, check=True)
    return out_path


def _load():
    global _lib
    if _lib is not None:
        return _lib
    override = os.environ.get("MOE_ORACLE_LIB")
    if override:
        _lib = _bind(override)
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    _lib = _bind(_LIB_PATH)
    return _lib


def use_library(lib):
    """Swap the loaded oracle library for another build (a path or a handle
    returned earlier).  Returns the previous handle.  The pin tests use this
    to run the same checks against copies with planted mistakes."""
    global _lib
    prev = _load()
    _lib = _bind(lib) if isinstance(lib, str) else lib
    return prev


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


# ---------------------------------------------------------------------------
# Array marshalling.  Inputs are numpy fp32 arrays, or bf16 values carried as
# their uint16 bit patterns, or torch CPU tensors of either dtype.

def _as_host(a) -> Tuple[np.ndarray, int]:
    """Return (contiguous numpy array, dtype code) without changing values."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().cpu().contiguous()
            if a.dtype == torch.bfloat16:
                return a.view(torch.int16).numpy().view(np.uint16), ORC_BF16
            if a.dtype == torch.float32:
                return a.numpy(), ORC_F32
            raise TypeError(f"oracle takes fp32 or bf16 tensors, got {a.dtype}")
    except ImportError:  # pragma: no cover
        pass
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a, ORC_F32
    if a.dtype == np.uint16:
        return a, ORC_BF16
    raise TypeError(f"oracle takes float32 or bf16-bit (uint16) arrays, got {a.dtype}")


def _same_dtype(*codes):
    if len(set(codes)) != 1:
        raise TypeError("all inputs of one oracle call must share a dtype")
    return codes[0]


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


# ---------------------------------------------------------------------------

def route(x, w_gate, threads: Optional[int] = None, return_logits: bool = False,
          top_k: int = 2):
    """Router for every token: returns idx int32 [T,k] (slots in decreasing
    logit order), w float64 [T,k], and optionally logits float64 [T,E]."""
    xa, dx = _as_host(x)
    ga, dg = _as_host(w_gate)
    dt = _same_dtype(dx, dg)
    T, d = xa.shape
    d2, E = ga.shape
    assert d == d2
    idx = np.zeros((T, top_k), np.int32)
    w = np.zeros((T, top_k), np.float64)
    logits = np.zeros((T, E), np.float64)
    rc = _load().oracle_route(T, d, E, top_k, _ptr(xa), _ptr(ga), dt, _ptr(idx), _ptr(w),
                              _ptr(logits), threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_route rejected its sizes")
    return (idx, w, logits) if return_logits else (idx, w)


def route_probs(x, w_gate, top_k: int = 2, threads: Optional[int] = None):
    """The router in the page's order of steps: softmax over all E logits,
    top-k of the probabilities, kept probabilities divided by their sum.
    Returns probs float64 [T,E], idx int32 [T,k], w float64 [T,k]."""
    xa, dx = _as_host(x)
    ga, dg = _as_host(w_gate)
    dt = _same_dtype(dx, dg)
    T, d = xa.shape
    d2, E = ga.shape
    assert d == d2
    probs = np.zeros((T, E), np.float64)
    idx = np.zeros((T, top_k), np.int32)
    w = np.zeros((T, top_k), np.float64)
    rc = _load().oracle_route_probs(T, d, E, top_k, _ptr(xa), _ptr(ga), dt, _ptr(probs),
                                    _ptr(idx), _ptr(w), threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_route_probs rejected its sizes")
    return probs, idx, w


def dispatch(idx: np.ndarray, n_experts: int):
    """Group the kT (token, slot) assignments by expert, keeping token order
    and then slot order inside each expert.

    Returns counts int32 [E], offsets int32 [E+1] (exclusive prefix sum of
    counts), pos int32 [T,k] (row of assignment (t, s) in the grouped order)
    and src int32 [kT] (the flat assignment t*k+s held by each grouped row).
    """
    idx = np.asarray(idx)
    T, k = idx.shape
    counts = np.zeros(n_experts, np.int32)
    for t in range(T):
        for s in range(k):
            counts[int(idx[t, s])] += 1
    offsets = np.zeros(n_experts + 1, np.int32)
    for e in range(n_experts):
        offsets[e + 1] = offsets[e] + counts[e]
    fill = offsets[:-1].copy()
    pos = np.zeros((T, k), np.int32)
    src = np.zeros(k * T, np.int32)
    for t in range(T):
        for s in range(k):
            e = int(idx[t, s])
            pos[t, s] = fill[e]
            src[fill[e]] = k * t + s
            fill[e] += 1
    return counts, offsets, pos, src


def expert_rows(rows, expert: np.ndarray, w1, w3, w2, threads: Optional[int] = None):
    """out[r] = SwiGLU expert ``expert[r]`` applied to rows[r]; float64 [n, d]."""
    ra, dr = _as_host(rows)
    a1, d1 = _as_host(w1)
    a3, d3 = _as_host(w3)
    a2, d2 = _as_host(w2)
    dt = _same_dtype(dr, d1, d3, d2)
    n, d = ra.shape
    E, d_, f = a1.shape
    assert d_ == d and a3.shape == a1.shape and a2.shape == (E, f, d)
    ex = np.ascontiguousarray(expert, dtype=np.int32)
    assert ex.shape == (n,)
    out = np.zeros((n, d), np.float64)
    rc = _load().oracle_expert_rows(n, d, f, E, _ptr(ra), _ptr(ex), _ptr(a1), _ptr(a3),
                                    _ptr(a2), dt, _ptr(out), threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_expert_rows rejected its sizes or expert ids")
    return out


def expert_hidden(rows, expert: np.ndarray, w1, w3, threads: Optional[int] = None):
    """SwiGLU hidden activation silu(rows[r] W1[e]) * (rows[r] W3[e]),
    e = expert[r]; float64 [n, f]."""
    ra, dr = _as_host(rows)
    a1, d1 = _as_host(w1)
    a3, d3 = _as_host(w3)
    dt = _same_dtype(dr, d1, d3)
    n, d = ra.shape
    E, d_, f = a1.shape
    assert d_ == d and a3.shape == a1.shape
    ex = np.ascontiguousarray(expert, dtype=np.int32)
    assert ex.shape == (n,)
    out = np.zeros((n, f), np.float64)
    rc = _load().oracle_expert_hidden(n, d, f, E, _ptr(ra), _ptr(ex), _ptr(a1), _ptr(a3), dt,
                                      _ptr(out), threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_expert_hidden rejected its sizes or expert ids")
    return out


def expert_down(hid, expert: np.ndarray, w2, threads: Optional[int] = None):
    """Down projection hid[r] W2[e], e = expert[r]; float64 [n, d]."""
    ha, dh = _as_host(hid)
    a2, d2 = _as_host(w2)
    dt = _same_dtype(dh, d2)
    n, f = ha.shape
    E, f_, d = a2.shape
    assert f_ == f
    ex = np.ascontiguousarray(expert, dtype=np.int32)
    assert ex.shape == (n,)
    out = np.zeros((n, d), np.float64)
    rc = _load().oracle_expert_down(n, d, f, E, _ptr(ha), _ptr(ex), _ptr(a2), dt, _ptr(out),
                                    threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_expert_down rejected its sizes or expert ids")
    return out


def combine(o_slot: np.ndarray, w: np.ndarray) -> np.ndarray:
    """y[t] = w[t,0] * o_slot[t,0] + w[t,1] * o_slot[t,1] + ..., fp64, in
    slot order; o_slot is [T, k, d] (each token's expert outputs)."""
    o = np.asarray(o_slot, np.float64)
    w = np.asarray(w, np.float64)
    y = np.zeros((o.shape[0], o.shape[2]), np.float64)
    for s in range(o.shape[1]):
        y = y + w[:, s:s + 1] * o[:, s, :]
    return y


def forward(x, w_gate, w1, w3, w2, threads: Optional[int] = None, return_logits=False,
            top_k: int = 2):
    """The whole layer: returns y float64 [T,d], idx int32 [T,k], w float64
    [T,k] (and logits float64 [T,E] when asked)."""
    xa, dx = _as_host(x)
    ga, dg = _as_host(w_gate)
    a1, d1 = _as_host(w1)
    a3, d3 = _as_host(w3)
    a2, d2 = _as_host(w2)
    dt = _same_dtype(dx, dg, d1, d3, d2)
    T, d = xa.shape
    E, d_, f = a1.shape
    assert d_ == d and ga.shape == (d, E) and a3.shape == a1.shape and a2.shape == (E, f, d)
    y = np.zeros((T, d), np.float64)
    idx = np.zeros((T, top_k), np.int32)
    w = np.zeros((T, top_k), np.float64)
    logits = np.zeros((T, E), np.float64)
    rc = _load().oracle_forward(T, d, f, E, top_k, _ptr(xa), _ptr(ga), _ptr(a1), _ptr(a3),
                                _ptr(a2), dt, _ptr(y), _ptr(idx), _ptr(w), _ptr(logits),
                                threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_forward rejected its sizes")
    return (y, idx, w, logits) if return_logits else (y, idx, w)


# ---------------------------------------------------------------------------
# Block boundary ("Mixtral 8x7B -- The Evolving Transformer", section 06
# BLOCK, with the norm of section 03 RMSNORM): the layer runs on rms_2 of
# the residual stream h and its output is added back onto the stream.

def rmsnorm(h, g, eps: float, threads: Optional[int] = None):
    """xn = h * rstd * g, rounded once to h's dtype (RNE), with
    rstd[t] = 1/sqrt(mean_j h[t,j]^2 + eps) in fp64.  Returns (xn as a torch
    CPU tensor of h's dtype, rstd float64 [T])."""
    import torch
    ha, dh = _as_host(h)
    ga, dg = _as_host(g)
    dt = _same_dtype(dh, dg)
    T, d = ha.shape
    assert ga.shape == (d,)
    xn = np.zeros_like(ha)
    rstd = np.zeros(T, np.float64)
    rc = _load().oracle_rmsnorm(T, d, _ptr(ha), _ptr(ga), ctypes.c_double(eps), dt, _ptr(xn),
                                _ptr(rstd), threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_rmsnorm rejected its sizes or eps")
    out = torch.from_numpy(xn.view(np.int16)).view(torch.bfloat16) if dt == ORC_BF16 \
        else torch.from_numpy(xn)
    return out, rstd


def block_forward(h, g, eps: float, w_gate, w1, w3, w2, residual=None,
                  threads: Optional[int] = None, top_k: int = 2):
    """out = residual + layer(rmsnorm(h)) in fp64 (residual None: no add).
    Returns (out float64 [T,d], idx, w, xn)."""
    xn, _ = rmsnorm(h, g, eps, threads=threads)
    y, idx, w = forward(xn, w_gate, w1, w3, w2, threads=threads, top_k=top_k)
    if residual is not None:
        ra, code = _as_host(residual)
        y = y + _to_f64(ra, code)
    return y, idx, w, xn


def _to_f64(a: np.ndarray, code: int) -> np.ndarray:
    """Exact widening of an fp32 array or bf16 bit patterns to float64."""
    if code == ORC_F32:
        return a.astype(np.float64)
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# Near-tie screening, used to keep the routing decision unambiguous in parity
# inputs: a token whose 1st/2nd or 2nd/3rd largest logits lie within ``gap``
# of each other could be routed differently by any change of summation order.

NEAR_TIE_GAP = 1e-3


def near_tie_tokens(x, w_gate, gap: float = NEAR_TIE_GAP, threads: Optional[int] = None,
                    top_k: int = 2):
    """Bool [T]: tokens whose fp64 logits have a gap < gap between the
    s-th and (s+1)-th largest for some s <= top_k (1st/2nd and 2nd/3rd for
    top-2): the picks and their order must be clear."""
    import torch
    _, _, logits = route(x, w_gate, threads=threads, return_logits=True, top_k=1)
    srt = -np.sort(-logits, axis=1)
    bad = np.zeros(logits.shape[0], bool)
    for s in range(min(top_k, logits.shape[1] - 1)):
        bad |= (srt[:, s] - srt[:, s + 1] < gap)
    return torch.from_numpy(bad)


# ---------------------------------------------------------------------------
# Weight-only int8 expert weights (one fp32 scale per output channel).

def quantize_int8(w, threads: Optional[int] = None):
    """W [E, K, N] (fp32 or bf16) -> (q int8 [E, K, N], scale float32 [E, N]):
    s[n] = max_j |W[j,n]| / 127 and q = rint(W / s) clamped to [-127, 127],
    both in fp32; a zero column gets s = 0 and q = 0."""
    wa, dw = _as_host(w)
    E, K, N = wa.shape
    q = np.zeros((E, K, N), np.int8)
    scale = np.zeros((E, N), np.float32)
    rc = _load().oracle_quantize_int8(E, K, N, _ptr(wa), dw, _ptr(q), _ptr(scale),
                                      threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_quantize_int8 rejected its sizes")
    return q, scale


def forward_w8(x, w_gate, q1, s1, q3, s3, q2, s2, top_k: int = 2,
               threads: Optional[int] = None):
    """The layer with int8 expert weights W~ = s * q (router and x in their
    own dtype): returns y float64 [T,d], idx int32 [T,k], w float64 [T,k]."""
    xa, dx = _as_host(x)
    ga, dg = _as_host(w_gate)
    dt = _same_dtype(dx, dg)
    T, d = xa.shape
    E = ga.shape[1]
    f = q1.shape[2]
    arrs = [np.ascontiguousarray(a) for a in (q1, s1, q3, s3, q2, s2)]
    for a, dtype, shape in zip(arrs, (np.int8, np.float32) * 3,
                               ((E, d, f), (E, f), (E, d, f), (E, f), (E, f, d), (E, d))):
        if a.dtype != dtype or a.shape != shape:
            raise ValueError(f"int8 weights: expected {dtype.__name__} {shape}, got "
                             f"{a.dtype} {a.shape}")
    y = np.zeros((T, d), np.float64)
    idx = np.zeros((T, top_k), np.int32)
    w = np.zeros((T, top_k), np.float64)
    rc = _load().oracle_forward_w8(T, d, f, E, top_k, _ptr(xa), _ptr(ga), dt,
                                   *[_ptr(a) for a in arrs], _ptr(y), _ptr(idx), _ptr(w),
                                   threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_forward_w8 rejected its sizes")
    return y, idx, w


def _w8_stage(mode, rows, expert, d, f, E, mats, threads):
    ra, dr = _as_host(rows)
    n = ra.shape[0]
    ex = np.ascontiguousarray(expert, np.int32)
    z8, z32 = np.zeros(1, np.int8), np.zeros(1, np.float32)
    arrs = [np.ascontiguousarray(a) if a is not None else z for a, z in
            zip(mats, (z8, z32) * 3)]
    out = np.zeros((n, f if mode == 0 else d), np.float64)
    rc = _load().oracle_expert_stage_w8(mode, n, d, f, E, _ptr(ra), _ptr(ex), dr,
                                        *[_ptr(a) for a in arrs], _ptr(out),
                                        threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_expert_stage_w8 rejected its sizes")
    return out


def expert_hidden_w8(rows, expert: np.ndarray, q1, s1, q3, s3, threads: Optional[int] = None):
    """silu(s1 * (rows[r] q1[e])) * (s3 * (rows[r] q3[e])), e = expert[r];
    float64 [n, f]."""
    E, d, f = q1.shape
    return _w8_stage(0, rows, expert, d, f, E, (q1, s1, q3, s3, None, None), threads)


def expert_down_w8(hid, expert: np.ndarray, q2, s2, threads: Optional[int] = None):
    """s2 * (hid[r] q2[e]), e = expert[r]; float64 [n, d]."""
    E, f, d = q2.shape
    return _w8_stage(1, hid, expert, d, f, E, (None, None, None, None, q2, s2), threads)


# ---------------------------------------------------------------------------
# Backward.

def backward(x, w_gate, w1, w3, w2, dy, top_k: int = 2, threads: Optional[int] = None):
    """Gradients of L = sum(dy * y) with y = forward(x, ...): returns a dict
    with dx [T,d], dw_gate [d,E], dw1, dw3 [E,d,f], dw2 [E,f,d] (float64),
    and the routing idx [T,k], w [T,k].  dy is any float array [T,d]; it is
    used in float64 as given."""
    xa, dx_ = _as_host(x)
    ga, dg_ = _as_host(w_gate)
    a1, d1 = _as_host(w1)
    a3, d3 = _as_host(w3)
    a2, d2 = _as_host(w2)
    dt = _same_dtype(dx_, dg_, d1, d3, d2)
    try:
        import torch
        if isinstance(dy, torch.Tensor):
            dy = dy.detach().cpu().double().numpy()
    except ImportError:  # pragma: no cover
        pass
    dya = np.ascontiguousarray(dy, np.float64)
    T, d = xa.shape
    E = ga.shape[1]
    f = a1.shape[2]
    assert dya.shape == (T, d)
    out = {"dx": np.zeros((T, d)), "dw_gate": np.zeros((d, E)), "dw1": np.zeros((E, d, f)),
           "dw3": np.zeros((E, d, f)), "dw2": np.zeros((E, f, d)),
           "idx": np.zeros((T, top_k), np.int32), "w": np.zeros((T, top_k))}
    rc = _load().oracle_backward(T, d, f, E, top_k, _ptr(xa), _ptr(ga), _ptr(a1), _ptr(a3),
                                 _ptr(a2), dt, _ptr(dya), _ptr(out["dx"]), _ptr(out["dw_gate"]),
                                 _ptr(out["dw1"]), _ptr(out["dw3"]), _ptr(out["dw2"]),
                                 _ptr(out["idx"]), _ptr(out["w"]), threads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle_backward failed ({rc})")
    return out
