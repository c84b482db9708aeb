"""The C-ABI library without a GPU: it loads, exports every entry point that
include/moe.h declares, and rejects bad arguments before touching any
device memory (every call here returns from its argument checks)."""
import ctypes
import os
import re
import subprocess

import pytest

import sparse_mixture_experts_top2_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

P16 = ctypes.c_void_p(0x10000)   # aligned fake pointers: never dereferenced here
P16B = ctypes.c_void_p(0x90000000)
P17 = ctypes.c_void_p(0x10001)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(moe.EXPORTED)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", moe.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (moe_\w+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(moe.load_library(), name)
    # and nothing else: the C++ internals are built with hidden visibility
    code = set(re.findall(r"\b[TW] (\S+)", out))
    assert code == set(declared_functions()), sorted(code - set(declared_functions()))


def shape(T=64, d=128, f=256, E=8, k=2, dtype=moe.MOE_BF16):
    return moe.MoeShape(T, d, f, E, k, dtype)


def call_forward(s, ws_bytes=1 << 40, x=P16, y=P16B, ws=P16):
    lib = moe.load_library()
    return lib.moe_forward(ctypes.byref(s) if s is not None else None, x, P16, P16, P16, P16, y,
                           None, None, ws, ws_bytes, None)


def test_status_strings():
    for code, name in enumerate(moe.STATUS_NAMES):
        assert moe.status_str(code).startswith(name)
    assert moe.status_str(99) == "unknown moe status"


@pytest.mark.parametrize("bad,expect", [
    (dict(k=0), "MOE_ERR_UNSUPPORTED"), (dict(k=5, E=8), "MOE_ERR_UNSUPPORTED"),
    (dict(k=3, E=2), "MOE_ERR_UNSUPPORTED"), (dict(k=-1), "MOE_ERR_UNSUPPORTED"),
    (dict(E=1, k=1), "MOE_ERR_UNSUPPORTED"), (dict(E=65), "MOE_ERR_UNSUPPORTED"),
    (dict(T=(1 << 27) + 1, k=4), "MOE_ERR_SHAPE"),
    (dict(T=-1), "MOE_ERR_SHAPE"), (dict(d=100), "MOE_ERR_SHAPE"), (dict(f=12), "MOE_ERR_SHAPE"),
    (dict(d=0), "MOE_ERR_SHAPE"), (dict(dtype=7), "MOE_ERR_DTYPE"),
])
def test_shape_checks(bad, expect):
    s = shape(**bad)
    st = call_forward(s)
    assert moe.STATUS_NAMES[st] == expect
    assert moe.load_library().moe_workspace_bytes(ctypes.byref(s)) == 0


@pytest.mark.parametrize("E,k", [(2, 1), (2, 2), (8, 1), (8, 3), (8, 4), (16, 4), (33, 2),
                                 (64, 1), (64, 4), (4, 4)])
def test_supported_routings(E, k):
    # every E in [2, 64] with k in [1, min(4, E)] passes the shape check
    s = shape(E=E, k=k)
    assert call_forward(shape(T=0, E=E, k=k)) == moe.MOE_OK
    assert moe.load_library().moe_workspace_bytes(ctypes.byref(s)) > 0


def test_workspace_scales_with_top_k():
    lib = moe.load_library()
    sizes = [lib.moe_workspace_bytes(ctypes.byref(shape(T=256, E=8, k=k))) for k in (1, 2, 3, 4)]
    assert sizes == sorted(sizes) and len(set(sizes)) == 4
    # the routed rows (xp, h, o: bf16 d + bf16 f + fp32 d per row) grow by T per extra slot
    assert sizes[3] - sizes[2] >= 256 * (128 * 2 + 256 * 2 + 128 * 4)


def test_null_alignment_alias_workspace_checks():
    lib = moe.load_library()
    s = shape()
    need = lib.moe_workspace_bytes(ctypes.byref(s))
    assert need > 0
    assert moe.STATUS_NAMES[call_forward(None)] == "MOE_ERR_NULL"
    assert moe.STATUS_NAMES[call_forward(s, x=None)] == "MOE_ERR_NULL"
    assert moe.STATUS_NAMES[call_forward(s, x=P17)] == "MOE_ERR_ALIGN"
    assert moe.STATUS_NAMES[call_forward(s, y=P16)] == "MOE_ERR_ALIAS"
    assert moe.STATUS_NAMES[call_forward(s, ws_bytes=need - 1)] == "MOE_ERR_WORKSPACE"
    assert moe.STATUS_NAMES[call_forward(s, ws=None)] == "MOE_ERR_WORKSPACE"
    st = lib.moe_route(ctypes.byref(s), P16, P16, P17, P16, None)
    assert moe.STATUS_NAMES[st] == "MOE_ERR_ALIGN"
    st = lib.moe_dispatch(ctypes.byref(s), P16, P16, P16, P16, P16, P16, None)
    assert moe.STATUS_NAMES[st] == "MOE_ERR_ALIAS"
    # page-form router: null, alignment and every output-overlap case
    rp = lambda x, g, p, i, w: moe.STATUS_NAMES[lib.moe_route_probs(ctypes.byref(s), x, g, p,
                                                                     i, w, None)]
    A, B, C, D, G = (ctypes.c_void_p(0x10000000 * n) for n in (1, 2, 3, 4, 5))
    assert rp(A, G, None, C, None) == "MOE_ERR_NULL"
    assert rp(None, G, B, C, D) == "MOE_ERR_NULL"
    assert rp(A, G, P17, C, D) == "MOE_ERR_ALIGN"
    assert rp(A, G, B, C, P17) == "MOE_ERR_ALIGN"
    assert rp(A, G, A, C, D) == "MOE_ERR_ALIAS"       # probs over x
    assert rp(A, G, B, G, D) == "MOE_ERR_ALIAS"       # idx over w_gate
    assert rp(A, G, B, B, D) == "MOE_ERR_ALIAS"       # idx over probs
    assert rp(A, G, None, C, C) == "MOE_ERR_ALIAS"    # w over idx
    assert rp(A, G, B, C, ctypes.c_void_p(0x30000000 + 64 * 2 * 4 - 16)) == "MOE_ERR_ALIAS"
    st = lib.moe_combine(ctypes.byref(s), P16, P16, P16, None, None)
    assert moe.STATUS_NAMES[st] == "MOE_ERR_NULL"
    st = lib.moe_experts(ctypes.byref(s), P16, P16, P16, P16, P16, P16, P16B, P16, 16, None)
    assert moe.STATUS_NAMES[st] == "MOE_ERR_WORKSPACE"


def call_block(s, h=P16, g=P16, eps=1e-5, res=None, out=P16B, ws=P16, ws_bytes=1 << 40):
    lib = moe.load_library()
    return lib.moe_block_forward(ctypes.byref(s), h, g, eps, res, P16, P16, P16, P16, out, None,
                                 None, ws, ws_bytes, None)


def test_block_boundary_checks():
    lib = moe.load_library()
    s = shape()
    name = lambda st: moe.STATUS_NAMES[st]
    assert name(call_block(s, g=None)) == "MOE_ERR_NULL"
    assert name(call_block(s, h=None)) == "MOE_ERR_NULL"
    assert name(call_block(s, eps=-1.0)) == "MOE_ERR_SHAPE"
    assert name(call_block(s, eps=float("nan"))) == "MOE_ERR_SHAPE"
    assert name(call_block(s, eps=float("inf"))) == "MOE_ERR_SHAPE"
    assert name(call_block(s, g=P17)) == "MOE_ERR_ALIGN"
    assert name(call_block(s, res=P17)) == "MOE_ERR_ALIGN"
    assert name(call_block(s, ws_bytes=16)) == "MOE_ERR_WORKSPACE"
    # out may be exactly h or exactly the residual, never a shifted view of them
    row = 128 * 2
    shifted = ctypes.c_void_p(0x10000 + row)
    assert name(call_block(s, out=shifted)) == "MOE_ERR_ALIAS"
    assert name(call_block(s, res=P16B, out=ctypes.c_void_p(0x90000000 + row))) == \
        "MOE_ERR_ALIAS"
    assert call_block(shape(T=0), out=P16) == moe.MOE_OK
    st = lib.moe_rmsnorm_route(ctypes.byref(s), P16, P16, 1e-5, P16, P16, P16B, P16B, None)
    assert name(st) == "MOE_ERR_ALIAS"          # xn written over h
    st = lib.moe_rmsnorm_route(ctypes.byref(s), P16, None, 1e-5, P16, P16B, P16, P16, None)
    assert name(st) == "MOE_ERR_NULL"


def test_zero_tokens_is_a_valid_no_op():
    # T = 0 passes every check and returns before any HIP call.
    s = shape(T=0)
    assert moe.load_library().moe_workspace_bytes(ctypes.byref(s)) > 0
    assert call_forward(s) == moe.MOE_OK


def test_workspace_grows_with_every_dimension():
    lib = moe.load_library()
    base = lib.moe_workspace_bytes(ctypes.byref(shape()))
    for kw in (dict(T=65), dict(d=136), dict(f=264)):
        assert lib.moe_workspace_bytes(ctypes.byref(shape(**kw))) > base, kw
    # decode shape: xp 64 x 4096 bf16, h 64 x 14336 bf16, o 64 x 4096 fp32 and small tables
    s = shape(T=32, d=4096, f=14336)
    assert lib.moe_workspace_bytes(ctypes.byref(s)) >= 64 * (4096 * 2 + 14336 * 2 + 4096 * 4)
    # bf16 prefill: o holds the down product's two K parts
    s = shape(T=4096, d=4096, f=14336)
    assert lib.moe_workspace_bytes(ctypes.byref(s)) >= 8192 * (4096 * 2 + 14336 * 2 + 2 * 4096 * 4)
    # fp32 prefill: one o, 4-byte xp and h
    s = shape(T=4096, d=4096, f=14336, dtype=moe.MOE_F32)
    assert lib.moe_workspace_bytes(ctypes.byref(s)) >= 8192 * (4096 * 4 + 14336 * 4 + 4096 * 4)


def test_gateup_with_workspace_checks():
    lib = moe.load_library()
    name = lambda st: moe.STATUS_NAMES[st]
    s = shape(T=32, d=256, f=512)
    need = lib.moe_workspace_bytes(ctypes.byref(s))
    W0 = 0x40000000
    tail = ctypes.c_void_p(W0 + need - 1024)   # inside the partial-sum region (last)

    def G(xp=P16, c=P16, o=P16, h=P16B, ws=ctypes.c_void_p(W0), n=need, sh=s):
        return name(lib.moe_expert_gateup_ws(ctypes.byref(sh), xp, c, o, P16, P16, h, ws, n,
                                             None))
    assert G(ws=None) == "MOE_ERR_NULL"
    assert G(h=None) == "MOE_ERR_NULL"
    assert G(ws=P17) == "MOE_ERR_ALIGN"
    assert G(n=need - 1) == "MOE_ERR_WORKSPACE"
    assert G(h=P16) == "MOE_ERR_ALIAS"        # h over xp
    assert G(h=tail) == "MOE_ERR_ALIAS"       # h inside the region the call writes
    assert G(c=tail) == "MOE_ERR_ALIAS"       # counts there
    assert G(o=tail) == "MOE_ERR_ALIAS"       # offsets there
    assert G(xp=tail) == "MOE_ERR_ALIAS"      # xp there
    assert G(sh=shape(T=0)) == "MOE_OK"

    # the int8 gate/up stage with the workspace: the same checks, plus the
    # int8 calls' own limits (decode sizes, bf16 activations)
    def G8(xp=P16, c=P16, o=P16, h=P16B, ws=ctypes.c_void_p(W0), n=need, sh=s):
        return name(lib.moe_expert_gateup_w8_ws(ctypes.byref(sh), xp, c, o, P16, P16, P16, P16,
                                                h, ws, n, None))
    assert G8(ws=None) == "MOE_ERR_NULL"
    assert G8(h=None) == "MOE_ERR_NULL"
    assert G8(ws=P17) == "MOE_ERR_ALIGN"
    assert G8(n=need - 1) == "MOE_ERR_WORKSPACE"
    assert G8(h=P16) == "MOE_ERR_ALIAS"
    assert G8(h=tail) == "MOE_ERR_ALIAS"
    assert G8(c=tail) == "MOE_ERR_ALIAS"
    assert G8(o=tail) == "MOE_ERR_ALIAS"
    assert G8(xp=tail) == "MOE_ERR_ALIAS"
    assert G8(sh=shape(T=0)) == "MOE_OK"
    assert G8(sh=shape(T=40)) == "MOE_ERR_UNSUPPORTED"
    assert G8(sh=shape(T=16, dtype=moe.MOE_F32)) == "MOE_ERR_UNSUPPORTED"


def test_python_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(4, 16, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        moe.route(x, torch.zeros(16, 8, dtype=torch.bfloat16))


def test_int8_row_pair_layout():
    """unpack_int8 inverts the byte layout the header documents: code of
    W[m, j, n] at byte m*K*N + ((j/2)*(N/8) + n/8)*16 + (j%2)*8 + n%8."""
    import torch
    n, K, N = 2, 6, 24
    plain = (torch.arange(n * K * N, dtype=torch.int32) % 251 - 125).to(torch.int8).reshape(n, K, N)
    packed = torch.empty(n * K * N, dtype=torch.int8)
    for m in range(n):
        for j in range(K):
            for c in range(N):
                at = m * K * N + ((j // 2) * (N // 8) + c // 8) * 16 + (j % 2) * 8 + c % 8
                packed[at] = plain[m, j, c]
    assert torch.equal(moe.unpack_int8(packed.reshape(n, K // 2, N // 8, 2, 8)), plain)


def test_int8_weight_checks():
    lib = moe.load_library()
    name = lambda st: moe.STATUS_NAMES[st]
    Q = lambda *a: name(lib.moe_quantize_int8(*a))
    A, B, C = (ctypes.c_void_p(0x10000000 * n) for n in (1, 2, 3))
    assert Q(2, 64, 256, 7, A, B, C, None) == "MOE_ERR_DTYPE"
    assert Q(0, 64, 256, moe.MOE_BF16, A, B, C, None) == "MOE_ERR_SHAPE"
    assert Q(2, 64, 12, moe.MOE_BF16, A, B, C, None) == "MOE_ERR_SHAPE"
    assert Q(2, 0, 256, moe.MOE_BF16, A, B, C, None) == "MOE_ERR_SHAPE"
    assert Q(2, 63, 256, moe.MOE_BF16, A, B, C, None) == "MOE_ERR_SHAPE"   # K odd: no row pairs
    assert Q(70000, 8, 8, moe.MOE_BF16, A, B, C, None) == "MOE_ERR_SHAPE"
    assert Q(2, 64, 256, moe.MOE_BF16, None, B, C, None) == "MOE_ERR_NULL"
    assert Q(2, 64, 256, moe.MOE_BF16, A, P17, C, None) == "MOE_ERR_ALIGN"
    assert Q(2, 64, 256, moe.MOE_BF16, A, ctypes.c_void_p(0x10000000 + 4096), C, None) == \
        "MOE_ERR_ALIAS"                                   # codes over the weights
    assert Q(2, 64, 256, moe.MOE_BF16, A, B, ctypes.c_void_p(0x20000000 + 256), None) == \
        "MOE_ERR_ALIAS"                                   # scales over the codes
    # the layer calls: bf16 at decode sizes only
    F = lambda s: name(lib.moe_forward_w8(ctypes.byref(s), P16, P16, P16, P16, P16, P16, P16,
                                          P16, P16B, None, None, P16, 1 << 40, None))
    assert F(shape(T=33)) == "MOE_ERR_UNSUPPORTED"
    assert F(shape(T=16, dtype=moe.MOE_F32)) == "MOE_ERR_UNSUPPORTED"
    assert F(shape(T=16, k=5)) == "MOE_ERR_UNSUPPORTED"
    assert F(shape(T=0)) == "MOE_OK"
    assert F(shape(T=16, d=32768, f=65536)) == "MOE_ERR_SHAPE"   # codes past 32-bit offsets
    assert F(shape(T=0, d=32768, f=65536)) == "MOE_ERR_SHAPE"
    s = shape(T=16)
    assert name(lib.moe_forward_w8(ctypes.byref(s), P16, P16, None, P16, P16, P16, P16, P16,
                                   P16B, None, None, P16, 1 << 40, None)) == "MOE_ERR_NULL"
    assert name(lib.moe_forward_w8(ctypes.byref(s), P16, P16, P16, P17, P16, P16, P16, P16,
                                   P16B, None, None, P16, 1 << 40, None)) == "MOE_ERR_ALIGN"
    assert name(lib.moe_forward_w8(ctypes.byref(s), P16, P16, P16, P16, P16, P16, P16, P16,
                                   P16, None, None, P16B, 1 << 40, None)) == "MOE_ERR_ALIAS"
    assert name(lib.moe_forward_w8(ctypes.byref(s), P16, P16, P16, P16, P16, P16, P16, P16,
                                   P16B, None, None, P16, 16, None)) == "MOE_ERR_WORKSPACE"
    G = lambda s: name(lib.moe_expert_gateup_w8(ctypes.byref(s), P16, P16, P16, P16, P16, P16,
                                                P16, P16, None))
    D = lambda s: name(lib.moe_expert_down_w8(ctypes.byref(s), P16, P16, P16, P16, P16, P16,
                                              None))
    assert G(shape(T=40)) == "MOE_ERR_UNSUPPORTED" and D(shape(T=40)) == "MOE_ERR_UNSUPPORTED"
    assert G(shape(T=8)) == "MOE_ERR_ALIAS" and D(shape(T=8)) == "MOE_ERR_ALIAS"


def test_decode_workspace_holds_the_down_slices():
    # T <= 32: o holds two K-slice partial sums of kT x d fp32
    lib = moe.load_library()
    s = shape(T=32, d=4096, f=14336, k=2)
    assert lib.moe_workspace_bytes(ctypes.byref(s)) >= 2 * 64 * 4096 * 4 + 64 * 14336 * 2


def test_backward_checks():
    lib = moe.load_library()
    name = lambda st: moe.STATUS_NAMES[st]
    s = shape(T=64)
    need = lib.moe_backward_workspace_bytes(ctypes.byref(s))
    assert need > lib.moe_workspace_bytes(ctypes.byref(s))
    assert lib.moe_backward_workspace_bytes(ctypes.byref(shape(E=65))) == 0
    # x, w_gate, w1, w3, w2, dy, dx, dwg, dw1, dw3, dw2 at distinct fake addresses
    base = [ctypes.c_void_p(0x100000000 * (i + 1)) for i in range(11)]
    ws = ctypes.c_void_p(0x2000000000)
    B = lambda args, ws=ws, n=need: name(lib.moe_backward(ctypes.byref(s), *args, ws, n, None))
    args = list(base)
    bad = list(args); bad[6] = None
    assert B(bad) == "MOE_ERR_NULL"
    bad = list(args); bad[8] = P17
    assert B(bad) == "MOE_ERR_ALIGN"
    assert B(args, n=need - 1) == "MOE_ERR_WORKSPACE"
    bad = list(args); bad[6] = base[5]            # dx over dy
    assert B(bad) == "MOE_ERR_ALIAS"
    bad = list(args); bad[9] = base[8]            # dw3 over dw1
    assert B(bad) == "MOE_ERR_ALIAS"
    assert B(args, ws=base[10]) == "MOE_ERR_ALIAS"   # workspace over dw2
    assert name(lib.moe_backward(ctypes.byref(shape(k=5)), *args, ws, need, None)) == \
        "MOE_ERR_UNSUPPORTED"


# Every entry point's buffers by role: "i" input, "o" output, "w" workspace
# (with ws_bytes after it), "f" a float argument.  Outputs may not overlap
# inputs, other outputs or the workspace, and the workspace may not overlap
# inputs; moe_block_forward alone takes out == h or out == residual.
ALIAS_CASES = [
    ("moe_route", "iioo", {}),
    ("moe_route_probs", "iiooo", {}),
    ("moe_dispatch", "iioooo", {}),
    ("moe_expert_gateup", "iiiiio", {}),
    ("moe_expert_down", "iiiio", {}),
    ("moe_experts", "iiiiiiow", {}),
    ("moe_combine", "iiio", {}),
    ("moe_forward", "iiiiiooow", {}),
    ("moe_forward_noalloc", "iiiiiooo", {}),
    ("moe_rmsnorm_route", "iifiooo", {}),
    ("moe_block_forward", "iifiiiiiooow", {"allowed": {(8, 0), (8, 3)}}),
    ("moe_expert_gateup_w8", "iiiiiiio", {"T": 16}),
    ("moe_expert_down_w8", "iiiiio", {"T": 16}),
    ("moe_forward_w8", "iiiiiiiiooow", {"T": 16}),
    ("moe_backward", "iiiiiiooooow", {}),
]


@pytest.mark.parametrize("fn,roles,opt", ALIAS_CASES, ids=[c[0] for c in ALIAS_CASES])
def test_every_overlap_is_refused(fn, roles, opt):
    lib = moe.load_library()
    s = shape(T=opt.get("T", 64))
    call = getattr(lib, fn)
    spaced = [ctypes.c_void_p(0x100000000 * (i + 1)) for i in range(len(roles))]

    def run(ptrs):
        args = [ctypes.byref(s)]
        for r, p in zip(roles, ptrs):
            if r == "f":
                args.append(1e-5)
            elif r == "w":
                args += [p, 1 << 40]
            else:
                args.append(p)
        args.append(None)                      # stream
        return moe.STATUS_NAMES[call(*args)]

    idx = {r: [i for i, x in enumerate(roles) if x == r] for r in "iow"}
    pairs = [(o, j) for o in idx["o"] for j in idx["i"] + idx["w"]]
    pairs += [(o, j) for o in idx["o"] for j in idx["o"] if j > o]
    pairs += [(w, j) for w in idx["w"] for j in idx["i"]]
    assert pairs
    for a, b in pairs:
        if (a, b) in opt.get("allowed", ()):
            continue
        ptrs = list(spaced)
        ptrs[a] = spaced[b]
        assert run(ptrs) == "MOE_ERR_ALIAS", (fn, a, b)
        # a buffer that starts just inside another one overlaps it too
        ptrs[a] = ctypes.c_void_p(spaced[b].value + 16)
        assert run(ptrs) == "MOE_ERR_ALIAS", (fn, a, b, "+16")


def test_noalloc_checks():
    """moe_forward_noalloc: moe_forward's checks, and MOE_ERR_SCRATCH for a
    shape whose workspace exceeds the library's fixed array (returned before
    the array is looked up, so no GPU is needed to see it)."""
    lib = moe.load_library()
    name = lambda st: moe.STATUS_NAMES[st]
    call = lambda s, x=P16, y=P16B: lib.moe_forward_noalloc(
        ctypes.byref(s) if s is not None else None, x, P16, P16, P16, P16, y, None, None, None)
    assert name(call(None)) == "MOE_ERR_NULL"
    assert name(call(shape(), x=None)) == "MOE_ERR_NULL"
    assert name(call(shape(), x=P17)) == "MOE_ERR_ALIGN"
    assert name(call(shape(), y=P16)) == "MOE_ERR_ALIAS"
    assert name(call(shape(k=5))) == "MOE_ERR_UNSUPPORTED"
    assert call(shape(T=0)) == moe.MOE_OK
    big = shape(T=4096, d=4096, f=14336)
    assert lib.moe_workspace_bytes(ctypes.byref(big)) > moe.SCRATCH_BYTES
    assert name(call(big)) == "MOE_ERR_SCRATCH"
    # the decode steps of the 8x7B and larger expert shapes fit
    for d, f in ((4096, 14336), (6144, 16384)):
        s = shape(T=32, d=d, f=f)
        assert 0 < lib.moe_workspace_bytes(ctypes.byref(s)) <= moe.SCRATCH_BYTES
