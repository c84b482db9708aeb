"""Shared test helpers: seeded inputs with near-tie screening (the screen
uses the oracle's router), error metrics and tolerances."""
import numpy as np
import torch

import oracle
from sparse_mixture_experts_top2_amd import workloads as W

# Output tolerance, row-max-normalised: max_t max_m |y - ref| / max_m |ref|.
# bf16 I/O with fp32 accumulation: 2e-2; fp32 layers: 1e-5.
Y_TOL = {W.F32: 1e-5, W.BF16: 2e-2}
# Routing weight tolerance (absolute).
RW_TOL = {W.F32: 1e-5, W.BF16: 1e-4}


def checked_inputs(wl, seed=None, device="cpu"):
    """Seeded inputs whose routing decisions have a clear margin (for top-k,
    every token's s-th and (s+1)-th largest logits differ by at least 1e-3
    for s = 1 .. k)."""
    def gap(x, w_gate):
        return oracle.near_tie_tokens(x, w_gate, top_k=wl.top_k)
    return W.make_inputs(wl, seed, gap_fn=gap, device=device)


def checked_block_inputs(wl, g, eps, seed=None, device="cpu"):
    """Seeded inputs for the block boundary (the layer runs on RMSNorm(x)):
    the near-tie screen looks at the logits of the normalised rows, which
    is where the routing is decided."""
    def gap(x, w_gate):
        xn, _ = oracle.rmsnorm(x, g, eps)
        return oracle.near_tie_tokens(xn, w_gate, top_k=wl.top_k)
    return W.make_inputs(wl, seed, gap_fn=gap, device=device)


def to_f64(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().float().cpu().numpy().astype(np.float64)
    return np.asarray(t, np.float64)


def row_max_rel_err(y, ref) -> float:
    y = to_f64(y)
    ref = to_f64(ref)
    if y.size == 0:
        return 0.0
    num = np.abs(y - ref).max(axis=1)
    den = np.abs(ref).max(axis=1)
    return float((num / np.maximum(den, 1e-30)).max())


def bf16_bits(t: torch.Tensor) -> torch.Tensor:
    return t.contiguous().view(torch.int16)


def down_split_parts(counts, n_cols, cus, k_stages, max_parts=2):
    """The part count the prefill down kernel picks (its estimate: rounds of
    one workgroup per CU over 8 XCDs, plus a fifth of a round per extra
    part), written out here to choose a test shape."""
    tiles = sum(-(-int(c) // 256) for c in counts) * n_cols
    cpx = cus // 8
    best, best_cost = 1, None
    for parts in range(1, max_parts + 1):
        if parts > k_stages:
            break
        per_xcd = -(-tiles * parts // 8)
        cost = -(-per_xcd // cpx) / parts + 0.2 * (parts - 1)
        if best_cost is None or cost < best_cost:
            best, best_cost = parts, cost
    return best


def tile_sample(idx, n_experts, tile=256, seed=0, extra=()):
    """Tokens to check at full size, chosen from the grouped order of the
    routing `idx` [T, k] (the oracle's stable grouping) so that every row
    tile of every expert is hit: the first and the last grouped row of
    each expert (its last tile is the ragged one), the first row of its
    last tile, and one random row inside each of its tiles.  Tokens 0 and
    T - 1 and `extra` are added.  Returns sorted unique token indices."""
    counts, offsets, _, src = oracle.dispatch(idx, n_experts)
    T, k = np.asarray(idx).shape
    rng = np.random.default_rng(seed)
    rows = []
    for e in range(n_experts):
        c, o = int(counts[e]), int(offsets[e])
        if c == 0:
            continue
        n_tiles = -(-c // tile)
        rows += [o, o + c - 1, o + (n_tiles - 1) * tile]
        for i in range(n_tiles):
            lo = i * tile
            rows.append(o + lo + int(rng.integers(0, min(tile, c - lo))))
    toks = {int(src[r]) // k for r in rows} | {0, T - 1} | {int(t) for t in extra}
    return np.array(sorted(toks), dtype=np.int64)


def tile_columns(n, tile=128, seed=0, per_tile=1):
    """Column indices of an n-column matrix that hit both edges of every
    `tile`-wide column tile, and `per_tile` random columns inside each."""
    rng = np.random.default_rng(seed)
    cols = set()
    for lo in range(0, n, tile):
        hi = min(n, lo + tile)
        cols |= {lo, hi - 1}
        cols |= {int(c) for c in rng.integers(lo, hi, per_tile)}
    return np.array(sorted(cols), dtype=np.int64)
