"""Float64 oracle of the sparse pre-filling path (TEST INFRASTRUCTURE ONLY).

Only tests/, the package smoke check and the benchmark's CPU-baseline leg use
this module.  See the package docstring for the sources [P1], [P1-PIT], [P2]
and the readings R1..R8 taken where the pages are silent.

Notation: n keys/rows, d = 128, BM = 64 query rows per query block,
NB = n / BM, c = 1/sqrt(d).  q_last is the last L rows of one Q head, k and v
are the rows of its KV head.  Index of one head = a list over query blocks of
(ranges, cols): ranges an int64 array [r, 2] of half-open [lo, hi) key spans,
sorted, disjoint and non-touching; cols an ascending int64 array of single
key columns that lie in no range.
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

BM = 64  # query rows per block, and the pooling block of Block-Sparse heads ([P2] "Key points")

# Pattern codes of the per-head parameters (the offline search's output, [P2] "Summary").
A_SHAPE, VERTICAL_SLASH, BLOCK_SPARSE, DENSE, GRID = 0, 1, 2, 3, 4

BlockIndex = Tuple[np.ndarray, np.ndarray]


# --------------------------------------------------------------------------
# Vertical-Slash estimation ([P2] "Key points": the last query vectors are
# scored against all keys).  Readings R2, R3.
# --------------------------------------------------------------------------
def vs_probabilities(q_last: np.ndarray, k: np.ndarray, scale: Optional[float] = None) -> np.ndarray:
    """Causal softmax of the last L rows against all n keys.

    Row r stands for sequence position i = n - L + r; key j is allowed iff
    j <= i.  Returns P with shape [L, n] (zeros where j > i).
    """
    L, d = q_last.shape
    n = k.shape[0]
    c = 1.0 / math.sqrt(d) if scale is None else scale
    z = (q_last @ k.T) * c                       # [L, n] logits
    rows = np.arange(n - L, n)[:, None]
    allowed = np.arange(n)[None, :] <= rows
    z = np.where(allowed, z, -np.inf)
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)                            # exp(-inf) = 0 on masked keys
    return e / e.sum(axis=1, keepdims=True)


def vs_scores(q_last: np.ndarray, k: np.ndarray, scale: Optional[float] = None):
    """Vertical scores v[j] and slash scores s[o], o = i - j (R3).

    v[j] = sum over the L rows of P[i, j];
    s[o] = sum over the L rows with i - o >= 0 of P[i, i - o].
    """
    p = vs_probabilities(q_last, k, scale)
    L, n = p.shape
    v = p.sum(axis=0)
    s = np.zeros(n)
    for r in range(L):
        i = n - L + r
        # p[r, i::-1] lists P[i, i], P[i, i-1], ..., P[i, 0], i.e. offsets o = 0..i
        s[: i + 1] += p[r, i::-1]
    return v, s


# --------------------------------------------------------------------------
# Top-k (R4, R5): the k largest, equal values resolved toward the lower index,
# all candidates when k exceeds their number, returned ascending.
# --------------------------------------------------------------------------
def topk(scores: np.ndarray, k: int) -> np.ndarray:
    scores = np.asarray(scores, dtype=np.float64)
    idx = np.arange(scores.shape[0])
    order = np.lexsort((idx, -scores))           # by score descending, then index ascending
    return np.sort(order[: min(k, scores.shape[0])]).astype(np.int64)


# --------------------------------------------------------------------------
# Block-Sparse estimation ([P2] "Key points": queries and keys mean-pooled in
# 64-token blocks).  Reading R6: rank the raw dot products of the means.
# --------------------------------------------------------------------------
def bs_pool(x: np.ndarray) -> np.ndarray:
    n, d = x.shape
    return x.reshape(n // BM, BM, d).mean(axis=1)


def bs_scores(q: np.ndarray, k: np.ndarray, q_block0: int = 0) -> np.ndarray:
    """S[b, c] = mean(q over block b) . mean(k over block c) for c <= b; -inf above.

    q holds the query rows from block q_block0 on (chunked prefill, reading
    R15); row r of the result is query block q_block0 + r."""
    qh, kh = bs_pool(q), bs_pool(k)
    s = qh @ kh.T
    b = q_block0 + np.arange(s.shape[0])[:, None]
    c = np.arange(s.shape[1])[None, :]
    return np.where(c <= b, s, -np.inf)


def bs_select(scores: np.ndarray, top_k: int, q_block0: int = 0) -> List[np.ndarray]:
    """B_b = top-min(k, b+1) of S[b, 0..b], ascending (R5); row r is block q_block0 + r."""
    return [topk(scores[r, : q_block0 + r + 1], top_k) for r in range(scores.shape[0])]


# --------------------------------------------------------------------------
# Index conversion (R7): per query block, merged key ranges plus columns.
# --------------------------------------------------------------------------
def _merge(lo: np.ndarray, hi: np.ndarray) -> np.ndarray:
    """Merge half-open spans that overlap or touch; returns sorted [r, 2]."""
    if lo.size == 0:
        return np.zeros((0, 2), dtype=np.int64)
    order = np.argsort(lo, kind="stable")
    lo, hi = lo[order], hi[order]
    out = [[int(lo[0]), int(hi[0])]]
    for a, b in zip(lo[1:].tolist(), hi[1:].tolist()):
        if a <= out[-1][1]:
            out[-1][1] = max(out[-1][1], b)
        else:
            out.append([a, b])
    return np.asarray(out, dtype=np.int64)


def vs_block_index(vert: np.ndarray, slash: np.ndarray, b: int, bm: int = BM) -> BlockIndex:
    """Ranges and columns of query block b (rows [b*bm, b*bm + bm)).

    bm is the query-block height: 64 (reading R7) or 32 (reading R17, the
    finer granularity: each slash keeps a 32-key span per 32-row block)."""
    row0, last = b * bm, b * bm + bm - 1
    o = np.asarray(slash, dtype=np.int64)
    o = o[o <= last]                              # diagonals that reach some row of the block
    ranges = _merge(np.maximum(0, row0 - o), row0 + bm - o)
    j = np.asarray(vert, dtype=np.int64)
    j = j[j <= last]
    if ranges.shape[0]:
        pos = np.searchsorted(ranges[:, 0], j, side="right") - 1
        covered = (pos >= 0) & (j < ranges[np.maximum(pos, 0), 1])
        j = j[~covered]
    return ranges, np.sort(j)


def vs_index(vert: np.ndarray, slash: np.ndarray, n: int, bm: int = BM) -> List[BlockIndex]:
    return [vs_block_index(vert, slash, b, bm) for b in range(n // bm)]


def bs_block_index(blocks: np.ndarray) -> BlockIndex:
    c = np.asarray([x for x in blocks if x >= 0], dtype=np.int64)
    return _merge(c * BM, c * BM + BM), np.zeros(0, dtype=np.int64)


def bs_index(selected: Sequence[np.ndarray]) -> List[BlockIndex]:
    return [bs_block_index(s) for s in selected]


def ashape_block_index(sink: int, window: int, b: int) -> BlockIndex:
    """Union over the block's rows of {j < sink} and {i - window < j <= i} (R1)."""
    row0, end = b * BM, b * BM + BM
    lo = [max(0, row0 - window + 1)]
    hi = [end]
    if sink > 0:
        lo.append(0)
        hi.append(min(sink, end))
    return _merge(np.asarray(lo, dtype=np.int64), np.asarray(hi, dtype=np.int64)), np.zeros(0, dtype=np.int64)


def ashape_index(sink: int, window: int, n: int) -> List[BlockIndex]:
    return [ashape_block_index(sink, window, b) for b in range(n // BM)]


# --------------------------------------------------------------------------
# Grid pattern (the MMInference abstract: video tokens attend along a grid,
# from the temporal and spatial locality of frames).  Reading R16: with P
# tokens per frame, a query keeps the keys of its own spatial neighbourhood
# (half-width w) in each of the T previous frames, offsets o = i - j in
# tP - w .. tP + w, plus the local offsets 0 .. window - 1; the index of a
# 64-row query block is the Vertical-Slash conversion (R7) of that fixed
# slash set with no verticals.
# --------------------------------------------------------------------------
def grid_offsets(stride: int, frames: int, width: int, window: int, n: int) -> np.ndarray:
    """The kept offsets, ascending and distinct, within [0, n)."""
    o = set(range(min(window, n)))
    for t in range(1, frames + 1):
        for delta in range(-width, width + 1):
            x = t * stride + delta
            if 0 <= x < n:
                o.add(x)
    return np.asarray(sorted(o), dtype=np.int64)


def grid_block_index(stride: int, frames: int, width: int, window: int, b: int, n: int) -> BlockIndex:
    return vs_block_index(np.zeros(0, dtype=np.int64), grid_offsets(stride, frames, width, window, n), b)


def dense_block_index(b: int) -> BlockIndex:
    return np.asarray([[0, b * BM + BM]], dtype=np.int64), np.zeros(0, dtype=np.int64)


def dense_index(n: int) -> List[BlockIndex]:
    return [dense_block_index(b) for b in range(n // BM)]


def index_to_csr(index: Sequence[BlockIndex]):
    """(rng_ptr[NB+1], rng[R, 2], col_ptr[NB+1], col[C]) as int32 arrays."""
    nr = [r.shape[0] for r, _ in index]
    nc = [c.shape[0] for _, c in index]
    rng_ptr = np.concatenate([[0], np.cumsum(nr)]).astype(np.int32)
    col_ptr = np.concatenate([[0], np.cumsum(nc)]).astype(np.int32)
    rng = (np.concatenate([r for r, _ in index]) if sum(nr) else np.zeros((0, 2))).astype(np.int32).reshape(-1, 2)
    col = (np.concatenate([c for _, c in index]) if sum(nc) else np.zeros(0)).astype(np.int32)
    return rng_ptr, rng, col_ptr, col


def csr_to_index(rng_ptr, rng, col_ptr, col) -> List[BlockIndex]:
    nb = len(rng_ptr) - 1
    return [(np.asarray(rng[rng_ptr[b]:rng_ptr[b + 1]], dtype=np.int64).reshape(-1, 2),
             np.asarray(col[col_ptr[b]:col_ptr[b + 1]], dtype=np.int64)) for b in range(nb)]


# --------------------------------------------------------------------------
# Mask and attention ([P1]: attention only over the estimated indices; [P2]
# "Summary", third stage).  Readings R1 (A-shape window), R7, R8.
# --------------------------------------------------------------------------
def block_mask(bidx: BlockIndex, b: int, n: int, ashape: Optional[Tuple[int, int]] = None,
               bm: int = BM) -> np.ndarray:
    """Boolean [bm, n]: row i = b*bm + r may attend key j."""
    ranges, cols = bidx
    keep = np.zeros(n, dtype=bool)
    for lo, hi in ranges.tolist():
        keep[lo:hi] = True
    keep[np.asarray(cols, dtype=np.int64)] = True
    i = np.arange(b * bm, b * bm + bm)[:, None]
    j = np.arange(n)[None, :]
    m = keep[None, :] & (j <= i)
    if ashape is not None:
        sink, window = ashape
        m &= (j < sink) | (i - j < window)
    return m


def attention_block(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray, bidx: BlockIndex, b: int,
                    scale: Optional[float] = None, ashape: Optional[Tuple[int, int]] = None, bm: int = BM):
    """Masked softmax attention for the bm rows of block b; returns (out [bm, d], lse [bm])."""
    n, d = k.shape
    c = 1.0 / math.sqrt(d) if scale is None else scale
    ranges, cols = bidx
    keys = np.unique(np.concatenate([np.concatenate([np.arange(lo, hi) for lo, hi in ranges.tolist()])
                                     if ranges.shape[0] else np.zeros(0, dtype=np.int64),
                                     np.asarray(cols, dtype=np.int64)]).astype(np.int64))
    out = np.zeros((bm, d))
    lse = np.full(bm, -np.inf)
    if keys.size == 0:
        return out, lse
    z = (q_rows @ k[keys].T) * c                  # [bm, |keys|]
    i = np.arange(b * bm, b * bm + bm)[:, None]
    j = keys[None, :]
    allowed = j <= i
    if ashape is not None:
        sink, window = ashape
        allowed &= (j < sink) | (i - j < window)
    z = np.where(allowed, z, -np.inf)
    has = allowed.any(axis=1)
    m = np.where(has, z.max(axis=1), 0.0)
    e = np.exp(z - m[:, None])
    l = e.sum(axis=1)
    out[has] = (e[has] @ v[keys]) / l[has, None]
    lse[has] = m[has] + np.log(l[has])
    return out, lse


def attention_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, index: Sequence[BlockIndex],
                   scale: Optional[float] = None, ashape: Optional[Tuple[int, int]] = None,
                   blocks: Optional[Sequence[int]] = None, bm: int = BM):
    """Attention of one Q head over its index of bm-row query blocks;
    ``blocks`` restricts to some query blocks.

    Returns (out [n, d], lse [n]); rows of skipped blocks stay NaN.
    """
    n, d = q.shape
    out = np.full((n, d), np.nan)
    lse = np.full(n, np.nan)
    for b in (range(n // bm) if blocks is None else blocks):
        o, l = attention_block(q[b * bm:(b + 1) * bm], k, v, index[b], b, scale, ashape, bm)
        out[b * bm:(b + 1) * bm] = o
        lse[b * bm:(b + 1) * bm] = l
    return out, lse


# --------------------------------------------------------------------------
# One head, end to end: estimation then index ([P1]: pattern fixed offline,
# indices built per prompt).
# --------------------------------------------------------------------------
def attention_recall(q: np.ndarray, k: np.ndarray, index: Sequence[BlockIndex], scale: Optional[float] = None,
                     ashape: Optional[Tuple[int, int]] = None,
                     blocks: Optional[Sequence[int]] = None) -> np.ndarray:
    """Share of each row's full causal attention mass that the index keeps
    ([P2] "Key points": the pages judge the estimated indices by the attention
    mass they capture).  Row i: softmax over all keys j <= i, summed over the
    keys the index (and, for A-shape heads, the row's window) allows.
    Returns [n]; rows of skipped blocks stay NaN."""
    n, d = q.shape
    c = 1.0 / math.sqrt(d) if scale is None else scale
    mass = np.full(n, np.nan)
    for b in (range(n // BM) if blocks is None else blocks):
        rows = slice(b * BM, b * BM + BM)
        z = (q[rows] @ k.T) * c                       # [BM, n]
        i = np.arange(b * BM, b * BM + BM)[:, None]
        j = np.arange(n)[None, :]
        z = np.where(j <= i, z, -np.inf)
        p = np.exp(z - z.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        mass[rows] = np.where(block_mask(index[b], b, n, ashape), p, 0.0).sum(axis=1)
    return mass


def topk_mass(q: np.ndarray, k: np.ndarray, rows: Sequence[int], budget: Sequence[int],
              scale: Optional[float] = None) -> np.ndarray:
    """The most attention mass any index could keep with the same number of
    keys: for row i, the sum of its budget[i] largest causal softmax
    probabilities (the exact top entries of full attention)."""
    n, d = k.shape
    c = 1.0 / math.sqrt(d) if scale is None else scale
    out = np.empty(len(rows))
    for t, (i, kk) in enumerate(zip(rows, budget)):
        z = (k[:i + 1] @ q[i]) * c
        p = np.exp(z - z.max())
        p /= p.sum()
        out[t] = np.sort(p)[::-1][:int(kk)].sum() if kk > 0 else 0.0
    return out


def estimate_head(params, q: np.ndarray, k: np.ndarray, scale: Optional[float] = None, q_block0: int = 0):
    """Selections of one Q head: ('vs', vert, slash), ('bs', list of B_b) or (pattern,).

    q holds the query rows from block q_block0 on, the last of them the last
    row of the sequence (chunked prefill, reading R15): Vertical-Slash scores
    its last L rows against every key, Block-Sparse selects for its blocks."""
    m = q.shape[0]
    if params.pattern == VERTICAL_SLASH:
        L = min(params.last_q, m)
        v_sc, s_sc = vs_scores(q[m - L:], k, scale)
        return "vs", topk(v_sc, params.n_vertical), topk(s_sc, params.n_slash)
    if params.pattern == BLOCK_SPARSE:
        return "bs", bs_select(bs_scores(q, k, q_block0), params.top_k_blocks, q_block0)
    return ("static",)


def query_block_rows(params) -> int:
    """Rows per query block of a head's index: 32 for a Vertical-Slash head
    that asks for the finer granularity (reading R17), 64 otherwise."""
    return 32 if params.pattern == VERTICAL_SLASH and getattr(params, "block", BM) == 32 else BM


def head_index(params, sel, n: int, q_block0: int = 0) -> List[BlockIndex]:
    """Index of query blocks q_block0 .. n/64 - 1 (entry r is block q_block0 + r);
    a head with 32-row blocks (reading R17) lists blocks 2 q_block0 .. n/32 - 1."""
    blocks = range(q_block0, n // BM)
    if params.pattern == VERTICAL_SLASH:
        bm = query_block_rows(params)
        return [vs_block_index(sel[1], sel[2], b, bm) for b in range(q_block0 * BM // bm, n // bm)]
    if params.pattern == BLOCK_SPARSE:
        return bs_index(sel[1])
    if params.pattern == A_SHAPE:
        return [ashape_block_index(params.sink, params.window, b) for b in blocks]
    if params.pattern == GRID:
        offs = grid_offsets(params.grid_stride, params.grid_frames, params.grid_width, params.window, n)
        return [vs_block_index(np.zeros(0, dtype=np.int64), offs, b) for b in blocks]
    return [dense_block_index(b) for b in blocks]
