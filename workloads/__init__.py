"""Seeded synthetic inputs for MInference-style sparse pre-filling attention.

This module is shared by the CPU oracle, the GPU tests and the benchmark.  It
holds the five workload descriptions and the seeded generators of Q, K, V and
of the per-head pattern assignment.  It contains none of the method's
arithmetic (no scoring, selection, index building or attention): only random
draws and the planted structure that makes the synthetic inputs look like the
long-context attention described on the MInference 1.0 pages (abstract: the
A-shape, Vertical-Slash and Block-Sparse patterns; "Key points": the last
queries scored against all keys, and 64-token blocks).

Streams.  Every tensor is drawn from its own ``torch.Generator`` seeded from
(config id, seed, tensor id, head).  Values are built in float32 and rounded to
bfloat16 once, at the end (round-to-nearest-even).  The stream depends on the
device kind: a generator on the CPU and one on the GPU give different numbers,
so a workload is named by (config, seed, device kind).  Parity tests always
feed the oracle and the GPU path the very same bytes.

Layouts.  Q is [H_q, n, 128], K and V are [H_kv, n, 128], bfloat16, row-major.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import List, Optional, Sequence

import torch

HEAD_DIM = 128
BLOCK = 64

# Pattern codes; the same numbers are used by the C ABI (ms_pattern).
A_SHAPE = 0
VERTICAL_SLASH = 1
BLOCK_SPARSE = 2
DENSE = 3
GRID = 4

PATTERN_NAMES = {A_SHAPE: "a_shape", VERTICAL_SLASH: "vertical_slash",
                 BLOCK_SPARSE: "block_sparse", DENSE: "dense", GRID: "grid"}


@dataclasses.dataclass(frozen=True)
class HeadParams:
    """Per-Q-head pattern and budgets (the output of the offline search)."""
    pattern: int
    last_q: int = 64
    n_vertical: int = 0
    n_slash: int = 0
    block: int = 64
    top_k_blocks: int = 0
    sink: int = 0
    window: int = 0
    grid_stride: int = 0
    grid_frames: int = 0
    grid_width: int = 0


def vs(n_vertical: int, n_slash: int, last_q: int = 64, block: int = 64) -> HeadParams:
    """A Vertical-Slash head; block = 32 indexes it by 32-row query blocks."""
    return HeadParams(VERTICAL_SLASH, last_q=last_q, n_vertical=n_vertical, n_slash=n_slash, block=block)


def bs(top_k: int) -> HeadParams:
    return HeadParams(BLOCK_SPARSE, top_k_blocks=top_k)


def ashape(sink: int, window: int) -> HeadParams:
    return HeadParams(A_SHAPE, sink=sink, window=window)


def dense() -> HeadParams:
    return HeadParams(DENSE)


def grid(stride: int, frames: int, width: int, window: int) -> HeadParams:
    return HeadParams(GRID, window=window, grid_stride=stride, grid_frames=frames, grid_width=width)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention layer: shapes, per-head parameters and the input recipe."""
    name: str
    config_id: int
    n: int
    n_q_heads: int
    n_kv_heads: int
    heads: tuple            # HeadParams per Q head
    recipe: str             # "vs_planted", "bs_lowrank", "ashape_sink"
    scale_qkv: float = 1.0  # std of the base Gaussian draw
    n_planted: int = 0      # planted key columns per KV head
    lowrank_frac: float = 0.0
    seed: int = 0
    query_mean: float = 0.0  # vs_planted: std of a shared mean added to the group's queries

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def nb(self) -> int:
        return self.n // BLOCK


def _mixed_heads(seed: int, n_q: int, n_vs: int, n_bs: int, n_a: int) -> tuple:
    g = torch.Generator(device="cpu")
    g.manual_seed(_seed_of(3, seed, 99, 0))
    perm = torch.randperm(n_q, generator=g).tolist()
    heads: List[Optional[HeadParams]] = [None] * n_q
    for r, h in enumerate(perm):
        if r < n_vs:
            heads[h] = vs(1000, 6096)
        elif r < n_vs + n_bs:
            heads[h] = bs(100)
        else:
            heads[h] = ashape(128, 4096)
    assert n_vs + n_bs + n_a == n_q
    return tuple(heads)


def config(config_id: int, seed: int = 0, n: Optional[int] = None) -> Workload:
    """The five workloads; ``n`` shrinks the sequence for small parity cases."""
    if config_id == 0:
        nn = n or 4096
        return Workload("vs_4k", 0, nn, 1, 1, (vs(256, 512),), "vs_planted",
                        scale_qkv=2 ** -0.5, n_planted=8, seed=seed)
    if config_id == 1:
        nn = n or 32768
        return Workload("bs_32k", 1, nn, 32, 32, tuple(bs(100) for _ in range(32)), "bs_lowrank",
                        lowrank_frac=0.05, seed=seed)
    if config_id == 2:
        nn = n or 131072
        return Workload("ashape_128k", 2, nn, 32, 32, tuple(ashape(128, 4096) for _ in range(32)),
                        "ashape_sink", seed=seed)
    if config_id == 3:
        nn = n or 131072
        return Workload("mixed_128k", 3, nn, 32, 8, _mixed_heads(seed, 32, 24, 6, 2), "vs_planted",
                        n_planted=8, seed=seed)
    if config_id == 4:
        nn = n or 1048576
        return Workload("vs_1m", 4, nn, 32, 8, tuple(vs(1000, 6096) for _ in range(32)), "vs_planted",
                        n_planted=64, seed=seed)
    if config_id == 5:
        # Diagnostic beside the five workloads (not one of them): the 1M
        # Vertical-Slash layer with a shared query mean per KV group, so that
        # the planted key columns are real verticals and the slashes through
        # them (64 offsets per column, seen by the last 64 rows) win the slash
        # budget, as structured attention would; the rest of the budget stays
        # scattered.
        nn = n or 1048576
        return Workload("vs_1m_s", 5, nn, 32, 8, tuple(vs(1000, 6096) for _ in range(32)), "vs_planted",
                        n_planted=64, seed=seed, query_mean=0.5)
    if config_id == 6:
        # The 1M layer (same inputs as vs_1m: same config id for the draws)
        # with its Vertical-Slash heads indexed by 32-row query blocks.
        nn = n or 1048576
        return Workload("vs_1m_b32", 4, nn, 32, 8, tuple(vs(1000, 6096, block=32) for _ in range(32)), "vs_planted",
                        n_planted=64, seed=seed)
    raise ValueError(f"unknown config {config_id}")


def custom(name: str, n: int, n_q_heads: int, n_kv_heads: int, heads: Sequence[HeadParams],
           recipe: str = "vs_planted", seed: int = 0, n_planted: int = 4,
           scale_qkv: float = 1.0, lowrank_frac: float = 0.05, config_id: int = 7) -> Workload:
    """A small workload for tests (any shape the library accepts)."""
    return Workload(name, config_id, n, n_q_heads, n_kv_heads, tuple(heads), recipe,
                    scale_qkv=scale_qkv, n_planted=n_planted, lowrank_frac=lowrank_frac, seed=seed)


def _seed_of(*parts: int) -> int:
    h = hashlib.sha256(",".join(str(int(p)) for p in parts).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(w: Workload, tensor_id: int, head: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed_of(w.config_id, w.seed, tensor_id, head, w.n))
    return g


_Q, _K, _V, _PLANT, _LOWRANK_U, _LOWRANK_W, _LOWRANK_BLK, _GRID_U, _QMEAN = range(9)


def _randn(w: Workload, tensor_id: int, head: int, shape, device) -> torch.Tensor:
    g = _gen(w, tensor_id, head, device)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def generate(w: Workload, device="cpu"):
    """Return (q, k, v) as bfloat16 tensors on ``device``.

    Recipes (float32 construction, then one RNE rounding to bfloat16):
      vs_planted  q, k, v ~ N(0, s^2).  Per KV head: n_planted key columns j
                  (drawn without replacement) get k_j += 3 * mean(q), the mean
                  over the group's Q heads and all positions; then every key
                  gets k_j += 0.5 * mean over the group's Q heads of q_j (the
                  local bias toward the main diagonal).  With query_mean = m > 0
                  every query of a KV group first gets += mu, one draw of
                  mu ~ N(0, m^2 I) per group (a shared query direction).
      bs_lowrank  q, k, v ~ N(0, 1).  Per head, round(frac * NB) blocks are
                  chosen; U (128x4) ~ N(0, 1/4); each chosen block draws
                  w ~ N(0, I_4) and all 64 of its tokens, in Q and in K, get
                  += 2 * U w.
      ashape_sink q, k, v ~ N(0, 1).  u = mean(q) / |mean(q)| per head; the
                  first 128 keys get k_j += 2 (k_j . u) u, i.e. x3 along u.
      grid_video  video-like tokens, frames of P = n_planted tokens: q, k, v ~
                  N(0, s^2); per KV head a table U [P, 128] ~ N(0, 1) (one
                  vector per spatial position); the group's queries and the
                  keys at position i get += 0.7 U[i mod P], so a query leans
                  toward the keys at its own spatial position in every frame
                  (about +5.5 on the scaled logit).
    """
    n, d = w.n, HEAD_DIM
    hq, hkv, grp = w.n_q_heads, w.n_kv_heads, w.group
    q = torch.empty((hq, n, d), dtype=torch.bfloat16, device=device)
    k = torch.empty((hkv, n, d), dtype=torch.bfloat16, device=device)
    v = torch.empty((hkv, n, d), dtype=torch.bfloat16, device=device)
    s = w.scale_qkv
    for kv in range(hkv):
        v[kv] = (_randn(w, _V, kv, (n, d), device) * s).to(torch.bfloat16)
    if w.recipe == "vs_planted":
        for kv in range(hkv):
            qf = [(_randn(w, _Q, h, (n, d), device) * s) for h in range(kv * grp, (kv + 1) * grp)]
            if w.query_mean > 0:
                mu = _randn(w, _QMEAN, kv, (d,), device) * w.query_mean
                for x in qf:
                    x += mu
            kf = _randn(w, _K, kv, (n, d), device) * s
            qmean_all = torch.stack([x.mean(dim=0) for x in qf]).mean(dim=0)
            if w.n_planted > 0:
                g = _gen(w, _PLANT, kv, "cpu")
                cols = torch.randperm(n, generator=g)[: w.n_planted].to(device)
                kf[cols] += 3.0 * qmean_all
            qmean_tok = torch.stack(qf).mean(dim=0)
            kf += 0.5 * qmean_tok
            for i, h in enumerate(range(kv * grp, (kv + 1) * grp)):
                q[h] = qf[i].to(torch.bfloat16)
            k[kv] = kf.to(torch.bfloat16)
            del qf, kf, qmean_tok
    elif w.recipe == "bs_lowrank":
        assert hq == hkv, "bs_lowrank is an MHA recipe"
        nb = n // BLOCK
        nsel = int(round(w.lowrank_frac * nb))
        for h in range(hq):
            qf = _randn(w, _Q, h, (n, d), device) * s
            kf = _randn(w, _K, h, (n, d), device) * s
            if nsel > 0:
                g = _gen(w, _LOWRANK_BLK, h, "cpu")
                blocks = torch.randperm(nb, generator=g)[:nsel].tolist()
                u = _randn(w, _LOWRANK_U, h, (d, 4), device) * 0.5
                wv = _randn(w, _LOWRANK_W, h, (nsel, 4), device)
                for i, b in enumerate(blocks):
                    add = 2.0 * (u @ wv[i])
                    qf[b * BLOCK:(b + 1) * BLOCK] += add
                    kf[b * BLOCK:(b + 1) * BLOCK] += add
            q[h] = qf.to(torch.bfloat16)
            k[h] = kf.to(torch.bfloat16)
    elif w.recipe == "ashape_sink":
        assert hq == hkv, "ashape_sink is an MHA recipe"
        for h in range(hq):
            qf = _randn(w, _Q, h, (n, d), device) * s
            kf = _randn(w, _K, h, (n, d), device) * s
            mu = qf.mean(dim=0)
            u = mu / mu.norm()
            ns = min(128, n)
            proj = kf[:ns] @ u
            kf[:ns] += 2.0 * proj[:, None] * u[None, :]
            q[h] = qf.to(torch.bfloat16)
            k[h] = kf.to(torch.bfloat16)
    elif w.recipe == "grid_video":
        P = w.n_planted
        assert P >= 1, "grid_video needs the frame size in n_planted"
        pos = torch.arange(n, device=device) % P
        for kv in range(hkv):
            u = _randn(w, _GRID_U, kv, (P, d), device)[pos] * 0.7
            for h in range(kv * grp, (kv + 1) * grp):
                q[h] = (_randn(w, _Q, h, (n, d), device) * s + u).to(torch.bfloat16)
            k[kv] = (_randn(w, _K, kv, (n, d), device) * s + u).to(torch.bfloat16)
            del u
    else:
        raise ValueError(w.recipe)
    return q, k, v
