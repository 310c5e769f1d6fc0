"""Offline, kernel-aware pattern and budget search per head.

The MInference 1.0 pages describe three stages (summary page, section
"Summary"): an offline search that fixes each attention head's sparse pattern
and budget, the online index estimation, and the sparse kernels; the abstract
adds that the search is kernel-aware (the cost that matters is the kernel's).
This module is that first stage, on whatever Q, K, V it is given (here:
synthetic layers; a real model's calibration activations are out of scope).

For every candidate (pattern + budget) it runs the whole sparse path of the
library on the layer, with every head set to the candidate, and records

  * the measured cost: milliseconds of the layer (estimation + index +
    attention, HIP events) divided by the number of heads; and
  * each head's attention-mass recall: the share of that head's full causal
    attention mass the candidate's index keeps (ms_attention_recall on the
    sparse and dense log-sum-exps).

Each head then takes the cheapest candidate whose recall reaches the target,
unless dense attention (recall 1, its own measured cost per head) is cheaper
or no candidate reaches the target.  Everything runs through the C ABI;
nothing here computes attention itself.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import torch

from . import (A_SHAPE, BLOCK_SPARSE, DENSE, VERTICAL_SLASH, empty_workspace, head_params, ms_attention_recall,
               ms_attn_workspace_bytes, ms_dense_attn, ms_sparse_attn, ms_workspace_bytes, problem)


@dataclasses.dataclass(frozen=True)
class Candidate:
    """A pattern and its budget (the fields of ms_head_params)."""
    pattern: int
    n_vertical: int = 0
    n_slash: int = 0
    top_k_blocks: int = 0
    sink: int = 0
    window: int = 0
    last_q: int = 64
    block: int = 64

    @property
    def name(self) -> str:
        if self.pattern == VERTICAL_SLASH:
            return f"vs({self.n_vertical},{self.n_slash})"
        if self.pattern == BLOCK_SPARSE:
            return f"bs({self.top_k_blocks})"
        if self.pattern == A_SHAPE:
            return f"a({self.sink},{self.window})"
        return "dense"


@dataclasses.dataclass
class Trial:
    candidate: Candidate
    ms_per_head: float       # measured layer time / heads
    recall: List[float]      # per head


def default_candidates(n: int) -> List[Candidate]:
    """A small grid over the three patterns' budgets that fit a sequence of n."""
    nb = n // 64
    out: List[Candidate] = []
    for w in (1024, 2048, 4096, 8192, 16384):
        if 128 + w <= n:
            out.append(Candidate(A_SHAPE, sink=128, window=w))
    for s in (512, 1024, 2048, 4096, 6096):
        if s <= n:
            out.append(Candidate(VERTICAL_SLASH, n_vertical=min(1000, n), n_slash=s))
    for k in (25, 50, 100, 200):
        if k <= nb:
            out.append(Candidate(BLOCK_SPARSE, top_k_blocks=k))
    return out


def measure(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, candidates: Sequence[Candidate],
            repeats: int = 2, scale: float = 0.0) -> tuple:
    """Run every candidate on the layer; returns (trials, dense ms per head).

    q: [H_q, n, 128], k, v: [H_kv, n, 128] bfloat16 device tensors."""
    hq, n, _ = q.shape
    hkv = k.shape[0]
    prob = problem(n, hq, hkv, scale=scale)
    out = torch.empty_like(q)
    lse_d = torch.empty((hq, n), dtype=torch.float32, device=q.device)
    aws = empty_workspace(ms_attn_workspace_bytes(prob))
    ms_dense_attn(prob, q, k, v, out, aws, lse_d)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(repeats):
        ms_dense_attn(prob, q, k, v, out, aws)
    e1.record()
    torch.cuda.synchronize()
    dense_ms = e0.elapsed_time(e1) / repeats / hq
    del aws
    lse_s = torch.empty_like(lse_d)
    rec = torch.empty(hq, dtype=torch.float32, device=q.device)
    trials = []
    for c in candidates:
        hp = head_params([c] * hq)
        ws = empty_workspace(ms_workspace_bytes(prob, hp))
        ms_sparse_attn(prob, hp, q, k, v, out, ws, lse_s)       # warm, and the recall
        ms_attention_recall(prob, lse_s, lse_d, rec)
        e0.record()
        for _ in range(repeats):
            ms_sparse_attn(prob, hp, q, k, v, out, ws)
        e1.record()
        torch.cuda.synchronize()
        trials.append(Trial(c, e0.elapsed_time(e1) / repeats / hq, rec.cpu().tolist()))
        del ws
    return trials, dense_ms


def choose(trials: Sequence[Trial], n_heads: int, target: float,
           dense_ms: Optional[float] = None) -> List[Optional[Candidate]]:
    """Per head, the cheapest candidate whose recall reaches `target` (ties:
    the earlier candidate); None (dense attention) when none does, or when
    dense_ms, the dense cost per head, is lower than that candidate's."""
    picks: List[Optional[Candidate]] = []
    for h in range(n_heads):
        best = None
        for t in trials:
            if t.recall[h] >= target and (best is None or t.ms_per_head < best.ms_per_head):
                best = t
        if best is not None and dense_ms is not None and dense_ms < best.ms_per_head:
            best = None
        picks.append(best.candidate if best is not None else None)
    return picks


def search_layer(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, target: float = 0.95,
                 candidates: Optional[Sequence[Candidate]] = None, repeats: int = 2):
    """Pattern per head for a layer: (choices as Candidate with DENSE for the
    heads no candidate satisfies, trials, dense ms per head)."""
    cands = list(candidates) if candidates is not None else default_candidates(q.shape[1])
    trials, dense_ms = measure(q, k, v, cands, repeats)
    picks = choose(trials, q.shape[0], target, dense_ms)
    return [p if p is not None else Candidate(DENSE) for p in picks], trials, dense_ms


if __name__ == "__main__":
    import argparse
    import json
    import os
    import sys

    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import workloads as W

    ap = argparse.ArgumentParser(description="kernel-aware pattern search on a synthetic layer")
    ap.add_argument("--workload", type=int, default=3, help="workload id 0..4")
    ap.add_argument("--n", type=int, default=None, help="shorter sequence")
    ap.add_argument("--target", type=float, default=0.95)
    a = ap.parse_args()
    w = W.config(a.workload, n=a.n)
    q, k, v = W.generate(w, device="cuda")
    picks, trials, dense_ms = search_layer(q, k, v, a.target)
    print(json.dumps({
        "workload": w.name, "n": w.n, "target": a.target, "dense_ms_per_head": round(dense_ms, 4),
        "trials": [{"candidate": t.candidate.name, "ms_per_head": round(t.ms_per_head, 4),
                    "recall_min": round(min(t.recall), 4), "recall_mean": round(sum(t.recall) / len(t.recall), 4)}
                   for t in trials],
        "choices": [p.name for p in picks],
    }))
