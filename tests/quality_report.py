"""Index-quality report on the synthetic workloads (needs a GPU:
``python tests/quality_report.py [workload ...]``).

For each workload: the layer's estimated index is built on the GPU, the
sparse and dense kernels give each row's log-sum-exp, and ms_attention_recall
gives every head's attention-mass recall (the share of the full causal
attention mass the index keeps).  On sampled heads and query blocks the
float64 oracle recomputes that recall from scratch and gives the best recall
any index could reach with the same number of keys per row (the row's top
entries of full attention).  Prints one JSON object per workload.
"""
import json
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import dynamic_sparse_attention_est_amd as ms  # noqa: E402
import oracle  # noqa: E402
import workloads as W  # noqa: E402
from gpu_common import ashape_of, f64, kv_of, make, read_index_blocks, run_staged  # noqa: E402

WORKLOADS = {"vs_4k": 0, "bs_32k": 1, "ashape_128k": 2, "mixed_128k": 3, "vs_1m": 4}


def report(name, n_heads=2, n_blocks=2, rows_per_block=16, seed=0):
    w = W.config(WORKLOADS[name])
    st = run_staged(make(w), debug=False)
    lse_d = torch.empty_like(st.lse)
    ms.ms_dense_attn(st.prob, st.q, st.k, st.v, torch.empty_like(st.q),
                     ms.empty_workspace(ms.ms_attn_workspace_bytes(st.prob)), lse_d)
    rec = torch.empty(w.n_q_heads, device="cuda")
    ms.ms_attention_recall(st.prob, st.lse, lse_d, rec)
    torch.cuda.synchronize()
    rec = rec.cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(seed)
    heads = sorted(rng.choice(w.n_q_heads, size=min(n_heads, w.n_q_heads), replace=False).tolist())
    samples = []
    for h in heads:
        p = w.heads[h]
        blocks = sorted({w.nb - 1, *rng.choice(w.nb, size=n_blocks - 1, replace=False).tolist()})
        idx_b = read_index_blocks(st.prob, st.hp, st.index, h, blocks)
        q, k = f64(st.q[h]), f64(st.k[kv_of(w, h)])
        full = [idx_b.get(b, (np.zeros((0, 2), np.int64), np.zeros(0, np.int64))) for b in range(w.nb)]
        mass = oracle.attention_recall(q, k, full, ashape=ashape_of(p), blocks=blocks)
        for b in blocks:
            budget = oracle.block_mask(full[b], b, w.n, ashape_of(p)).sum(axis=1)
            rows = sorted(rng.choice(64, size=rows_per_block, replace=False).tolist())
            best = oracle.topk_mass(q, k, [64 * b + r for r in rows], budget[rows])
            got = mass[64 * b + np.array(rows)]
            gpu = np.exp(st.lse[h, 64 * b:64 * b + 64].cpu().numpy().astype(np.float64)
                         - lse_d[h, 64 * b:64 * b + 64].cpu().numpy().astype(np.float64))[rows]
            samples.append({"head": h, "pattern": int(p.pattern), "block": b,
                            "recall_oracle": float(got.mean()), "recall_gpu_rows": float(gpu.mean()),
                            "best_same_budget": float(best.mean()),
                            "keys_per_row": float(budget[rows].mean())})
    by_pat = {}
    for pat in sorted({int(p.pattern) for p in w.heads}):
        vals = [rec[h] for h, p in enumerate(w.heads) if p.pattern == pat]
        by_pat[pat] = float(np.mean(vals))
    return {"workload": name, "n": w.n, "recall_mean": float(rec.mean()), "recall_min": float(rec.min()),
            "recall_by_pattern": by_pat, "samples": samples}


if __name__ == "__main__":
    names = sys.argv[1:] or ["vs_4k", "bs_32k", "ashape_128k", "mixed_128k", "vs_1m"]
    for nm in names:
        r = report(nm)
        print(json.dumps(r), flush=True)
        torch.cuda.empty_cache()
