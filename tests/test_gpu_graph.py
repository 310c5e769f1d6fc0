"""The one-shot call (estimation, index, attention) enqueues kernels only: no
allocation, no memset, no synchronisation, so a caller can capture it in a
HIP graph.  Every replay, with eager work of the program between replays,
must give the eager call's output and log-sum-exps bit for bit."""
import pytest
import torch

import dynamic_sparse_attention_est_amd as ms
import workloads as W

pytestmark = pytest.mark.gpu


def test_one_shot_call_replays_in_a_graph():
    heads = [W.vs(64, 96), W.bs(4), W.ashape(32, 200), W.vs(100, 40)]
    w = W.custom("graph", 2048, 4, 2, heads, recipe="vs_planted", seed=5)
    q, k, v = W.generate(w, device="cuda")
    prob, hp = ms.problem(w.n, w.n_q_heads, w.n_kv_heads), ms.head_params(w.heads)
    ws = ms.empty_workspace(ms.ms_workspace_bytes(prob, hp))
    ref, ref_lse = torch.empty_like(q), torch.empty((4, w.n), device="cuda")
    ms.ms_sparse_attn(prob, hp, q, k, v, ref, ws, ref_lse)
    torch.cuda.synchronize()
    out, lse = torch.empty_like(q), torch.empty((4, w.n), device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ms.ms_sparse_attn(prob, hp, q, k, v, out, ws, lse)
    for _ in range(3):
        out.zero_()
        lse.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
        assert torch.equal(lse, ref_lse)
        # eager work between replays: the same call on the same workspace
        other = torch.empty_like(q)
        ms.ms_sparse_attn(prob, hp, q, k, v, other, ws)
        torch.cuda.synchronize()
        assert torch.equal(other.view(torch.int16), ref.view(torch.int16))
