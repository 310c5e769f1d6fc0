"""Chunked prefill (ms_problem.q_block0) on the GPU, through the C ABI.

A call with q_block0 = c computes query blocks c .. n/64-1 of a sequence
whose n keys are all present (reading R15 of the design notes: the chunk's
last 64 query rows are the sequence's last rows, Block-Sparse pools the
chunk's own query blocks).  Under that reading every output of the chunk is
the whole-sequence output restricted to the chunk's rows, so the chunk call
must reproduce the tail of the whole call bit for bit (the kernels compute
each (head, query block) the same way whichever blocks share the call); a
second test checks a chunk against the oracle directly.
"""
import numpy as np
import pytest
import torch

import dynamic_sparse_attention_est_amd as ms
import oracle
import workloads as W
from gpu_common import ashape_of, check_attention, f64
from test_gpu_parity import LSE_ATOL

pytestmark = pytest.mark.gpu


def _run(prob, hp, heads, q, k, v, scores=False, dense=False):
    """All stages of one call; returns the host-visible results."""
    dev = "cuda"
    nq, m = q.shape[0], q.shape[1]
    nb = prob.n // 64
    nbq = nb - prob.q_block0
    out = torch.empty((nq, m, 128), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((nq, m), dtype=torch.float32, device=dev)
    res = {"out": out, "lse": lse}
    if dense:
        ws = ms.empty_workspace(ms.ms_attn_workspace_bytes(prob))
        ms.ms_dense_attn(prob, q, k, v, out, ws, lse)
        torch.cuda.synchronize()
        return res
    nv, ns, nbk = ms.ms_selection_sizes(prob, hp)
    vert = torch.full((max(nv, 1),), -7, dtype=torch.int32, device=dev)
    slash = torch.full((max(ns, 1),), -7, dtype=torch.int32, device=dev)
    blocks = torch.full((max(nbk, 1),), -7, dtype=torch.int32, device=dev)
    ews = ms.empty_workspace(ms.ms_estimate_workspace_bytes(prob, hp))
    dbg = torch.full((nq, nbq, nb), float("nan"), device=dev) if scores else None
    ms.ms_estimate_vs(prob, hp, q, k, vert, slash, ews)
    ms.ms_estimate_block(prob, hp, q, k, blocks, ews, dbg)
    index = ms.empty_workspace(ms.ms_index_bytes(prob, hp))
    ms.ms_build_index(prob, hp, vert, slash, blocks, index)
    aws = ms.empty_workspace(ms.ms_attn_workspace_bytes(prob))
    ms.ms_sparse_attn_indexed(prob, hp, q, k, v, index, out, aws, lse)
    torch.cuda.synchronize()
    res.update(vert=vert.cpu().numpy(), slash=slash.cpu().numpy(), blocks=blocks.cpu().numpy(),
               csr=[oracle.csr_to_index(*c) for c in ms.read_index(prob, hp, index)], dbg=dbg)
    # selections per head, as the oracle's index functions take them
    sel, ov, os_, ob = [], 0, 0, 0
    for h in heads:
        if h.pattern == W.VERTICAL_SLASH:
            sel.append(("vs", res["vert"][ov:ov + h.n_vertical].astype(np.int64),
                        res["slash"][os_:os_ + h.n_slash].astype(np.int64)))
            ov += h.n_vertical
            os_ += h.n_slash
        elif h.pattern == W.BLOCK_SPARSE:
            rows = res["blocks"][ob:ob + nbq * h.top_k_blocks].reshape(nbq, h.top_k_blocks)
            sel.append(("bs", [r[r >= 0].astype(np.int64) for r in rows], rows))
            ob += nbq * h.top_k_blocks
        else:
            sel.append(("static",))
    res["sel"] = sel
    return res


def heads_for(nblk):
    """Every pattern, with a Block-Sparse budget above 256 blocks when the
    sequence allows it."""
    return [W.vs(40, 60), W.bs(6), W.ashape(40, 150), W.dense(), W.vs(5, 2), W.ashape(0, 64),
            W.bs(min(300, nblk)), W.vs(300, 500)]


@pytest.mark.parametrize("nblk,q_block0", [(45, 1), (45, 22), (45, 44), (512, 300)])
def test_chunk_reproduces_the_tail_of_the_whole_call(nblk, q_block0):
    n = 64 * nblk
    HEADS = heads_for(nblk)
    w = W.custom("chunk", n, 8, 2, HEADS, recipe="vs_planted", seed=61)
    q, k, v = W.generate(w, device="cuda")
    hp = ms.head_params(HEADS)
    print(f"[chunk] n={n} q_block0={q_block0}", flush=True)
    full = _run(ms.problem(n, 8, 2), hp, HEADS, q, k, v, scores=True)
    qc = q[:, 64 * q_block0:].contiguous()
    part = _run(ms.problem(n, 8, 2, q_block0=q_block0), hp, HEADS, qc, k, v, scores=True)
    for h, p in enumerate(HEADS):
        if p.pattern == W.VERTICAL_SLASH:
            np.testing.assert_array_equal(part["sel"][h][1], full["sel"][h][1])
            np.testing.assert_array_equal(part["sel"][h][2], full["sel"][h][2])
        elif p.pattern == W.BLOCK_SPARSE:
            np.testing.assert_array_equal(part["sel"][h][2], full["sel"][h][2][q_block0:])
            assert torch.equal(part["dbg"][h], full["dbg"][h][q_block0:])
        for r, (cr, fr) in enumerate(zip(part["csr"][h], full["csr"][h][q_block0:])):
            np.testing.assert_array_equal(cr[0], fr[0], err_msg=f"head {h} block {q_block0 + r} ranges")
            np.testing.assert_array_equal(cr[1], fr[1], err_msg=f"head {h} block {q_block0 + r} cols")
    assert torch.equal(part["out"].view(torch.int16), full["out"][:, 64 * q_block0:].view(torch.int16))
    assert torch.equal(part["lse"], full["lse"][:, 64 * q_block0:])
    # dense baseline and the recall instrument over the chunk's rows
    dfull = _run(ms.problem(n, 8, 2), hp, HEADS, q, k, v, dense=True)
    dpart = _run(ms.problem(n, 8, 2, q_block0=q_block0), hp, HEADS, qc, k, v, dense=True)
    assert torch.equal(dpart["out"].view(torch.int16), dfull["out"][:, 64 * q_block0:].view(torch.int16))
    assert torch.equal(dpart["lse"], dfull["lse"][:, 64 * q_block0:])
    rec = torch.empty(8, dtype=torch.float32, device="cuda")
    ms.ms_attention_recall(ms.problem(n, 8, 2, q_block0=q_block0), part["lse"], dpart["lse"], rec)
    ref = np.exp(f64(part["lse"]) - f64(dpart["lse"]))
    ref = np.where(np.isfinite(f64(part["lse"])), ref, 0.0).mean(axis=1)
    np.testing.assert_allclose(rec.cpu().numpy(), ref, rtol=1e-5, atol=1e-6)


def test_chunk_against_the_oracle():
    """Chunk of 15 query blocks of a 40-block sequence: the GPU CSR equals the
    oracle's index of the GPU's selections, Block-Sparse scores match the
    oracle's chunk scores, and attention of every chunk block meets the bar."""
    n, q_block0 = 64 * 40, 25
    HEADS = heads_for(40)
    w = W.custom("chunk_oracle", n, 8, 2, HEADS, recipe="vs_planted", seed=62)
    q, k, v = W.generate(w, device="cuda")
    hp = ms.head_params(HEADS)
    qc = q[:, 64 * q_block0:].contiguous()
    part = _run(ms.problem(n, 8, 2, q_block0=q_block0), hp, HEADS, qc, k, v, scores=True)
    qh, kh, vh = f64(qc), f64(k), f64(v)
    for h, p in enumerate(HEADS):
        kv = h // 4
        ref_idx = oracle.head_index(p, part["sel"][h], n, q_block0=q_block0)
        assert len(ref_idx) == len(part["csr"][h]) == 40 - q_block0
        for r, (g, e) in enumerate(zip(part["csr"][h], ref_idx)):
            np.testing.assert_array_equal(g[0], e[0], err_msg=f"head {h} block {q_block0 + r}")
            np.testing.assert_array_equal(g[1], e[1], err_msg=f"head {h} block {q_block0 + r}")
        if p.pattern == W.BLOCK_SPARSE:
            ref = oracle.bs_scores(qh[h], kh[kv], q_block0=q_block0)
            got = f64(part["dbg"][h])
            fin = np.isfinite(ref)
            assert np.array_equal(np.isfinite(got), fin)
            scale = np.abs(oracle.bs_pool(qh[h])) @ np.abs(oracle.bs_pool(kh[kv])).T
            assert (np.abs(got[fin] - ref[fin]) / (scale[fin] + 1e-30)).max() <= 1e-5
            # the GPU selection is the oracle's top-k of the GPU's own scores
            for r in range(40 - q_block0):
                b = q_block0 + r
                np.testing.assert_array_equal(part["sel"][h][1][r], oracle.topk(got[r, :b + 1], p.top_k_blocks))
        for r in range(40 - q_block0):
            b = q_block0 + r
            ro, rl = oracle.attention_block(qh[h, 64 * r:64 * r + 64], kh[kv], vh[kv], ref_idx[r], b,
                                            ashape=ashape_of(p))
            rows = slice(64 * r, 64 * r + 64)
            check_attention(f64(part["out"][h, rows]), ro, f"head {h} block {b}")
            gl = f64(part["lse"][h, rows])
            fin = np.isfinite(rl)
            assert np.all(np.isneginf(gl[~fin]))
            np.testing.assert_allclose(gl[fin], rl[fin], rtol=0, atol=LSE_ATOL)


def test_chunk_of_a_long_sequence_paced():
    """n = 262144: paced heads (launches of 1024 workgroups from the last
    block down) with a first query block other than 0; the chunk's output
    and lse equal the tail of the whole call."""
    n, q_block0 = 262144, 4096 - 700
    heads = [W.vs(100, 1500), W.bs(500), W.ashape(1024, 40000), W.vs(30, 60)] * 2
    w = W.custom("chunk_seg", n, 8, 2, heads, recipe="vs_planted", seed=63)
    q, k, v = W.generate(w, device="cuda")
    hp = ms.head_params(heads)
    full = _run(ms.problem(n, 8, 2), hp, heads, q, k, v)
    full_out = full["out"][:, 64 * q_block0:].clone()
    full_lse = full["lse"][:, 64 * q_block0:].clone()
    del full
    torch.cuda.empty_cache()
    qc = q[:, 64 * q_block0:].contiguous()
    part = _run(ms.problem(n, 8, 2, q_block0=q_block0), hp, heads, qc, k, v)
    assert torch.equal(part["out"].view(torch.int16), full_out.view(torch.int16))
    assert torch.equal(part["lse"], full_lse)


def test_batch_by_stacking_heads():
    """Two sequences of one length stacked along the head axis (their Q heads,
    then their KV heads) give, head for head, the results of two separate
    calls."""
    n = 64 * 21
    heads = [W.vs(30, 50), W.bs(5), W.ashape(30, 100), W.dense()]
    seqs = [W.generate(W.custom(f"batch{i}", n, 4, 2, heads, recipe="vs_planted", seed=70 + i), device="cuda")
            for i in range(2)]
    sep = [_run(ms.problem(n, 4, 2), ms.head_params(heads), heads, *s) for s in seqs]
    q = torch.cat([s[0] for s in seqs]).contiguous()
    k = torch.cat([s[1] for s in seqs]).contiguous()
    v = torch.cat([s[2] for s in seqs]).contiguous()
    both = _run(ms.problem(n, 8, 4), ms.head_params(heads * 2), heads * 2, q, k, v)
    for i in range(2):
        assert torch.equal(both["out"][4 * i:4 * i + 4].view(torch.int16), sep[i]["out"].view(torch.int16))
        assert torch.equal(both["lse"][4 * i:4 * i + 4], sep[i]["lse"])
