"""Parity on the five workloads at their full sizes, through the C ABI.

Small workload 0 runs end to end in tests/test_gpu_parity.py.  Here the
GPU runs the whole layer at full size; the float64 oracle checks every
head's selection against the GPU's own scores (bit-exact), sampled heads'
scores and oracle selections (near-tie aware), the index of sampled query
blocks (bit-exact), and attention on sampled query blocks (the bar of
tests/test_gpu_parity.py).  The one-shot call must reproduce the staged
output bit for bit.
"""
import numpy as np
import pytest
import torch

import dynamic_sparse_attention_est_amd as ms
import oracle
import workloads as W
from gpu_common import (ashape_of, check_attention, f64, kv_of, make, read_index_blocks, run_staged,
                        sample_blocks, selections)
from test_gpu_parity import LSE_ATOL, _near_tie_ok, _score_check

pytestmark = pytest.mark.gpu


def _check_layer(cid, heads_checked, n_blocks, seed, est_heads=(), edge_blocks=()):
    w = W.config(cid)
    print(f"[config {cid}] {w.name}: n={w.n} heads={w.n_q_heads}/{w.n_kv_heads}", flush=True)
    st = run_staged(make(w), debug=True)
    sel = selections(st)
    # every head: GPU selection == oracle top-k of the GPU's own scores
    dv = st.dbg_v.cpu().numpy() if st.dbg_v is not None else None
    ds = st.dbg_s.cpu().numpy() if st.dbg_s is not None else None
    sc = st.dbg_scores
    for h, p in enumerate(w.heads):
        if p.pattern == W.VERTICAL_SLASH:
            np.testing.assert_array_equal(sel[h][1], oracle.topk(dv[h].astype(np.float64), p.n_vertical))
            np.testing.assert_array_equal(sel[h][2], oracle.topk(ds[h].astype(np.float64), p.n_slash))
        elif p.pattern == W.BLOCK_SPARSE:
            s_h = sc[h].cpu().numpy().astype(np.float64)
            rows = sel[h][2]
            for b in sample_blocks(w.nb, 64, seed + h):
                np.testing.assert_array_equal(rows[b][: min(p.top_k_blocks, b + 1)],
                                              oracle.topk(s_h[b, : b + 1], p.top_k_blocks))
    # sampled heads: scores and end-to-end selections against the oracle
    for h in est_heads:
        p = w.heads[h]
        qh = f64(st.q[h])
        kh = f64(st.k[kv_of(w, h)])
        if p.pattern == W.VERTICAL_SLASH:
            v_ref, s_ref = oracle.vs_scores(qh[w.n - 64:], kh)
            _score_check(dv[h].astype(np.float64), v_ref, f"head {h} vertical")
            _score_check(ds[h].astype(np.float64), s_ref, f"head {h} slash")
            ties = _near_tie_ok(sel[h][1], oracle.topk(v_ref, p.n_vertical), v_ref, dv[h], p.n_vertical)
            ties += _near_tie_ok(sel[h][2], oracle.topk(s_ref, p.n_slash), s_ref, ds[h], p.n_slash)
            print(f"  head {h}: near-tie swaps {ties}", flush=True)
        elif p.pattern == W.BLOCK_SPARSE:
            ref = oracle.bs_scores(qh, kh)
            got = sc[h].cpu().numpy().astype(np.float64)
            low = np.tril(np.ones_like(ref, dtype=bool))
            scale = np.abs(oracle.bs_pool(qh)) @ np.abs(oracle.bs_pool(kh)).T
            assert (np.abs(got[low] - ref[low]) / (scale[low] + 1e-30)).max() <= 1e-5
    del sc
    # sampled heads and blocks: index and attention
    out = st.out
    lse = st.lse
    for h in heads_checked:
        p = w.heads[h]
        blocks = sorted(set(sample_blocks(w.nb, n_blocks, seed + 100 + h)) | set(edge_blocks))
        got_idx = read_index_blocks(st.prob, st.hp, st.index, h, blocks)
        qh = f64(st.q[h])
        kh, vh = f64(st.k[kv_of(w, h)]), f64(st.v[kv_of(w, h)])
        for b in blocks:
            if p.pattern == W.VERTICAL_SLASH:
                ref_b = oracle.vs_block_index(sel[h][1], sel[h][2], b)
            elif p.pattern == W.BLOCK_SPARSE:
                ref_b = oracle.bs_block_index(sel[h][1][b])
            elif p.pattern == W.A_SHAPE:
                ref_b = oracle.ashape_block_index(p.sink, p.window, b)
            else:
                ref_b = oracle.dense_block_index(b)
            np.testing.assert_array_equal(got_idx[b][0], ref_b[0], err_msg=f"head {h} block {b} ranges")
            np.testing.assert_array_equal(got_idx[b][1], ref_b[1], err_msg=f"head {h} block {b} cols")
            ro, rl = oracle.attention_block(qh[64 * b:64 * b + 64], kh, vh, ref_b, b, ashape=ashape_of(p))
            rows = slice(64 * b, 64 * b + 64)
            check_attention(f64(out[h, rows]), ro, f"head {h} block {b}")
            got_l = lse[h, rows].cpu().numpy().astype(np.float64)
            fin = np.isfinite(rl)
            assert np.all(np.isneginf(got_l[~fin]))
            np.testing.assert_allclose(got_l[fin], rl[fin], rtol=0, atol=LSE_ATOL)
        print(f"  head {h} ({p.pattern}): {len(blocks)} blocks ok", flush=True)
    # one-shot call reproduces the staged output bit for bit
    ws = ms.empty_workspace(ms.ms_workspace_bytes(st.prob, st.hp))
    out2 = torch.empty_like(out)
    ms.ms_sparse_attn(st.prob, st.hp, st.q, st.k, st.v, out2, ws)
    torch.cuda.synchronize()
    assert torch.equal(out2.view(torch.int16), out.view(torch.int16))


def test_config1_block_sparse_32k():
    _check_layer(1, heads_checked=[0, 17, 31], n_blocks=8, seed=1, est_heads=[0, 31])


def test_config2_ashape_128k():
    _check_layer(2, heads_checked=[0, 31], n_blocks=6, seed=2)


def test_config3_mixed_128k():
    w = W.config(3)
    pats = [p.pattern for p in w.heads]
    vs_h = [i for i, p in enumerate(pats) if p == W.VERTICAL_SLASH]
    bs_h = [i for i, p in enumerate(pats) if p == W.BLOCK_SPARSE]
    a_h = [i for i, p in enumerate(pats) if p == W.A_SHAPE]
    _check_layer(3, heads_checked=[vs_h[0], vs_h[-1], bs_h[0], a_h[0]], n_blocks=4, seed=3,
                 est_heads=[vs_h[0], bs_h[0]])


def _paced_launch_edges(nblk, heads):
    """Blocks on both sides of the launch boundaries of the paced mode: a
    launch holds 1024 workgroups, 1024 // heads blocks of every paced head,
    taken from the last block down (the lowest launch may be short)."""
    cb = 1024 // heads
    edges = set()
    for top in (nblk - cb, nblk - 64 * cb, nblk - (nblk // cb) * cb):
        edges |= {top - 1, top}
    return sorted(b for b in edges if 0 <= b < nblk)


def test_config4_vertical_slash_1m():
    """Scores and end-to-end selections of one Q head per KV head; index and
    attention of four heads (different KV heads) at the edges of the paced
    launches (32 blocks of all 32 heads each, from the last block down), at
    pacing-segment edges (a block whose rows end an 8192-key segment and the
    next), the first and last blocks, and random ones."""
    w = W.config(4)
    nb = w.nb
    seg_edges = [127, 128, 511, 512, 8191, 8192, nb - 129, nb - 128]
    edges = sorted({0, 1, nb - 2, nb - 1, *_paced_launch_edges(nb, 32), *[b for b in seg_edges if 0 <= b < nb]})
    _check_layer(4, heads_checked=[0, 9, 18, 27], n_blocks=2, seed=4, est_heads=list(range(0, 32, 4)),
                 edge_blocks=edges)


def test_union_of_many_ranges_per_block():
    """Four Vertical-Slash heads of one KV head, dense enough (4096 slashes at
    n = 262144, expected density 0.63) to be served over their union index,
    with scattered slashes: the late query blocks hold more ranges across the
    four heads than the union builder merges in LDS, so it takes the one-thread
    merge there.  Sampled late and early blocks against the oracle."""
    n = 262144
    heads = [W.vs(50, 4096)] * 4
    w = W.custom("union_many", n, 4, 1, heads, recipe="vs_planted", seed=31)
    st = run_staged(make(w), debug=False)
    sel = selections(st)
    nb = n // 64
    blocks = [0, 5, nb // 2, nb - 3, nb - 1]
    per_head = [read_index_blocks(st.prob, st.hp, st.index, h, blocks) for h in range(4)]
    assert sum(len(per_head[h][nb - 1][0]) for h in range(4)) > 4096, "late blocks should exceed the LDS merge"
    q, k, v = f64(st.q), f64(st.k[0]), f64(st.v[0])
    for h in range(4):
        for b in blocks:
            ref_b = oracle.vs_block_index(sel[h][1], sel[h][2], b)
            np.testing.assert_array_equal(per_head[h][b][0], ref_b[0])
            np.testing.assert_array_equal(per_head[h][b][1], ref_b[1])
            ro, rl = oracle.attention_block(q[h, 64 * b:64 * b + 64], k, v, ref_b, b)
            check_attention(f64(st.out[h, 64 * b:64 * b + 64]), ro, f"head {h} block {b}")


@pytest.mark.parametrize("out_dtype", [ms.OUT_BF16, ms.OUT_F32])
def test_paced_heads(out_dtype):
    """From n = 131072 on, heads served one by one whose key sets are long (on
    average 32768 keys or more per query block) run paced: launches of 1024
    workgroups (here 204 blocks of each of the five paced heads), whose
    workgroups on one XCD keep pace in 8192-key segments.  n = 262144 with
    five such heads (Vertical-Slash, Block-Sparse and A-shape of density
    0.3-0.4) beside three short ones that stay whole; blocks at pacing-segment
    edges (127/128, 511/512), at launch edges, the first and last blocks and
    random ones against the oracle, with lse; and the one-shot call bit for
    bit."""
    n = 262144
    heads = [W.vs(100, 1500), W.bs(500), W.ashape(1024, 40000), W.vs(30, 60),
             W.vs(100, 1500), W.bs(3), W.ashape(128, 900), W.vs(500, 2000)]
    w = W.custom("segments", n, 8, 2, heads, recipe="vs_planted", seed=41)
    st = run_staged(make(w, out_dtype=out_dtype), debug=False)
    sel = selections(st)
    nb = n // 64
    edges = sorted({0, 1, 127, 128, 511, 512, nb - 2, nb - 1, *_paced_launch_edges(nb, 5)})
    for h, p in enumerate(w.heads):
        blocks = sorted(set(edges[h % 2::2] + sample_blocks(nb, 2, 500 + h)))
        got_idx = read_index_blocks(st.prob, st.hp, st.index, h, blocks)
        qh = f64(st.q[h])
        kh, vh = f64(st.k[kv_of(w, h)]), f64(st.v[kv_of(w, h)])
        for b in blocks:
            if p.pattern == W.VERTICAL_SLASH:
                ref_b = oracle.vs_block_index(sel[h][1], sel[h][2], b)
            elif p.pattern == W.BLOCK_SPARSE:
                ref_b = oracle.bs_block_index(sel[h][1][b])
            else:
                ref_b = oracle.ashape_block_index(p.sink, p.window, b)
            np.testing.assert_array_equal(got_idx[b][0], ref_b[0], err_msg=f"head {h} block {b} ranges")
            np.testing.assert_array_equal(got_idx[b][1], ref_b[1], err_msg=f"head {h} block {b} cols")
            ro, rl = oracle.attention_block(qh[64 * b:64 * b + 64], kh, vh, ref_b, b, ashape=ashape_of(p))
            rows = slice(64 * b, 64 * b + 64)
            check_attention(f64(st.out[h, rows]), ro, f"head {h} block {b}", bf16_out=out_dtype == ms.OUT_BF16)
            got_l = st.lse[h, rows].cpu().numpy().astype(np.float64)
            fin = np.isfinite(rl)
            assert np.all(np.isneginf(got_l[~fin]))
            np.testing.assert_allclose(got_l[fin], rl[fin], rtol=0, atol=LSE_ATOL)
        print(f"  head {h} ({p.pattern}): blocks {blocks} ok", flush=True)
    ws = ms.empty_workspace(ms.ms_workspace_bytes(st.prob, st.hp))
    out2 = torch.empty_like(st.out)
    ms.ms_sparse_attn(st.prob, st.hp, st.q, st.k, st.v, out2, ws)
    torch.cuda.synchronize()
    assert torch.equal(out2.view(torch.int16), st.out.view(torch.int16))


def test_union_of_many_columns_per_block():
    """Four Vertical-Slash heads of one KV head, dense enough to be grouped
    through their many verticals (16000 of 32768 keys, few slashes): late
    query blocks hold more union columns than LDS takes at once, so the union
    builder merges them in several windows.  Sampled blocks against the
    oracle."""
    n = 32768
    heads = [W.vs(16000, 20)] * 4
    w = W.custom("union_cols", n, 4, 1, heads, recipe="vs_planted", seed=32)
    st = run_staged(make(w), debug=False)
    sel = selections(st)
    nb = n // 64
    blocks = [0, 7, nb // 2, nb - 2, nb - 1]
    per_head = [read_index_blocks(st.prob, st.hp, st.index, h, blocks) for h in range(4)]
    assert sum(len(per_head[h][nb - 1][1]) for h in range(4)) > 8192, "late blocks should exceed one window"
    q, k, v = f64(st.q), f64(st.k[0]), f64(st.v[0])
    for h in range(4):
        for b in blocks:
            ref_b = oracle.vs_block_index(sel[h][1], sel[h][2], b)
            np.testing.assert_array_equal(per_head[h][b][0], ref_b[0])
            np.testing.assert_array_equal(per_head[h][b][1], ref_b[1])
            ro, rl = oracle.attention_block(q[h, 64 * b:64 * b + 64], k, v, ref_b, b)
            check_attention(f64(st.out[h, 64 * b:64 * b + 64]), ro, f"head {h} block {b}")


def test_longest_sequence():
    """The longest sequence a call accepts (2^23 keys): byte offsets of K/V rows
    reach 2^31, the CSR spans 131072 query blocks.  Selections against the
    GPU's own scores, and the index and attention of sampled query blocks
    (the first, the last and random ones) against the oracle."""
    n = 1 << 23
    heads = [W.vs(16, 32), W.ashape(128, 1024)]
    w = W.custom("longest", n, 2, 1, heads, recipe="vs_planted", n_planted=2, seed=23)
    print(f"[longest] n={n}", flush=True)
    st = run_staged(make(w), debug=True)
    sel = selections(st)
    dv = st.dbg_v[0].cpu().numpy().astype(np.float64)
    ds = st.dbg_s[0].cpu().numpy().astype(np.float64)
    np.testing.assert_array_equal(sel[0][1], oracle.topk(dv, 16))
    np.testing.assert_array_equal(sel[0][2], oracle.topk(ds, 32))
    del dv, ds
    # K and V rows as float32 (exact for bf16); the oracle upcasts per block
    k32 = st.k[0].float().cpu().numpy()
    v32 = st.v[0].float().cpu().numpy()
    for h, p in enumerate(heads):
        blocks = sample_blocks(w.nb, 6, 23 + h)
        got_idx = read_index_blocks(st.prob, st.hp, st.index, h, blocks)
        for b in blocks:
            if p.pattern == W.VERTICAL_SLASH:
                ref_b = oracle.vs_block_index(sel[h][1], sel[h][2], b)
            else:
                ref_b = oracle.ashape_block_index(p.sink, p.window, b)
            np.testing.assert_array_equal(got_idx[b][0], ref_b[0], err_msg=f"head {h} block {b} ranges")
            np.testing.assert_array_equal(got_idx[b][1], ref_b[1], err_msg=f"head {h} block {b} cols")
            rows = slice(64 * b, 64 * b + 64)
            ro, rl = oracle.attention_block(f64(st.q[h, rows]), k32, v32, ref_b, b, ashape=ashape_of(p))
            check_attention(f64(st.out[h, rows]), ro, f"head {h} block {b}")
            got_l = st.lse[h, rows].cpu().numpy().astype(np.float64)
            fin = np.isfinite(rl)
            assert np.all(np.isneginf(got_l[~fin]))
            np.testing.assert_allclose(got_l[fin], rl[fin], rtol=0, atol=LSE_ATOL)
        print(f"  head {h}: {len(blocks)} blocks ok", flush=True)


def test_32_row_blocks_paced():
    """Vertical-Slash heads indexed by 32-row query blocks with long key sets
    run paced with one-wavefront workgroups (launches of 1024: 512 32-row
    blocks of each of the two paced heads).  n = 262144, two such heads
    beside a 64-row one and a short 32-row head that stays whole; 32-row
    blocks at pacing-segment edges (255/256, 1023/1024), at launch edges, the
    first, last and random ones."""
    n = 262144
    heads = [W.vs(100, 3000, block=32), W.vs(100, 1500), W.vs(50, 3000, block=32), W.vs(20, 40, block=32)]
    w = W.custom("seg32", n, 4, 2, heads, recipe="vs_planted", seed=43)
    st = run_staged(make(w), debug=False)
    sel = selections(st)
    nb32 = n // 32
    edges = sorted({0, 1, 255, 256, 1023, 1024, nb32 - 2, nb32 - 1, *_paced_launch_edges(nb32, 2)})
    q = f64(st.q)
    for h, p in enumerate(heads):
        bm = oracle.query_block_rows(p)
        kh, vh = f64(st.k[kv_of(w, h)]), f64(st.v[kv_of(w, h)])
        nbh = n // bm
        blocks = sorted({b for b in (edges if bm == 32 else [e // 2 for e in edges]) if b < nbh}
                        | set(sample_blocks(nbh, 2, 600 + h)))
        got_idx = read_index_blocks(st.prob, st.hp, st.index, h, blocks)
        for b in blocks:
            ref_b = oracle.vs_block_index(sel[h][1], sel[h][2], b, bm)
            np.testing.assert_array_equal(got_idx[b][0], ref_b[0], err_msg=f"head {h} block {b} ranges")
            np.testing.assert_array_equal(got_idx[b][1], ref_b[1], err_msg=f"head {h} block {b} cols")
            rows = slice(bm * b, bm * b + bm)
            ro, rl = oracle.attention_block(q[h, rows], kh, vh, ref_b, b, bm=bm)
            check_attention(f64(st.out[h, rows]), ro, f"head {h} block {b}")
            got_l = st.lse[h, rows].cpu().numpy().astype(np.float64)
            fin = np.isfinite(rl)
            assert np.all(np.isneginf(got_l[~fin]))
            np.testing.assert_allclose(got_l[fin], rl[fin], rtol=0, atol=LSE_ATOL)
        print(f"  head {h} ({bm}-row blocks): {len(blocks)} blocks ok", flush=True)
    ws = ms.empty_workspace(ms.ms_workspace_bytes(st.prob, st.hp))
    out2 = torch.empty_like(st.out)
    ms.ms_sparse_attn(st.prob, st.hp, st.q, st.k, st.v, out2, ws)
    torch.cuda.synchronize()
    assert torch.equal(out2.view(torch.int16), st.out.view(torch.int16))


def test_paced_results_do_not_depend_on_the_waits():
    """The paced mode orders the K/V reads only: with waiting switched off
    (every workgroup walks at its own pace) the one-shot call's out and lse
    equal the paced call's bit for bit.  n = 262144, the paced heads of the
    paced-heads layer beside short ones."""
    n = 262144
    heads = [W.vs(100, 1500), W.bs(500), W.ashape(1024, 40000), W.vs(30, 60),
             W.vs(100, 1500), W.bs(3), W.ashape(128, 900), W.vs(500, 2000)]
    w = W.custom("segments", n, 8, 2, heads, recipe="vs_planted", seed=42)
    q, k, v = W.generate(w, device="cuda")
    prob, hp = ms.problem(n, 8, 2), ms.head_params(heads)
    ws = ms.empty_workspace(ms.ms_workspace_bytes(prob, hp))
    res = []
    try:
        for polls in (4096, 0):
            ms.ms_set_pace_polls(polls)
            out = torch.empty_like(q)
            lse = torch.empty((8, n), device="cuda")
            ms.ms_sparse_attn(prob, hp, q, k, v, out, ws, lse)
            torch.cuda.synchronize()
            res.append((out, lse))
    finally:
        ms.ms_set_pace_polls(4096)
    assert torch.equal(res[0][0].view(torch.int16), res[1][0].view(torch.int16))
    assert torch.equal(res[0][1], res[1][1])
