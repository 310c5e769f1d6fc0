"""Pins of the float64 oracle against things other than itself.

Each test ties one oracle function to a closed form, a library routine with a
different code path (numpy's trace, torch's softmax / logsumexp /
scaled-dot-product attention), brute force on tiny inputs, or a fixture worked
by hand under tests/golden/.  A plausible slip in the oracle (a dropped term,
an off-by-one in a span, a flipped diagonal sign, a transposed operand, a
wrong tie-break) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle.core import BM

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- softmax / VS scores
def test_vs_rows_sum_to_one_and_causal_zeros():
    r = rng(0)
    n, L, d = 320, 64, 128
    q = r.standard_normal((L, d))
    k = r.standard_normal((n, d))
    p = oracle.vs_probabilities(q, k)
    assert np.all(np.abs(p.sum(axis=1) - 1.0) <= 1e-12)
    for rr in range(L):
        i = n - L + rr
        assert np.all(p[rr, i + 1:] == 0.0)
        assert np.all(p[rr, : i + 1] > 0.0)


def test_vs_scores_zero_query_closed_form():
    # q = 0: every allowed logit is 0, so P[i, j] = 1/(i+1) for j <= i.
    n, L, d = 256, 64, 128
    q = np.zeros((L, d))
    k = rng(1).standard_normal((n, d))
    v, s = oracle.vs_scores(q, k)
    rows = range(n - L, n)
    v_ref = np.array([sum(1.0 / (i + 1) for i in rows if i >= j) for j in range(n)])
    s_ref = np.array([sum(1.0 / (i + 1) for i in rows if i - o >= 0) for o in range(n)])
    np.testing.assert_allclose(v, v_ref, rtol=1e-13, atol=0)
    np.testing.assert_allclose(s, s_ref, rtol=1e-13, atol=0)


def test_vs_scores_against_library_routines():
    # torch.softmax over masked logits, column sums of the embedded [n, n]
    # matrix and numpy's trace along each sub-diagonal (offset -o).
    r = rng(2)
    n, L, d = 200 + 56, 64, 128
    q = r.standard_normal((L, d))
    k = r.standard_normal((n, d))
    v, s = oracle.vs_scores(q, k)
    z = torch.from_numpy(q @ k.T / math.sqrt(d))
    i = torch.arange(n - L, n)[:, None]
    z = z.masked_fill(torch.arange(n)[None, :] > i, float("-inf"))
    p = torch.softmax(z, dim=1).numpy()
    full = np.zeros((n, n))
    full[n - L:] = p
    np.testing.assert_allclose(v, full.sum(axis=0), rtol=1e-12, atol=1e-15)
    s_ref = np.array([np.trace(full, offset=-o) for o in range(n)])
    np.testing.assert_allclose(s, s_ref, rtol=1e-12, atol=1e-15)


def test_vs_one_hot_key_is_top_vertical():
    r = rng(3)
    n, L, d = 512, 64, 128
    q = r.standard_normal((L, d)) * 0.1
    k = r.standard_normal((n, d)) * 0.1
    jstar = 77
    k[jstar] = 40.0 * q.mean(axis=0) / np.linalg.norm(q.mean(axis=0))
    v, s = oracle.vs_scores(q, k)
    assert oracle.topk(v, 1).tolist() == [jstar]


def test_vs_pure_diagonal_is_top_slash():
    # Keys equal to their own query (large) make offset 0 dominate.
    r = rng(4)
    n, L, d = 512, 64, 128
    qfull = r.standard_normal((n, d))
    k = r.standard_normal((n, d)) * 0.05
    k += 3.0 * qfull
    v, s = oracle.vs_scores(qfull[n - L:], k)
    assert oracle.topk(s, 1).tolist() == [0]


# ---------------------------------------------------------------- top-k
def _topk_brute(x, k):
    x = list(map(float, x))
    chosen = []
    alive = set(range(len(x)))
    for _ in range(min(k, len(x))):
        best = None
        for i in sorted(alive):
            if best is None or x[i] > x[best]:
                best = i
        chosen.append(best)
        alive.remove(best)
    return sorted(chosen)


@pytest.mark.parametrize("seed", range(6))
def test_topk_matches_brute_force_with_ties(seed):
    r = rng(10 + seed)
    n = int(r.integers(1, 300))
    x = r.integers(-5, 6, size=n).astype(np.float64)   # many exact ties
    for k in (0, 1, 7, n // 2, n, n + 3):
        assert oracle.topk(x, k).tolist() == _topk_brute(x, k)


def test_topk_signed_zero_and_ascending_output():
    x = np.array([0.0, -0.0, 1.0, -0.0, 0.0, 2.0])
    # -0 and +0 compare equal, so the lower indices win among the zeros.
    assert oracle.topk(x, 3).tolist() == [0, 2, 5]
    assert oracle.topk(x, 4).tolist() == [0, 1, 2, 5]


# ---------------------------------------------------------------- Block-Sparse
def _integer_blocks(coeffs, d=128, delta=0.25):
    """Block b's rows are coeffs[b]*e1 plus +-delta*e2 in pairs; the mean is exactly coeffs[b]*e1."""
    rows = []
    for a in coeffs:
        blk = np.zeros((BM, d))
        blk[:, 0] = a
        blk[0::2, 1] = delta
        blk[1::2, 1] = -delta
        rows.append(blk)
    return np.concatenate(rows)


def test_bs_integer_construction_hand_worked():
    # Pooled means are exactly a_b e1, so S[b, c] = a_b * a_c.
    qa = [1, 2, -1, 2, 0, 3]
    ka = [1, 2, -1, 2, 0, 3]
    q, k = _integer_blocks(qa), _integer_blocks(ka)
    sc = oracle.bs_scores(q, k)
    np.testing.assert_array_equal(oracle.bs_pool(q)[:, 0], qa)
    np.testing.assert_array_equal(oracle.bs_pool(q)[:, 1], 0.0)
    # Row b = 5: S = 3*[1, 2, -1, 2, 0, 3] = [3, 6, -3, 6, 0, 9].
    np.testing.assert_array_equal(sc[5], [3, 6, -3, 6, 0, 9])
    assert np.all(np.isneginf(sc[0, 1:]))
    sel = oracle.bs_select(sc, 2)
    # b=0: only c=0.  b=1: S=[2,4] -> both.  b=2: S=[-1,-2,1] -> {0,2}.
    # b=3: S=[2,4,-2,4] -> 4 at c=1 and c=3 -> {1,3}.  b=4: S all 0 -> lowest {0,1}.
    # b=5: 9 at c=5, then the tie 6 at c=1 and c=3 goes to c=1 -> {1,5}.
    assert [s.tolist() for s in sel] == [[0], [0, 1], [0, 2], [1, 3], [0, 1], [1, 5]]
    sel3 = oracle.bs_select(sc, 3)
    assert sel3[5].tolist() == [1, 3, 5]


def test_bs_pool_is_block_mean():
    r = rng(20)
    x = r.standard_normal((4 * BM, 128))
    ref = np.stack([x[b * BM:(b + 1) * BM].sum(axis=0) / BM for b in range(4)])
    np.testing.assert_allclose(oracle.bs_pool(x), ref, rtol=1e-13, atol=1e-15)


def test_bs_index_merges_consecutive_blocks():
    ranges, cols = oracle.bs_block_index(np.array([0, 1, 3, 5, 6, 7, -1, -1]))
    assert ranges.tolist() == [[0, 128], [192, 256], [320, 512]]
    assert cols.size == 0


# ---------------------------------------------------------------- index conversion
def test_vs_index_golden_hand_worked():
    g = json.load(open(os.path.join(GOLDEN, "vs_index_n512.json")))
    idx = oracle.vs_index(np.array(g["vertical"]), np.array(g["slash"]), g["n"])
    for blk in g["blocks"]:
        r, c = idx[blk["b"]]
        assert r.tolist() == blk["ranges"], blk
        assert c.tolist() == blk["cols"], blk


def test_ashape_index_golden_hand_worked():
    g = json.load(open(os.path.join(GOLDEN, "ashape_index_n512.json")))
    idx = oracle.ashape_index(g["sink"], g["window"], g["n"])
    for blk in g["blocks"]:
        assert idx[blk["b"]][0].tolist() == blk["ranges"], blk
    rm = g["row_masks"][0]
    b = rm["row"] // BM
    m = oracle.block_mask(idx[b], b, g["n"], ashape=(g["sink"], g["window"]))[rm["row"] % BM]
    kept = np.nonzero(m)[0]
    assert kept.tolist() == list(range(rm["sink_kept"])) + list(range(rm["kept_lo"], rm["kept_hi"] + 1))


def _vs_mask_by_definition(vert, slash, n):
    """(i, j) kept iff j <= i and (j is a vertical, or some slash o reaching block(i)
    has 64b - o <= j < 64b + 64 - o); built element by element."""
    vert, slash = set(int(x) for x in vert), [int(x) for x in slash]
    m = np.zeros((n, n), dtype=bool)
    for i in range(n):
        b = i // BM
        row0 = b * BM
        for j in range(i + 1):
            keep = j in vert
            if not keep:
                for o in slash:
                    if o <= row0 + BM - 1 and row0 - o <= j < row0 + BM - o:
                        keep = True
                        break
            m[i, j] = keep
    return m


@pytest.mark.parametrize("seed", range(4))
def test_vs_index_matches_elementwise_definition(seed):
    r = rng(30 + seed)
    n = 256
    vert = np.sort(r.choice(n, size=int(r.integers(1, 12)), replace=False))
    slash = np.sort(r.choice(n, size=int(r.integers(1, 10)), replace=False))
    idx = oracle.vs_index(vert, slash, n)
    ref = _vs_mask_by_definition(vert, slash, n)
    got = np.concatenate([oracle.block_mask(idx[b], b, n) for b in range(n // BM)])
    np.testing.assert_array_equal(got, ref)
    # Canonical form: sorted, disjoint and non-touching ranges inside [0, 64b+64);
    # columns ascending, causal for the block, and outside every range.
    for b, (rg, cols) in enumerate(idx):
        end = b * BM + BM
        assert np.all(rg[:, 0] < rg[:, 1])
        assert np.all(rg[1:, 0] > rg[:-1, 1])
        assert np.all((rg >= 0) & (rg <= end))
        assert np.all(np.diff(cols) > 0)
        assert np.all(cols < end)
        for j in cols:
            assert not np.any((rg[:, 0] <= j) & (j < rg[:, 1]))


def test_csr_round_trip():
    r = rng(40)
    n = 512
    idx = oracle.vs_index(np.sort(r.choice(n, 9, replace=False)), np.sort(r.choice(n, 7, replace=False)), n)
    back = oracle.csr_to_index(*oracle.index_to_csr(idx))
    for (a, b), (c, d) in zip(idx, back):
        np.testing.assert_array_equal(a, c)
        np.testing.assert_array_equal(b, d)


# ---------------------------------------------------------------- attention
def _qkv(seed, n, d=128, scale=1.0):
    r = rng(seed)
    return (r.standard_normal((n, d)) * scale, r.standard_normal((n, d)) * scale,
            r.standard_normal((n, d)))


def test_dense_equals_torch_causal_sdpa():
    n = 256
    q, k, v = _qkv(50, n)
    out, lse = oracle.attention_head(q, k, v, oracle.dense_index(n))
    tq, tk, tv = (torch.from_numpy(x)[None, None] for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)[0, 0].numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)
    z = torch.from_numpy(q @ k.T / math.sqrt(128)).masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(z, dim=1).numpy(), rtol=1e-12, atol=1e-12)


def test_zero_query_gives_masked_mean_of_values():
    # q = 0: all allowed logits tie, so out_i is the plain mean of v over row i's keys.
    n = 512
    _, k, v = _qkv(51, n)
    q = np.zeros_like(k)
    r = rng(52)
    vert = np.sort(r.choice(n, 6, replace=False))
    slash = np.sort(r.choice(n, 5, replace=False))
    idx = oracle.vs_index(vert, slash, n)
    out, lse = oracle.attention_head(q, k, v, idx)
    mask = _vs_mask_by_definition(vert, slash, n)
    for i in range(n):
        js = np.nonzero(mask[i])[0]
        if js.size == 0:
            assert np.all(out[i] == 0) and np.isneginf(lse[i])
        else:
            np.testing.assert_allclose(out[i], v[js].mean(axis=0), rtol=1e-11, atol=1e-13)
            assert abs(lse[i] - math.log(js.size)) < 1e-12


def test_single_key_per_row_returns_own_value():
    n = 256
    q, k, v = _qkv(53, n)
    out, _ = oracle.attention_head(q, k, v, oracle.ashape_index(0, 1, n), ashape=(0, 1))
    np.testing.assert_array_equal(out, v)


@pytest.mark.parametrize("case", ["ashape_wide", "bs_all", "vs_all_offsets"])
def test_full_coverage_reduces_to_dense(case):
    n = 320
    q, k, v = _qkv(54, n)
    ref, ref_lse = oracle.attention_head(q, k, v, oracle.dense_index(n))
    if case == "ashape_wide":
        out, lse = oracle.attention_head(q, k, v, oracle.ashape_index(0, n, n), ashape=(0, n))
    elif case == "bs_all":
        out, lse = oracle.attention_head(q, k, v, oracle.bs_index(oracle.bs_select(oracle.bs_scores(q, k), n // BM)))
    else:
        out, lse = oracle.attention_head(q, k, v, oracle.vs_index(np.arange(0), np.arange(n), n))
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-13, atol=1e-13)


def test_attention_brute_force_masked_softmax():
    # Full [n, n] masked softmax from the element-wise mask definition.
    n = 256
    q, k, v = _qkv(55, n)
    r = rng(56)
    vert = np.sort(r.choice(n, 10, replace=False))
    slash = np.sort(r.choice(n, 4, replace=False))
    out, _ = oracle.attention_head(q, k, v, oracle.vs_index(vert, slash, n))
    mask = _vs_mask_by_definition(vert, slash, n)
    z = torch.from_numpy(q @ k.T / math.sqrt(128)).masked_fill(~torch.from_numpy(mask), float("-inf"))
    p = torch.softmax(z, dim=1).nan_to_num(0.0).numpy()
    np.testing.assert_allclose(out, p @ v, rtol=1e-11, atol=1e-13)


def test_attention_invariant_to_range_and_column_order():
    n = 384
    q, k, v = _qkv(57, n)
    idx = oracle.vs_index(np.array([3, 90, 200, 333]), np.array([0, 40, 150]), n)
    shuffled = [(rg[::-1].copy(), c[::-1].copy()) for rg, c in idx]
    a, _ = oracle.attention_head(q, k, v, idx)
    b, _ = oracle.attention_head(q, k, v, shuffled)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------- index quality (attention-mass recall)
def test_recall_of_dense_index_is_one():
    r = rng(40)
    n, d = 256, 128
    q, k = r.standard_normal((n, d)), r.standard_normal((n, d))
    m = oracle.attention_recall(q, k, oracle.dense_index(n))
    assert np.all(np.abs(m - 1.0) <= 1e-12)


def test_recall_zero_query_closed_form():
    # q = 0: row i spreads its mass evenly over keys 0..i, so keeping key 0
    # alone (one vertical, no slash) captures 1 / (i + 1) of it.
    n, d = 320, 128
    q = np.zeros((n, d))
    k = rng(41).standard_normal((n, d))
    idx = oracle.vs_index(np.array([0]), np.zeros(0, dtype=np.int64), n)
    m = oracle.attention_recall(q, k, idx)
    np.testing.assert_allclose(m, 1.0 / (np.arange(n) + 1.0), rtol=0, atol=1e-14)


def test_recall_is_ratio_of_normalisers():
    # The identity the GPU instrument uses: kept mass = exp(lse_kept - lse_all),
    # with both log-sum-exps from torch on a different code path.
    r = rng(42)
    n, d = 256, 128
    q, k = r.standard_normal((n, d)), r.standard_normal((n, d))
    heads = [(oracle.vs_index(np.array([3, 90]), np.array([0, 17, 64]), n), None),
             (oracle.ashape_index(8, 40, n), (8, 40))]
    for idx, ash in heads:
        m = oracle.attention_recall(q, k, idx, ashape=ash)
        z = torch.from_numpy(q @ k.T / math.sqrt(d))
        causal = torch.ones(n, n, dtype=torch.bool).tril()
        kept = torch.from_numpy(np.concatenate([oracle.block_mask(idx[b], b, n, ash) for b in range(n // BM)]))
        lse_all = torch.logsumexp(z.masked_fill(~causal, -math.inf), dim=1)
        lse_kept = torch.logsumexp(z.masked_fill(~kept, -math.inf), dim=1)
        np.testing.assert_allclose(m, torch.exp(lse_kept - lse_all).numpy(), rtol=1e-12, atol=1e-15)


def test_recall_brute_force_tiny():
    r = rng(43)
    n, d = 128, 4
    q, k = r.standard_normal((n, d)), r.standard_normal((n, d))
    idx = oracle.bs_index([np.array([0])] + [np.array([1])])
    m = oracle.attention_recall(q, k, idx)
    for i in range(0, n, 7):
        w = [math.exp(float(q[i] @ k[j]) / 2.0) for j in range(i + 1)]   # 1/sqrt(4) = 1/2
        kept = [j for j in range(i + 1) if (i < 64 and j < 64) or (i >= 64 and 64 <= j < 128)]
        assert abs(m[i] - sum(w[j] for j in kept) / sum(w)) <= 1e-12


def test_topk_mass_exhaustive_and_bounds_any_index():
    import itertools
    r = rng(44)
    n, d = 8, 3
    q, k = r.standard_normal((n, d)), r.standard_normal((n, d))
    rows = list(range(n))
    for kk in range(0, 5):
        got = oracle.topk_mass(q, k, rows, [min(kk, i + 1) for i in rows])
        for i in rows:
            z = np.array([float(q[i] @ k[j]) / math.sqrt(d) for j in range(i + 1)])
            p = np.exp(z - z.max())
            p /= p.sum()
            best = max((sum(p[list(c)]) for c in itertools.combinations(range(i + 1), min(kk, i + 1))), default=0.0)
            assert abs(got[i] - best) <= 1e-12
    # no index keeps more mass per row than the top entries with its own budget
    n, d = 256, 128
    q, k = r.standard_normal((n, d)), r.standard_normal((n, d))
    idx = oracle.vs_index(np.array([5, 77]), np.array([0, 3, 40]), n)
    m = oracle.attention_recall(q, k, idx)
    budget = np.concatenate([oracle.block_mask(idx[b], b, n).sum(axis=1) for b in range(n // BM)])
    rows = list(range(0, n, 5))
    best = oracle.topk_mass(q, k, rows, budget[rows])
    assert np.all(m[rows] <= best + 1e-12)


# ------------------------------------------------------------ chunked prefill
@pytest.mark.parametrize("q_block0", [1, 7, 11])
def test_chunk_estimation_and_index_restrict_the_whole_sequence(q_block0):
    """A chunk of query blocks q_block0.. (with every key present) estimates
    and indexes exactly as the whole sequence does for those blocks: the
    Vertical-Slash selections are equal (same last 64 rows), the Block-Sparse
    selections and every block's index are the whole sequence's from block
    q_block0 on, and so is attention."""
    rng = np.random.default_rng(40 + q_block0)
    n, d = 64 * 12, 128
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    k[200] += 2.0 * q[-64:].mean(axis=0)  # one strong vertical
    qc = q[q_block0 * BM:]
    for params in (W.vs(8, 12), W.bs(3), W.ashape(20, 70), W.dense()):
        full = oracle.estimate_head(params, q, k)
        chunk = oracle.estimate_head(params, qc, k, q_block0=q_block0)
        if params.pattern == W.VERTICAL_SLASH:
            np.testing.assert_array_equal(chunk[1], full[1])
            np.testing.assert_array_equal(chunk[2], full[2])
        elif params.pattern == W.BLOCK_SPARSE:
            assert len(chunk[1]) == n // BM - q_block0
            for r, sel in enumerate(chunk[1]):
                np.testing.assert_array_equal(sel, full[1][q_block0 + r])
        idx_full = oracle.head_index(params, full, n)
        idx_chunk = oracle.head_index(params, chunk, n, q_block0=q_block0)
        assert len(idx_chunk) == n // BM - q_block0
        ashape = (params.sink, params.window) if params.pattern == W.A_SHAPE else None
        for r, bidx in enumerate(idx_chunk):
            b = q_block0 + r
            np.testing.assert_array_equal(bidx[0], idx_full[b][0])
            np.testing.assert_array_equal(bidx[1], idx_full[b][1])
            o1, l1 = oracle.attention_block(qc[r * BM:(r + 1) * BM], k, v, bidx, b, ashape=ashape)
            o2, l2 = oracle.attention_block(q[b * BM:(b + 1) * BM], k, v, idx_full[b], b, ashape=ashape)
            np.testing.assert_array_equal(o1, o2)
            np.testing.assert_array_equal(l1, l2)


def test_chunk_block_scores_are_rows_of_the_full_matrix():
    rng = np.random.default_rng(3)
    n, d = 64 * 9, 128
    q, k = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    full = oracle.bs_scores(q, k)
    part = oracle.bs_scores(q[4 * BM:], k, q_block0=4)
    assert part.shape == (5, 9)
    np.testing.assert_array_equal(part, full[4:])
    assert np.isneginf(part[0, 5:]).all() and np.isfinite(part[0, :5]).all()


# ------------------------------------------------------------ Grid pattern
def test_grid_index_hand_worked():
    """Reading R16 worked by hand.  P = 100, T = 2, w = 2, window = 10:
    offsets {0..9} u {98..102} u {198..202}.  Block 3 (rows 192..255): the
    local run gives keys [192-9, 256) = [183, 256); 98..102 (gap 89 > 64 from
    9) gives [192-102, 256-98) = [90, 158); 198..202 (gap 96) gives
    [max(0, -10), 58) = [0, 58).  Block 1 (rows 64..127): [0, 30) and
    [55, 128); 198 > 127 reaches nothing.  P = 50, w = 10, window = 20,
    T = 2: offsets 0..19, 40..60, 90..110 lie within 64 of each other, one run
    0..110: block 2 (rows 128..191) keeps [128-110, 192) = [18, 192)."""
    n = 64 * 8
    r, c = oracle.grid_block_index(100, 2, 2, 10, 3, n)
    np.testing.assert_array_equal(r, [[0, 58], [90, 158], [183, 256]])
    assert c.size == 0
    r, _ = oracle.grid_block_index(100, 2, 2, 10, 1, n)
    np.testing.assert_array_equal(r, [[0, 30], [55, 128]])
    r, _ = oracle.grid_block_index(50, 2, 10, 20, 2, n)
    np.testing.assert_array_equal(r, [[18, 192]])
    np.testing.assert_array_equal(oracle.grid_offsets(100, 2, 2, 10, n),
                                  list(range(10)) + list(range(98, 103)) + list(range(198, 203)))


@pytest.mark.parametrize("params", [(7, 3, 1, 4), (100, 5, 3, 50), (64, 2, 0, 1), (30, 9, 20, 200), (1, 1, 0, 1)])
def test_grid_mask_elementwise(params):
    """Brute force on a small sequence: row i of block b keeps key j iff j <= i
    and some kept offset o has j in the block's span [64b - o, 64b + 63 - o]."""
    P, T, w, W = params
    n = 64 * 6
    offs = set(range(min(W, n))) | {t * P + d for t in range(1, T + 1) for d in range(-w, w + 1) if 0 <= t * P + d < n}
    for b in range(n // 64):
        got = oracle.block_mask(oracle.grid_block_index(P, T, w, W, b, n), b, n)
        ref = np.zeros((64, n), dtype=bool)
        for r in range(64):
            i = 64 * b + r
            for j in range(i + 1):
                ref[r, j] = any(64 * b - o <= j <= 64 * b + 63 - o for o in offs)
        np.testing.assert_array_equal(got, ref)


# ------------------------------------------------------------ per-head dispatch
# head_index and estimate_head route one head's pattern and parameters to the
# per-pattern functions pinned above; these tests push the hand-worked fixtures
# and constructions through the dispatch itself, so a swapped argument or a
# wrong branch there fails here.
def _assert_index(got, blocks, b0=0):
    for blk in blocks:
        b = blk["b"]
        if b < b0:
            continue
        r, c = got[b - b0]
        assert r.tolist() == blk["ranges"], blk
        assert c.tolist() == blk.get("cols", []), blk


@pytest.mark.parametrize("q_block0", [0, 3])
def test_head_index_vertical_slash_golden(q_block0):
    g = json.load(open(os.path.join(GOLDEN, "vs_index_n512.json")))
    p = W.vs(len(g["vertical"]), len(g["slash"]))
    sel = ("vs", np.array(g["vertical"]), np.array(g["slash"]))
    got = oracle.head_index(p, sel, g["n"], q_block0=q_block0)
    assert len(got) == g["n"] // BM - q_block0
    _assert_index(got, g["blocks"], q_block0)


@pytest.mark.parametrize("q_block0", [0, 2])
def test_head_index_ashape_golden(q_block0):
    g = json.load(open(os.path.join(GOLDEN, "ashape_index_n512.json")))
    got = oracle.head_index(W.ashape(g["sink"], g["window"]), ("static",), g["n"], q_block0=q_block0)
    assert len(got) == g["n"] // BM - q_block0
    _assert_index(got, g["blocks"], q_block0)


def test_head_index_grid_hand_worked():
    # The cases worked by hand in test_grid_index_hand_worked, through the
    # dispatch: P = 100, T = 2, w = 2, window = 10, and P = 50, T = 2, w = 10,
    # window = 20.
    n = 64 * 8
    got = oracle.head_index(W.grid(100, 2, 2, 10), ("static",), n)
    assert got[3][0].tolist() == [[0, 58], [90, 158], [183, 256]]
    assert got[1][0].tolist() == [[0, 30], [55, 128]]
    assert all(c.size == 0 for _, c in got)
    got = oracle.head_index(W.grid(50, 2, 10, 20), ("static",), n)
    assert got[2][0].tolist() == [[18, 192]]
    got = oracle.head_index(W.grid(100, 2, 2, 10), ("static",), n, q_block0=3)
    assert got[0][0].tolist() == [[0, 58], [90, 158], [183, 256]]


def test_head_index_block_sparse_hand_worked():
    # Selections of test_bs_integer_construction_hand_worked: block c keeps
    # keys [64c, 64c + 64); consecutive blocks merge.
    sel = [np.array(s) for s in ([0], [0, 1], [0, 2], [1, 3], [0, 1], [1, 5])]
    got = oracle.head_index(W.bs(2), ("bs", sel), 6 * BM)
    assert [r.tolist() for r, _ in got] == [[[0, 64]], [[0, 128]], [[0, 64], [128, 192]], [[64, 128], [192, 256]],
                                            [[0, 128]], [[64, 128], [320, 384]]]
    assert all(c.size == 0 for _, c in got)


@pytest.mark.parametrize("q_block0", [0, 5])
def test_head_index_dense(q_block0):
    n = 64 * 7
    got = oracle.head_index(W.dense(), ("static",), n, q_block0=q_block0)
    assert [r.tolist() for r, _ in got] == [[[0, 64 * b + 64]] for b in range(q_block0, 7)]
    assert all(c.size == 0 for _, c in got)


def _one_hot_rows(n, plants, lam=30.0, d=128, seed=60):
    """Zero queries except row i = lam * e_t for each plant (i, j, t); key j =
    lam * e_t; every other key is random in the span of e_8 .. e_127, so it is
    orthogonal to every planted query and its logits are exactly 0."""
    r = rng(seed)
    q = np.zeros((n, d))
    k = np.zeros((n, d))
    k[:, 8:] = r.standard_normal((n, d - 8))
    for i, j, t in plants:
        q[i, t] = lam
        k[j] = 0.0
        k[j, t] = lam
    return q, k


def test_estimate_head_scores_exactly_the_last_64_rows():
    # Rows n-64 and n-1 each see one planted key strongly; row n-65 (outside
    # the last 64) sees a third.  Every other logit is 0, so the remaining
    # vertical scores tie and the lowest index fills the budget.  Scoring rows
    # n-64..n-1 gives verticals {0, 100, 300} and slashes {(n-1) - 300,
    # (n-64) - 100}; one row fewer at either end or one more changes them.
    n = 512
    q, k = _one_hot_rows(n, [(n - 64, 100, 0), (n - 1, 300, 1), (n - 65, 200, 2)])
    sel = oracle.estimate_head(W.vs(3, 2), q, k)
    assert sel[0] == "vs"
    assert sel[1].tolist() == [0, 100, 300]
    assert sel[2].tolist() == [(n - 1) - 300, (n - 64) - 100]
    # the same through a chunk whose query rows start at block 5
    sel_c = oracle.estimate_head(W.vs(3, 2), q[5 * BM:], k, q_block0=5)
    assert sel_c[1].tolist() == [0, 100, 300]
    assert sel_c[2].tolist() == [(n - 1) - 300, (n - 64) - 100]


def test_estimate_head_zero_query_scores_closed_form():
    # q = 0 on the last 64 rows: v_j = sum over rows i >= max(j, n-64) of
    # 1/(i+1) ties for every j < n - 64, so the top k verticals are 0..k-1;
    # a key planted for row n-64 only breaks that tie (row n-64 is scored).
    n = 448
    q, k = _one_hot_rows(n, [(n - 64, 250, 3)], lam=0.0)
    sel = oracle.estimate_head(W.vs(4, 3), q, k)
    assert sel[1].tolist() == [0, 1, 2, 3]
    # s_o = sum over rows i >= max(o, n-64) of 1/(i+1) ties for o <= n - 64
    assert sel[2].tolist() == [0, 1, 2]
    q, k = _one_hot_rows(n, [(n - 64, 250, 3)])
    sel = oracle.estimate_head(W.vs(4, 3), q, k)
    assert sel[1].tolist() == [0, 1, 2, 250]
    assert (n - 64) - 250 in sel[2].tolist()


def test_estimate_head_block_sparse_integer_construction():
    # The integer construction of test_bs_integer_construction_hand_worked,
    # through the dispatch, whole and as a chunk from query block 3.
    qa = [1, 2, -1, 2, 0, 3]
    q, k = _integer_blocks(qa), _integer_blocks(qa)
    sel = oracle.estimate_head(W.bs(2), q, k)
    assert sel[0] == "bs"
    assert [s.tolist() for s in sel[1]] == [[0], [0, 1], [0, 2], [1, 3], [0, 1], [1, 5]]
    sel = oracle.estimate_head(W.bs(2), q[3 * BM:], k, q_block0=3)
    assert [s.tolist() for s in sel[1]] == [[1, 3], [0, 1], [1, 5]]


def test_estimate_head_static_patterns_select_nothing():
    q = np.zeros((128, 128))
    for p in (W.ashape(4, 8), W.dense(), W.grid(10, 1, 0, 4)):
        assert oracle.estimate_head(p, q, q) == ("static",)



# ------------------------------------------------------------ 32-row query blocks (reading R17)
def _vs_mask_rows(vert, slash, n, bm):
    """(i, j) kept iff j <= i and (j is a vertical, or some slash o reaching
    block i // bm has bm*b - o <= j < bm*b + bm - o); element by element."""
    vert, slash = set(int(x) for x in vert), [int(x) for x in slash]
    m = np.zeros((n, n), dtype=bool)
    for i in range(n):
        row0 = (i // bm) * bm
        for j in range(i + 1):
            keep = j in vert
            if not keep:
                for o in slash:
                    if o <= row0 + bm - 1 and row0 - o <= j < row0 + bm - o:
                        keep = True
                        break
            m[i, j] = keep
    return m


def test_vs_index_32_row_blocks_golden_hand_worked():
    g = json.load(open(os.path.join(GOLDEN, "vs_index_bm32_n256.json")))
    idx = oracle.vs_index(np.array(g["vertical"]), np.array(g["slash"]), g["n"], bm=32)
    assert len(idx) == g["n"] // 32
    for blk in g["blocks"]:
        r, c = idx[blk["b"]]
        assert r.tolist() == blk["ranges"], blk
        assert c.tolist() == blk["cols"], blk
    # through the per-head dispatch: block = 32 asks for 32-row blocks
    p = W.HeadParams(W.VERTICAL_SLASH, n_vertical=4, n_slash=5, block=32)
    assert oracle.query_block_rows(p) == 32 and oracle.query_block_rows(W.vs(4, 5)) == 64
    got = oracle.head_index(p, ("vs", np.array(g["vertical"]), np.array(g["slash"])), g["n"])
    _assert_index(got, g["blocks"])
    got = oracle.head_index(p, ("vs", np.array(g["vertical"]), np.array(g["slash"])), g["n"], q_block0=2)
    assert len(got) == 4
    _assert_index(got, g["blocks"], 4)


@pytest.mark.parametrize("seed", range(4))
def test_vs_index_32_row_blocks_match_elementwise_definition(seed):
    r = rng(80 + seed)
    n = 256
    vert = np.sort(r.choice(n, size=int(r.integers(1, 12)), replace=False))
    slash = np.sort(r.choice(n, size=int(r.integers(1, 10)), replace=False))
    idx = oracle.vs_index(vert, slash, n, bm=32)
    ref = _vs_mask_rows(vert, slash, n, 32)
    got = np.concatenate([oracle.block_mask(idx[b], b, n, bm=32) for b in range(n // 32)])
    np.testing.assert_array_equal(got, ref)
    # the 64-row definition is the same brute force with 64
    np.testing.assert_array_equal(_vs_mask_rows(vert, slash, n, 64), _vs_mask_by_definition(vert, slash, n))
    # canonical form, and every 32-row block keeps a subset of its 64-row block
    m64 = np.concatenate([oracle.block_mask(b64, b, n) for b, b64 in enumerate(oracle.vs_index(vert, slash, n))])
    assert not np.any(got & ~m64)
    for b, (rg, cols) in enumerate(idx):
        end = 32 * b + 32
        assert np.all(rg[:, 0] < rg[:, 1]) and np.all(rg[1:, 0] > rg[:-1, 1])
        assert np.all((rg >= 0) & (rg <= end)) and np.all(np.diff(cols) > 0) and np.all(cols < end)


def test_single_slash_keeps_one_32_key_span_per_row():
    # One slash o: row i of 32-row block b keeps keys [32b - o, 32b + 32 - o) up
    # to its own diagonal, i.e. min(32, i - (32b - o) + 1) keys when they exist.
    n, o = 256, 40
    idx = oracle.vs_index(np.zeros(0, dtype=np.int64), np.array([o]), n, bm=32)
    m = np.concatenate([oracle.block_mask(idx[b], b, n, bm=32) for b in range(n // 32)])
    for i in range(n):
        lo = 32 * (i // 32) - o
        want = [j for j in range(max(0, lo), min(lo + 32, i + 1))]
        assert np.nonzero(m[i])[0].tolist() == want, i


def test_attention_32_row_blocks_brute_force_and_full_coverage():
    n = 256
    q, k, v = _qkv(81, n)
    r = rng(82)
    vert = np.sort(r.choice(n, 9, replace=False))
    slash = np.sort(r.choice(n, 5, replace=False))
    out, lse = oracle.attention_head(q, k, v, oracle.vs_index(vert, slash, n, bm=32), bm=32)
    mask = _vs_mask_rows(vert, slash, n, 32)
    z = torch.from_numpy(q @ k.T / math.sqrt(128)).masked_fill(~torch.from_numpy(mask), float("-inf"))
    p = torch.softmax(z, dim=1).nan_to_num(0.0).numpy()
    np.testing.assert_allclose(out, p @ v, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(lse, torch.logsumexp(z, dim=1).numpy(), rtol=1e-12, atol=1e-12)
    # every offset kept: 32-row blocks reduce to dense causal attention too
    ref, _ = oracle.attention_head(q, k, v, oracle.dense_index(n))
    full, _ = oracle.attention_head(q, k, v, oracle.vs_index(np.arange(0), np.arange(n), n, bm=32), bm=32)
    np.testing.assert_allclose(full, ref, rtol=1e-12, atol=1e-14)
