"""The kernel-aware pattern search: selection logic on the host, and a run on
the GPU whose choices must be consistent with its own measurements and whose
measured recall matches the oracle's."""
import numpy as np
import pytest
import torch

import dynamic_sparse_attention_est_amd as ms
from dynamic_sparse_attention_est_amd import search
import oracle
import workloads as W


def test_choose_takes_cheapest_candidate_reaching_the_target():
    a = search.Candidate(ms.A_SHAPE, sink=128, window=1024)
    b = search.Candidate(ms.VERTICAL_SLASH, n_vertical=100, n_slash=512)
    c = search.Candidate(ms.BLOCK_SPARSE, top_k_blocks=50)
    trials = [search.Trial(a, 1.0, [0.97, 0.50, 0.10]),
              search.Trial(b, 2.0, [0.99, 0.96, 0.20]),
              search.Trial(c, 0.5, [0.90, 0.99, 0.30])]
    picks = search.choose(trials, 3, 0.95)
    assert picks == [a, c, None]
    # equal cost: the earlier candidate stays
    t2 = [search.Trial(a, 1.0, [0.99]), search.Trial(b, 1.0, [0.99])]
    assert search.choose(t2, 1, 0.9) == [a]
    # dense attention wins when it is cheaper than every candidate that qualifies
    assert search.choose(trials, 3, 0.95, dense_ms=0.75) == [None, c, None]


@pytest.mark.parametrize("n", [4096, 32768, 131072])
def test_default_candidates_are_valid(n):
    for c in search.default_candidates(n):
        ms.ms_validate(ms.problem(n, 1, 1), ms.head_params([c]))
    assert {c.pattern for c in search.default_candidates(n)} == {ms.A_SHAPE, ms.VERTICAL_SLASH, ms.BLOCK_SPARSE}


@pytest.mark.gpu
def test_search_layer_choices_match_its_measurements():
    w = W.config(3, n=8192)
    q, k, v = W.generate(w, device="cuda")
    target = 0.9
    picks, trials, dense_ms = search.search_layer(q, k, v, target=target, repeats=1)
    assert len(picks) == w.n_q_heads and dense_ms > 0
    for t in trials:
        assert t.ms_per_head > 0 and all(0.0 <= r <= 1.0 + 1e-3 for r in t.recall)
    for h, p in enumerate(picks):
        ok = [t for t in trials if t.recall[h] >= target]
        if p.pattern == ms.DENSE:
            assert not ok or all(dense_ms < t.ms_per_head for t in ok)
        else:
            mine = next(t for t in trials if t.candidate == p)
            assert mine.recall[h] >= target and mine.ms_per_head <= dense_ms
            assert all(mine.ms_per_head <= t.ms_per_head for t in ok)
    # A trial's recall is the float64 oracle's attention-mass recall of that
    # candidate's index (an A-shape candidate, whose index is fixed by its
    # parameters), within twice the log-sum-exp tolerance per row.
    a = next(t for t in trials if t.candidate.pattern == ms.A_SHAPE)
    sink, window = a.candidate.sink, a.candidate.window
    q64 = q.float().cpu().numpy().astype(np.float64)
    k64 = k.float().cpu().numpy().astype(np.float64)
    for h in (0, w.n_q_heads - 1):
        ref = oracle.attention_recall(q64[h], k64[h // w.group], oracle.ashape_index(sink, window, w.n),
                                      ashape=(sink, window)).mean()
        assert abs(a.recall[h] - ref) <= 2.5e-3, f"head {h}: recall {a.recall[h]:.6f} vs {ref:.6f}"
