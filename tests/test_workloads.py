"""The seeded generators: determinism, shapes and the planted structure."""
import torch

import workloads as W


def test_same_seed_same_bytes_and_shapes():
    w = W.config(3, n=512)
    a = W.generate(w)
    b = W.generate(w)
    for x, y in zip(a, b):
        assert x.dtype == torch.bfloat16
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    q, k, v = a
    assert q.shape == (32, 512, 128) and k.shape == (8, 512, 128) and v.shape == (8, 512, 128)


def test_other_seed_other_bytes():
    q0 = W.generate(W.config(0, seed=0, n=256))[0]
    q1 = W.generate(W.config(0, seed=1, n=256))[0]
    assert not torch.equal(q0, q1)


def test_mixed_head_assignment_counts():
    w = W.config(3)
    pats = [h.pattern for h in w.heads]
    assert pats.count(W.VERTICAL_SLASH) == 24
    assert pats.count(W.BLOCK_SPARSE) == 6
    assert pats.count(W.A_SHAPE) == 2
    assert w.heads == W.config(3).heads


def test_ashape_sink_keys_stretched_along_query_mean():
    w = W.config(2, n=1024)
    q, k, _ = W.generate(w)
    qf, kf = q[0].float(), k[0].float()
    u = qf.mean(0)
    u = u / u.norm()
    head = (kf[:128] @ u).abs().mean()
    tail = (kf[128:] @ u).abs().mean()
    assert head > 2.0 * tail


def test_bs_lowrank_blocks_cluster():
    w = W.config(1, n=64 * 64)
    q, k, _ = W.generate(w)
    qb = q[0].float().reshape(64, 64, 128).mean(1)
    norms = qb.norm(dim=1)
    # round(0.05 * 64) = 3 planted blocks stand out of the pooled noise.
    assert (norms > 3 * norms.median()).sum().item() == 3


def test_query_mean_makes_planted_columns_real_verticals():
    """With the shared query mean (the 1M structured diagnostic's recipe, at a
    small n) every planted column has a logit far above the others for the
    last query rows; without it the planted columns sit in the noise."""
    import oracle
    for qm, expect in ((0.5, True), (0.0, False)):
        w = W.Workload("t", 9, 8192, 1, 1, (W.vs(8, 64),), "vs_planted", n_planted=8, seed=3, query_mean=qm)
        q, k, _ = W.generate(w)
        qh, kh = q[0].double().numpy(), k[0].double().numpy()
        v, _ = oracle.vs_scores(qh[-64:], kh)
        g = W._gen(w, W._PLANT, 0, "cpu")
        planted = sorted(torch.randperm(w.n, generator=g)[:8].tolist())
        got = oracle.topk(v, 8).tolist() == planted
        assert got == expect, (qm, oracle.topk(v, 8).tolist(), planted)


def test_structured_diagnostic_is_the_1m_layer_plus_a_query_mean():
    w4, w5 = W.config(4, n=4096), W.config(5, n=4096)
    assert (w5.n_q_heads, w5.n_kv_heads, w5.heads, w5.n_planted) == (w4.n_q_heads, w4.n_kv_heads, w4.heads,
                                                                      w4.n_planted)
    assert w4.query_mean == 0.0 and w5.query_mean == 0.5
