"""The C ABI library on a machine without a GPU: it loads, exports every
symbol include/msattn.h declares, and rejects bad arguments on the host
before enqueueing anything (no call here reaches a HIP launch)."""
import ctypes

import numpy as np
import os
import re

import pytest

import dynamic_sparse_attention_est_amd as ms
import oracle
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msattn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(ms.library_path()), reason="libmsattn.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ms_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = ms.load()
    names = declared_functions()
    assert len(names) >= 15
    for name in names:
        assert hasattr(lib, name), name


def test_version_and_status_strings():
    lib = ms.load()
    assert ms.ms_version() == 10000
    assert lib.ms_status_string(0) == b"ok"
    assert lib.ms_status_string(3) == b"insufficient capacity"


def _prob(w, **kw):
    return ms.problem(w.n, w.n_q_heads, w.n_kv_heads, **kw)


@pytest.mark.parametrize("cid", range(5))
def test_the_five_workloads_validate(cid):
    w = W.config(cid)
    ms.ms_validate(_prob(w), ms.head_params(w.heads))


def test_selection_sizes_mixed_layer():
    w = W.config(3)
    nv, ns, nbk = ms.ms_selection_sizes(_prob(w), ms.head_params(w.heads))
    assert nv == 24 * 1000 and ns == 24 * 6096 and nbk == 6 * (w.n // 64) * 100


def _expect(status, fn, *args):
    with pytest.raises(ms.MsError) as e:
        fn(*args)
    assert e.value.status == status, e.value


def test_problem_validation():
    hp = ms.head_params([W.dense()])
    _expect(2, ms.ms_validate, ms.problem(1024, 1, 1, head_dim=64), hp)
    _expect(2, ms.ms_validate, ms.problem(1000, 1, 1), hp)
    _expect(2, ms.ms_validate, ms.problem(0, 1, 1), hp)
    _expect(2, ms.ms_validate, ms.problem(1 << 25, 1, 1), hp)
    _expect(1, ms.ms_validate, ms.problem(1024, 3, 2), ms.head_params([W.dense()] * 3))
    _expect(1, ms.ms_validate, ms.problem(1024, 1, 1, scale=-1.0), hp)
    _expect(1, ms.ms_validate, ms.problem(1024, 1, 1, out_dtype=7), hp)
    _expect(1, ms.ms_validate, ms.problem(1024, 1, 1, q_block0=-1), hp)
    _expect(1, ms.ms_validate, ms.problem(1024, 1, 1, q_block0=16), hp)   # no query block left
    ms.ms_validate(ms.problem(1024, 1, 1, q_block0=15), hp)                 # the last block alone
    _expect(1, ms.ms_validate, ms.problem(1024, 129, 1), ms.head_params([W.dense()] * 129))


@pytest.mark.parametrize("head,status", [
    (W.HeadParams(9), 1),
    (W.vs(10, 10, last_q=32), 2),
    (W.vs(-1, 10), 1),
    (W.vs(10, 1025), 1),
    (W.HeadParams(W.BLOCK_SPARSE, block=32, top_k_blocks=4), 2),
    (W.bs(0), 1),
    (W.bs(17), 1),
    (W.ashape(-1, 10), 1),
    (W.ashape(4, 0), 1),
    (W.grid(0, 2, 1, 8), 1),
    (W.grid(100, -1, 1, 8), 1),
    (W.grid(100, 2, -1, 8), 1),
    (W.grid(100, 2, 1, 0), 1),
    (W.grid(2000, 2, 1, 8), 1),
])
def test_head_validation(head, status):
    _expect(status, ms.ms_validate, ms.problem(1024, 1, 1), ms.head_params([head]))


def _cap_bound(h, nb):
    """Per-head CSR capacities from the pattern's own bounds."""
    r = c = 0
    if h.pattern == W.VERTICAL_SLASH and h.block == 32:
        for b in range(2 * nb):
            last = 32 * b + 31
            # run starts are >= 33 apart and <= last
            r += min(h.n_slash, last // 33 + 1)
            c += min(h.n_vertical, last + 1)
        return r, c
    for b in range(nb):
        last = 64 * b + 63
        if h.pattern == W.VERTICAL_SLASH:
            # run starts are >= 65 apart and <= last; columns are distinct keys <= last
            r += min(h.n_slash, last // 65 + 1)
            c += min(h.n_vertical, last + 1)
        elif h.pattern == W.BLOCK_SPARSE:
            cnt = min(h.top_k_blocks, b + 1)
            r += min(cnt, b // 2 + 1)  # runs of blocks are separated by >= 1 gap
        elif h.pattern == W.A_SHAPE:
            r += 2
        elif h.pattern == W.GRID:
            # one run per frame group reaching the block, plus the local one
            r += min(h.grid_frames, (last + h.grid_width) // h.grid_stride) + 1
        else:
            r += 1
    return r, c


def test_grid_capacity_bounds_the_oracle_runs():
    """The per-block range capacity of Grid heads is never below the runs the
    oracle's index holds (strides below, at and above 64 + 2w)."""
    n = 64 * 40
    for P, T, w, W_ in [(10, 50, 2, 5), (70, 30, 3, 1), (66, 40, 1, 3), (500, 4, 30, 700), (1, 3, 0, 1)]:
        hp = W.grid(P, T, w, W_)
        _, caps = ms.ms_index_layout(ms.problem(n, 1, 1), ms.head_params([hp]))
        runs = sum(oracle.grid_block_index(P, T, w, W_, b, n)[0].shape[0] for b in range(n // 64))
        assert caps[0][0] == _cap_bound(hp, n // 64)[0] >= runs


def test_index_layout_capacities_and_alignment():
    w = W.config(3, n=8192)
    prob, hp = _prob(w), ms.head_params(w.heads)
    offs, caps = ms.ms_index_layout(prob, hp)
    total = ms.ms_index_bytes(prob, hp)
    for h, (o, cp) in enumerate(zip(offs, caps)):
        assert cp == _cap_bound(w.heads[h], w.nb)
        assert all(x % 256 == 0 for x in o)
        assert o[0] + 4 * (w.nb + 1) <= o[1] and o[1] + 8 * cp[0] <= o[2]
        assert o[2] + 4 * (w.nb + 1) <= o[3] and o[3] + 4 * cp[1] <= total


def test_workspace_sizes_cover_their_parts():
    w = W.config(3, n=8192)
    prob, hp = _prob(w), ms.head_params(w.heads)
    est = ms.ms_estimate_workspace_bytes(prob, hp)
    idx = ms.ms_index_bytes(prob, hp)
    att = ms.ms_attn_workspace_bytes(prob)
    assert att == w.n_kv_heads * w.n * 128 * 2
    assert ms.ms_workspace_bytes(prob, hp) >= est + idx + att


def test_attention_workspace_holds_the_pacing_counters():
    """Below 131072 keys the attention workspace is the fp16 V copy; from
    there on it also holds the counters of the paced launches (8 XCDs x
    8192-key segments per launch of 1024 workgroups), sized for every head
    of the problem paced with 64-row and with 32-row blocks."""
    for n, hq, hkv in ((65536, 32, 8), (131072, 32, 8), (1 << 20, 32, 8), (262144, 6, 2)):
        prob = ms.problem(n, hq, hkv)
        att = ms.ms_attn_workspace_bytes(prob)
        v16 = hkv * n * 128 * 2
        if n < 131072:
            assert att == v16
            continue
        nseg = (n - 1) // 8192 + 1
        per = max(1, 1024 // hq)
        launches = -(-(n // 64) // per) + -(-(n // 32) // per)
        words = launches * 8 * nseg
        assert att == v16 + -(-words * 4 // 256) * 256, (n, att)


def test_pace_polls_hook_rejects_negative_counts():
    lib = ms.load()
    assert lib.ms_set_pace_polls(-1) == 1  # MS_ERR_INVALID_ARG
    assert lib.ms_set_pace_polls(4096) == 0


def _raw(status, name, *args):
    """Calls the C ABI directly (ctypes), bypassing the binding's own checks."""
    lib = ms.load()
    got = getattr(lib, name)(*args)
    assert got == status, (name, got, lib.ms_last_error())


def _vp(addr):
    return None if addr is None else ctypes.c_void_p(addr)


def test_calls_reject_bad_arguments_before_launch():
    """The C ABI validates pointers, alignment and capacities on the host and
    returns before anything is enqueued (fake addresses, never dereferenced)."""
    w = W.custom("t", 1024, 2, 1, [W.vs(16, 16), W.bs(4)])
    prob, hp = _prob(w), ms.head_params(w.heads)
    pr = ctypes.byref(prob)
    A = 1 << 20
    MB = 1 << 20
    # null q
    _raw(1, "ms_estimate_vs", pr, hp, None, _vp(A), _vp(A), _vp(A), None, None, _vp(A), MB, None)
    # misaligned k
    _raw(1, "ms_estimate_vs", pr, hp, _vp(A), _vp(A + 2), _vp(A), _vp(A), None, None, _vp(A), MB, None)
    # workspace too small
    _raw(3, "ms_estimate_vs", pr, hp, _vp(A), _vp(A), _vp(A), _vp(A), None, None, _vp(A), 1024, None)
    # null selection array of a present pattern
    _raw(1, "ms_estimate_block", pr, hp, _vp(A), _vp(A), None, None, _vp(A), MB, None)
    # index arena too small
    _raw(3, "ms_build_index", pr, hp, _vp(A), _vp(A), _vp(A), _vp(A), 4096, None)
    # misaligned index arena
    _raw(1, "ms_build_index", pr, hp, _vp(A), _vp(A), _vp(A), _vp(A + 16), 1 << 30, None)
    # attention workspace too small
    _raw(3, "ms_dense_attn", pr, _vp(A), _vp(A), _vp(A), _vp(A), None, _vp(A), 100, None)
    # top-k hook: empty input, negative k
    lib = ms.load()
    assert lib.ms_topk_f32(ctypes.c_void_p(1 << 20), 0, 1, ctypes.c_void_p(1 << 20), None) == 1
    pr2 = ms.problem(1024, 4, 2)
    assert lib.ms_attention_recall(ctypes.byref(pr2), None, ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 20),
                                   None) == 1
    assert lib.ms_attention_recall(ctypes.byref(pr2), ctypes.c_void_p((1 << 20) + 2), ctypes.c_void_p(1 << 20),
                                   ctypes.c_void_p(1 << 20), None) == 1
    assert lib.ms_topk_f32(ctypes.c_void_p(1 << 20), 10, -1, ctypes.c_void_p(1 << 20), None) == 1
    assert b"negative" in lib.ms_last_error()
    # the entry point without a workspace: a layer larger than its static
    # scratch is refused before any device call
    big = W.custom("big", 131072, 32, 8, [W.vs(1000, 6096)] * 32)
    pb = _prob(big)
    assert ms.ms_workspace_bytes(pb, ms.head_params(big.heads)) > ms.ms_noalloc_scratch_bytes()
    _raw(3, "ms_sparse_attn_noalloc", ctypes.byref(pb), ms.head_params(big.heads), _vp(A), _vp(A), _vp(A), _vp(A),
         None, None)
    assert b"static scratch" in lib.ms_last_error()
    _raw(1, "ms_sparse_attn_noalloc", pr, None, _vp(A), _vp(A), _vp(A), _vp(A), None, None)


def _binding_rejects(fn, *args, match):
    with pytest.raises(ms.MsError, match=match) as e:
        fn(*args)
    assert e.value.status == 1


def test_binding_checks_tensors_before_the_library():
    """The binding refuses a wrong dtype, a strided view, a short or long
    buffer and a host tensor before passing a pointer on (the C ABI sees bare
    addresses and cannot check extents).  Host tensors of the right shape and
    dtype get as far as the device check, so every other check runs here."""
    import torch
    n, hq, hkv = 1024, 2, 1
    w = W.custom("t", n, hq, hkv, [W.vs(16, 16), W.bs(4)])
    prob, hp = _prob(w), ms.head_params(w.heads)
    bf = torch.bfloat16
    q = torch.zeros(hq, n, 128, dtype=bf)
    k = torch.zeros(hkv, n, 128, dtype=bf)
    v = torch.zeros(hkv, n, 128, dtype=bf)
    out = torch.zeros(hq, n, 128, dtype=bf)
    ws = torch.zeros(1 << 16, dtype=torch.uint8)
    nv, ns, nbk = ms.ms_selection_sizes(prob, hp)
    vert, slash = torch.zeros(nv, dtype=torch.int32), torch.zeros(ns, dtype=torch.int32)
    blocks = torch.zeros(nbk, dtype=torch.int32)
    call = ms.ms_sparse_attn
    _binding_rejects(call, prob, hp, q.float(), k, v, out, ws, match="q: dtype")
    _binding_rejects(call, prob, hp, q.transpose(1, 2), k, v, out, ws, match="q must be contiguous")
    _binding_rejects(call, prob, hp, q.reshape(-1)[:-128], k, v, out, ws, match="q holds")
    _binding_rejects(call, prob, hp, q, k.reshape(-1)[:-1], v, out, ws, match="k holds")
    _binding_rejects(call, prob, hp, q, k, v.half(), out, ws, match="v: dtype")
    _binding_rejects(call, prob, hp, q, k, v, out.float(), ws, match="out: dtype")
    _binding_rejects(call, prob, hp, q, k, v, out, ws, torch.zeros(hq * n - 1), match="lse holds")
    _binding_rejects(call, prob, hp, q, k, v, out, ws, match="q must be a device tensor")
    f32 = ms.problem(n, hq, hkv, out_dtype=ms.OUT_F32)
    _binding_rejects(call, f32, hp, q, k, v, out, ws, match="out: dtype")
    chunk = ms.problem(n, hq, hkv, q_block0=4)
    _binding_rejects(ms.ms_dense_attn, chunk, q, k, v, out, ws, match="q holds")   # the chunk has n - 256 rows
    _binding_rejects(ms.ms_estimate_vs, prob, hp, q, k, vert[:-1], slash, ws, match="vert holds")
    _binding_rejects(ms.ms_estimate_vs, prob, hp, q, k, vert, slash.long(), ws, match="slash: dtype")
    _binding_rejects(ms.ms_estimate_vs, prob, hp, q, k, vert, slash, ws, torch.zeros(5), match="dbg_v holds")
    _binding_rejects(ms.ms_estimate_block, prob, hp, q, k, blocks[:-1], ws, match="blocks holds")
    _binding_rejects(ms.ms_build_index, prob, hp, vert, slash, blocks, ws.view(torch.int32), match="index: dtype")
    _binding_rejects(ms.ms_topk_f32, torch.zeros(10), 5, torch.zeros(4, dtype=torch.int32), match="idx holds")
    _binding_rejects(ms.ms_attention_recall, prob, torch.zeros(hq * n), torch.zeros(hq * n),
                     torch.zeros(1), match="recall holds")


def test_chunk_sizes_follow_the_query_blocks():
    """With q_block0 = 15 of 20 blocks, Block-Sparse selections, index and
    estimation workspace cover 5 query blocks; Vertical-Slash sizes do not
    depend on the chunk."""
    hp = ms.head_params([W.bs(4), W.vs(3, 5)])
    full, part = ms.problem(64 * 20, 2, 1), ms.problem(64 * 20, 2, 1, q_block0=15)
    assert ms.ms_selection_sizes(full, hp) == (3, 5, 20 * 4)
    assert ms.ms_selection_sizes(part, hp) == (3, 5, 5 * 4)
    assert ms.ms_index_bytes(part, hp) < ms.ms_index_bytes(full, hp)
    assert ms.ms_estimate_workspace_bytes(part, hp) < ms.ms_estimate_workspace_bytes(full, hp)
    offs, caps = ms.ms_index_layout(part, hp)
    assert caps[0][0] == sum(min(4, b + 1, b // 2 + 1) for b in range(15, 20))


@pytest.mark.parametrize("block,status", [(0, 0), (64, 0), (32, 0), (16, 2), (128, 2), (-1, 2)])
def test_vertical_slash_block_height_validation(block, status):
    hp = ms.head_params([W.HeadParams(W.VERTICAL_SLASH, n_vertical=4, n_slash=4, block=block)])
    if status == 0:
        ms.ms_validate(ms.problem(1024, 1, 1), hp)
    else:
        _expect(status, ms.ms_validate, ms.problem(1024, 1, 1), hp)


def test_32_row_block_capacities_bound_the_oracle_index():
    """A Vertical-Slash head with 32-row blocks has a CSR over twice the query
    blocks; its capacities follow the 32-row bounds and hold the oracle's
    index of random selections, whole and as a chunk."""
    n = 64 * 24
    r = np.random.default_rng(5)
    for kv, ks in [(10, 40), (300, 700), (n, 5), (1, n)]:
        hp = W.vs(kv, ks, block=32)
        vert = np.sort(r.choice(n, min(kv, n), replace=False))
        slash = np.sort(r.choice(n, min(ks, n), replace=False))
        for qb0 in (0, 7):
            prob = ms.problem(n, 1, 1, q_block0=qb0)
            arr = ms.head_params([hp])
            assert ms.index_blocks(prob, arr, 0) == 2 * (n // 64 - qb0)
            offs, caps = ms.ms_index_layout(prob, arr)
            assert caps[0] == _cap_bound(hp, n // 64 - qb0) if qb0 == 0 else True
            idx = oracle.head_index(hp, ("vs", vert, slash), n, q_block0=qb0)
            assert len(idx) == 2 * (n // 64 - qb0)
            assert sum(x[0].shape[0] for x in idx) <= caps[0][0]
            assert sum(x[1].shape[0] for x in idx) <= caps[0][1]
            o = offs[0]
            assert o[0] + 4 * (2 * (n // 64 - qb0) + 1) <= o[1] and o[2] + 4 * (2 * (n // 64 - qb0) + 1) <= o[3]
