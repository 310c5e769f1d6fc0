"""The C ABI library on a machine without a GPU: it loads, exports every
symbol include/msattn.h declares, and rejects bad arguments on the host
before enqueueing anything (no call here reaches a HIP launch)."""
import ctypes
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


class _Fake:
    """Stands in for a tensor: an address the library never dereferences here."""

    def __init__(self, addr, nbytes=1 << 20):
        self.addr, self.nb = addr, nbytes

    def data_ptr(self):
        return self.addr

    def numel(self):
        return self.nb

    def element_size(self):
        return 1


class _Stream:
    cuda_stream = 0


def test_calls_reject_bad_arguments_before_launch():
    w = W.custom("t", 1024, 2, 1, [W.vs(16, 16), W.bs(4)])
    prob, hp = _prob(w), ms.head_params(w.heads)
    A = _Fake(1 << 20)
    st = _Stream()
    # null q
    _expect(1, ms.ms_estimate_vs, prob, hp, None, A, A, A, A, None, None, st)
    # misaligned k
    _expect(1, ms.ms_estimate_vs, prob, hp, A, _Fake((1 << 20) + 2), A, A, A, None, None, st)
    # workspace too small
    _expect(3, ms.ms_estimate_vs, prob, hp, A, A, A, A, _Fake(1 << 20, 1024), None, None, st)
    # null selection array of a present pattern
    _expect(1, ms.ms_estimate_block, prob, hp, A, A, None, A, None, st)
    # index arena too small
    _expect(3, ms.ms_build_index, prob, hp, A, A, A, _Fake(1 << 20, 4096), st)
    # misaligned index arena
    _expect(1, ms.ms_build_index, prob, hp, A, A, A, _Fake((1 << 20) + 16, 1 << 30), st)
    # attention workspace too small
    _expect(3, ms.ms_dense_attn, prob, A, A, A, A, _Fake(1 << 20, 100), None, st)
    # top-k hook: empty input, negative k
    lib = ms.load()
    assert lib.ms_topk_f32(ctypes.c_void_p(1 << 20), 0, 1, ctypes.c_void_p(1 << 20), None) == 1
    pr = ms.problem(1024, 4, 2)
    assert lib.ms_attention_recall(ctypes.byref(pr), None, ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 20),
                                   None) == 1
    assert lib.ms_attention_recall(ctypes.byref(pr), ctypes.c_void_p((1 << 20) + 2), ctypes.c_void_p(1 << 20),
                                   ctypes.c_void_p(1 << 20), None) == 1
    assert lib.ms_topk_f32(ctypes.c_void_p(1 << 20), 10, -1, ctypes.c_void_p(1 << 20), None) == 1
    assert b"negative" in lib.ms_last_error()


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
