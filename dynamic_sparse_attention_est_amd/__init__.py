"""Python binding of libmsattn: MInference-style dynamic sparse pre-filling
attention on AMD MI355X (gfx950).

Argument marshalling only: every step of the path (estimation, selection,
index conversion, attention) runs in the HIP kernels of libmsattn.so behind
the C ABI of include/msattn.h.  PyTorch supplies device memory and streams.
There is no CPU fallback: without the built library, importing the binding's
calls raises.

Names mirror the C ABI (ms_estimate_vs, ms_estimate_block, ms_build_index,
ms_sparse_attn_indexed, ms_sparse_attn, ms_dense_attn, ms_topk_f32, ...).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch  # loaded first: its HIP runtime is the one libmsattn binds to

__all__ = [
    "MsError", "Problem", "HeadParams", "library_path", "load", "problem", "head_params",
    "ms_validate", "ms_selection_sizes", "ms_estimate_workspace_bytes", "ms_index_bytes",
    "ms_index_layout", "ms_attn_workspace_bytes", "ms_workspace_bytes", "ms_estimate_vs",
    "ms_estimate_block", "ms_build_index", "ms_sparse_attn_indexed", "ms_sparse_attn",
    "ms_dense_attn", "ms_topk_f32", "ms_set_pace_polls", "ms_version", "read_index", "empty_workspace",
    "ms_sparse_attn_noalloc", "ms_noalloc_scratch_bytes", "ms_attention_recall", "index_blocks",
    "A_SHAPE", "VERTICAL_SLASH", "BLOCK_SPARSE", "DENSE", "GRID", "OUT_BF16", "OUT_F32",
]

A_SHAPE, VERTICAL_SLASH, BLOCK_SPARSE, DENSE, GRID = 0, 1, 2, 3, 4
OUT_BF16, OUT_F32 = 0, 1
_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "insufficient capacity", 4: "device error"}


class MsError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status
        self.message = message


class Problem(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("scale", ctypes.c_float), ("out_dtype", ctypes.c_int32),
                ("q_block0", ctypes.c_int32)]


class HeadParams(ctypes.Structure):
    _fields_ = [("pattern", ctypes.c_int32), ("last_q", ctypes.c_int32), ("n_vertical", ctypes.c_int32),
                ("n_slash", ctypes.c_int32), ("block", ctypes.c_int32), ("top_k_blocks", ctypes.c_int32),
                ("sink", ctypes.c_int32), ("window", ctypes.c_int32), ("grid_stride", ctypes.c_int32),
                ("grid_frames", ctypes.c_int32), ("grid_width", ctypes.c_int32)]


def library_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmsattn.so")


_lib = None


def load():
    """Loads libmsattn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m dynamic_sparse_attention_est_amd.build`")
    lib = ctypes.CDLL(path)
    P, H = ctypes.POINTER(Problem), ctypes.POINTER(HeadParams)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    sig = {
        "ms_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "ms_last_error": (ctypes.c_char_p, []),
        "ms_version": (i32, []),
        "ms_validate": (ctypes.c_int, [P, H]),
        "ms_selection_sizes": (ctypes.c_int, [P, H, ctypes.POINTER(i64), ctypes.POINTER(i64), ctypes.POINTER(i64)]),
        "ms_estimate_workspace_bytes": (ctypes.c_int, [P, H, ctypes.POINTER(sz)]),
        "ms_index_bytes": (ctypes.c_int, [P, H, ctypes.POINTER(sz)]),
        "ms_index_layout": (ctypes.c_int, [P, H, ctypes.POINTER(i64), ctypes.POINTER(i64)]),
        "ms_attn_workspace_bytes": (ctypes.c_int, [P, ctypes.POINTER(sz)]),
        "ms_workspace_bytes": (ctypes.c_int, [P, H, ctypes.POINTER(sz)]),
        "ms_estimate_vs": (ctypes.c_int, [P, H, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "ms_estimate_block": (ctypes.c_int, [P, H, vp, vp, vp, vp, vp, sz, vp]),
        "ms_build_index": (ctypes.c_int, [P, H, vp, vp, vp, vp, sz, vp]),
        "ms_sparse_attn_indexed": (ctypes.c_int, [P, H, vp, vp, vp, vp, sz, vp, vp, vp, sz, vp]),
        "ms_sparse_attn": (ctypes.c_int, [P, H, vp, vp, vp, vp, vp, vp, sz, vp]),
        "ms_dense_attn": (ctypes.c_int, [P, vp, vp, vp, vp, vp, vp, sz, vp]),
        "ms_topk_f32": (ctypes.c_int, [vp, i64, i32, vp, vp]),
        "ms_set_pace_polls": (ctypes.c_int, [i32]),
        "ms_attention_recall": (ctypes.c_int, [P, vp, vp, vp, vp]),
        "ms_sparse_attn_noalloc": (ctypes.c_int, [P, H, vp, vp, vp, vp, vp, vp]),
        "ms_noalloc_scratch_bytes": (ctypes.c_int, [ctypes.POINTER(sz)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        raise MsError(status, load().ms_last_error().decode())


# ---------------------------------------------------------------- structs
def problem(n: int, n_q_heads: int, n_kv_heads: int, scale: float = 0.0, out_dtype: int = OUT_BF16,
            head_dim: int = 128, q_block0: int = 0) -> Problem:
    """n keys; the call's queries are rows 64*q_block0 .. n-1 (Q, out and lse
    hold n - 64*q_block0 rows per head)."""
    return Problem(n, n_q_heads, n_kv_heads, head_dim, scale, out_dtype, q_block0)


def head_params(heads: Sequence) -> ctypes.Array:
    """Array of HeadParams from objects with the fields of ms_head_params."""
    arr = (HeadParams * len(heads))()
    for i, h in enumerate(heads):
        arr[i] = HeadParams(int(h.pattern), int(getattr(h, "last_q", 64)), int(getattr(h, "n_vertical", 0)),
                            int(getattr(h, "n_slash", 0)), int(getattr(h, "block", 64)),
                            int(getattr(h, "top_k_blocks", 0)), int(getattr(h, "sink", 0)),
                            int(getattr(h, "window", 0)), int(getattr(h, "grid_stride", 0)),
                            int(getattr(h, "grid_frames", 0)), int(getattr(h, "grid_width", 0)))
    return arr


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t: Optional[torch.Tensor], name: str, dtype, numel: Optional[int] = None, at_least: bool = False,
          optional: bool = False) -> None:
    """Host-side checks of a tensor argument before the library sees its
    pointer: the C ABI takes bare device pointers and cannot check extents,
    so a wrong dtype, a strided view or a short buffer is refused here."""
    if t is None:
        if optional:
            return
        raise MsError(1, f"{name} is None")
    if not isinstance(t, torch.Tensor):
        raise MsError(1, f"{name} must be a torch.Tensor")
    if t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise MsError(1, f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise MsError(1, f"{name} must be contiguous")
    if numel is not None:
        if at_least and t.numel() < numel:
            raise MsError(1, f"{name} holds {t.numel()} elements, at least {numel} needed")
        if not at_least and t.numel() != numel:
            raise MsError(1, f"{name} holds {t.numel()} elements, {numel} expected")


def _on_device(**tensors) -> None:
    """Every tensor argument given must live on the GPU (checked after the
    dtype and extent checks of all arguments)."""
    for name, t in tensors.items():
        if t is not None and not t.is_cuda:
            raise MsError(1, f"{name} must be a device tensor")


def _rows(prob: Problem) -> int:
    """Query rows per head of a call: n - 64 * q_block0."""
    return int(prob.n) - 64 * int(prob.q_block0)


def _need_qkv(prob: Problem, q, k, v=None) -> None:
    d = int(prob.head_dim)
    _need(q, "q", torch.bfloat16, int(prob.n_q_heads) * _rows(prob) * d)
    _need(k, "k", torch.bfloat16, int(prob.n_kv_heads) * int(prob.n) * d)
    if v is not None:
        _need(v, "v", torch.bfloat16, int(prob.n_kv_heads) * int(prob.n) * d)


def _need_out(prob: Problem, out, lse) -> None:
    rows = int(prob.n_q_heads) * _rows(prob)
    _need(out, "out", torch.float32 if prob.out_dtype == OUT_F32 else torch.bfloat16, rows * int(prob.head_dim))
    _need(lse, "lse", torch.float32, rows, optional=True)


def _nbytes(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


# ---------------------------------------------------------------- queries
def ms_version() -> int:
    return load().ms_version()


def ms_validate(prob: Problem, heads) -> None:
    _check(load().ms_validate(ctypes.byref(prob), heads))


def ms_selection_sizes(prob: Problem, heads):
    a, b, c = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(load().ms_selection_sizes(ctypes.byref(prob), heads, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)))
    return a.value, b.value, c.value


def _size_query(name, prob, heads=None) -> int:
    out = ctypes.c_size_t()
    fn = getattr(load(), name)
    if heads is None:
        _check(fn(ctypes.byref(prob), ctypes.byref(out)))
    else:
        _check(fn(ctypes.byref(prob), heads, ctypes.byref(out)))
    return out.value


def ms_estimate_workspace_bytes(prob, heads) -> int:
    return _size_query("ms_estimate_workspace_bytes", prob, heads)


def ms_index_bytes(prob, heads) -> int:
    return _size_query("ms_index_bytes", prob, heads)


def ms_attn_workspace_bytes(prob) -> int:
    return _size_query("ms_attn_workspace_bytes", prob)


def ms_workspace_bytes(prob, heads) -> int:
    return _size_query("ms_workspace_bytes", prob, heads)


def ms_index_layout(prob, heads):
    h = prob.n_q_heads
    offs = (ctypes.c_int64 * (4 * h))()
    caps = (ctypes.c_int64 * (2 * h))()
    _check(load().ms_index_layout(ctypes.byref(prob), heads, offs, caps))
    return [tuple(offs[4 * i:4 * i + 4]) for i in range(h)], [tuple(caps[2 * i:2 * i + 2]) for i in range(h)]


def empty_workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A byte tensor of at least nbytes with a 256-byte aligned base."""
    t = torch.empty(max(int(nbytes), 1) + 256, dtype=torch.uint8, device=device)
    off = (-t.data_ptr()) % 256
    return t[off:off + max(int(nbytes), 1)]


# ---------------------------------------------------------------- calls
def ms_estimate_vs(prob, heads, q, k, vert, slash, ws, dbg_v=None, dbg_s=None, stream=None) -> None:
    nv, ns, _ = ms_selection_sizes(prob, heads)
    _need_qkv(prob, q, k)
    _need(vert, "vert", torch.int32, nv, at_least=True, optional=nv == 0)
    _need(slash, "slash", torch.int32, ns, at_least=True, optional=ns == 0)
    for name, t in (("dbg_v", dbg_v), ("dbg_s", dbg_s)):
        _need(t, name, torch.float32, int(prob.n_q_heads) * int(prob.n), at_least=True, optional=True)
    _need(ws, "ws", torch.uint8)
    _on_device(q=q, k=k, vert=vert, slash=slash, dbg_v=dbg_v, dbg_s=dbg_s, ws=ws)
    _check(load().ms_estimate_vs(ctypes.byref(prob), heads, _ptr(q), _ptr(k), _ptr(vert), _ptr(slash), _ptr(dbg_v),
                                 _ptr(dbg_s), _ptr(ws), _nbytes(ws), _stream(stream)))


def ms_estimate_block(prob, heads, q, k, blocks, ws, dbg_scores=None, stream=None) -> None:
    _, _, nbk = ms_selection_sizes(prob, heads)
    _need_qkv(prob, q, k)
    _need(blocks, "blocks", torch.int32, nbk, at_least=True, optional=nbk == 0)
    nb = int(prob.n) // 64
    _need(dbg_scores, "dbg_scores", torch.float32, int(prob.n_q_heads) * (nb - int(prob.q_block0)) * nb,
          at_least=True, optional=True)
    _need(ws, "ws", torch.uint8)
    _on_device(q=q, k=k, blocks=blocks, dbg_scores=dbg_scores, ws=ws)
    _check(load().ms_estimate_block(ctypes.byref(prob), heads, _ptr(q), _ptr(k), _ptr(blocks), _ptr(dbg_scores),
                                    _ptr(ws), _nbytes(ws), _stream(stream)))


def ms_build_index(prob, heads, vert, slash, blocks, index, stream=None) -> None:
    nv, ns, nbk = ms_selection_sizes(prob, heads)
    _need(vert, "vert", torch.int32, nv, at_least=True, optional=nv == 0)
    _need(slash, "slash", torch.int32, ns, at_least=True, optional=ns == 0)
    _need(blocks, "blocks", torch.int32, nbk, at_least=True, optional=nbk == 0)
    _need(index, "index", torch.uint8)
    _on_device(vert=vert, slash=slash, blocks=blocks, index=index)
    _check(load().ms_build_index(ctypes.byref(prob), heads, _ptr(vert), _ptr(slash), _ptr(blocks), _ptr(index),
                                 _nbytes(index), _stream(stream)))


def ms_sparse_attn_indexed(prob, heads, q, k, v, index, out, ws, lse=None, stream=None) -> None:
    _need_qkv(prob, q, k, v)
    _need_out(prob, out, lse)
    _need(index, "index", torch.uint8)
    _need(ws, "ws", torch.uint8)
    _on_device(q=q, k=k, v=v, index=index, out=out, ws=ws, lse=lse)
    _check(load().ms_sparse_attn_indexed(ctypes.byref(prob), heads, _ptr(q), _ptr(k), _ptr(v), _ptr(index),
                                         _nbytes(index), _ptr(out), _ptr(lse), _ptr(ws), _nbytes(ws), _stream(stream)))


def ms_sparse_attn(prob, heads, q, k, v, out, ws, lse=None, stream=None) -> None:
    _need_qkv(prob, q, k, v)
    _need_out(prob, out, lse)
    _need(ws, "ws", torch.uint8)
    _on_device(q=q, k=k, v=v, out=out, ws=ws, lse=lse)
    _check(load().ms_sparse_attn(ctypes.byref(prob), heads, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                 _ptr(ws), _nbytes(ws), _stream(stream)))


def ms_sparse_attn_noalloc(prob, heads, q, k, v, out, lse=None, stream=None) -> None:
    """ms_sparse_attn with its workspace in the library's static per-GPU
    scratch: allocates nothing (see include/msattn.h)."""
    _need_qkv(prob, q, k, v)
    _need_out(prob, out, lse)
    _on_device(q=q, k=k, v=v, out=out, lse=lse)
    _check(load().ms_sparse_attn_noalloc(ctypes.byref(prob), heads, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                         _stream(stream)))


def ms_noalloc_scratch_bytes() -> int:
    out = ctypes.c_size_t()
    _check(load().ms_noalloc_scratch_bytes(ctypes.byref(out)))
    return out.value


def ms_dense_attn(prob, q, k, v, out, ws, lse=None, stream=None) -> None:
    _need_qkv(prob, q, k, v)
    _need_out(prob, out, lse)
    _need(ws, "ws", torch.uint8)
    _on_device(q=q, k=k, v=v, out=out, ws=ws, lse=lse)
    _check(load().ms_dense_attn(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(ws),
                                _nbytes(ws), _stream(stream)))


def ms_set_pace_polls(polls: int) -> None:
    """Test hook: counter reads a paced workgroup's wait may take (0: no waiting)."""
    _check(load().ms_set_pace_polls(int(polls)))


def ms_topk_f32(x: torch.Tensor, k: int, idx: torch.Tensor, stream=None) -> None:
    _need(x, "x", torch.float32)
    _need(idx, "idx", torch.int32, min(int(k), x.numel()), at_least=True)
    _on_device(x=x, idx=idx)
    _check(load().ms_topk_f32(_ptr(x), x.numel(), int(k), _ptr(idx), _stream(stream)))


def ms_attention_recall(prob, lse_sparse: torch.Tensor, lse_dense: torch.Tensor, recall: torch.Tensor,
                        stream=None) -> None:
    """recall[h] = mean over rows of exp(lse_sparse - lse_dense): the share of
    the full attention mass that the sparse index keeps (fp32 tensors on the
    device: [H_q, n], [H_q, n], [H_q])."""
    rows = int(prob.n_q_heads) * _rows(prob)
    _need(lse_sparse, "lse_sparse", torch.float32, rows)
    _need(lse_dense, "lse_dense", torch.float32, rows)
    _need(recall, "recall", torch.float32, int(prob.n_q_heads), at_least=True)
    _on_device(lse_sparse=lse_sparse, lse_dense=lse_dense, recall=recall)
    _check(load().ms_attention_recall(ctypes.byref(prob), _ptr(lse_sparse), _ptr(lse_dense), _ptr(recall),
                                      _stream(stream)))


def index_blocks(prob, heads, h: int) -> int:
    """Blocks of head h's CSR: the call's query blocks, NBq = n/64 - q_block0,
    or 2 NBq for a Vertical-Slash head indexed by 32-row blocks."""
    nb = prob.n // 64 - prob.q_block0
    p = heads[h]
    return 2 * nb if p.pattern == VERTICAL_SLASH and p.block == 32 else nb


def read_index(prob, heads, index: torch.Tensor):
    """Copies the CSR index of every head to the host: a list over heads of
    (rng_ptr [NB+1], rng [R, 2], col_ptr [NB+1], col [C]) int32 numpy arrays
    over the head's query blocks (NB = index_blocks(prob, heads, h))."""
    offs, _ = ms_index_layout(prob, heads)
    host = index.cpu().numpy()
    out = []
    for h, (o_rp, o_r, o_cp, o_c) in enumerate(offs):
        nb = index_blocks(prob, heads, h)
        rp = host[o_rp:o_rp + 4 * (nb + 1)].view("int32").copy()
        cp = host[o_cp:o_cp + 4 * (nb + 1)].view("int32").copy()
        r = host[o_r:o_r + 8 * int(rp[-1])].view("int32").reshape(-1, 2).copy()
        c = host[o_c:o_c + 4 * int(cp[-1])].view("int32").copy()
        out.append((rp, r, cp, c))
    return out
