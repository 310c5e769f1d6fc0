"""Helpers of the GPU parity tests: run the library stage by stage through the
C ABI binding and bring every stage's output to the host for the oracle."""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np
import torch

import dynamic_sparse_attention_est_amd as ms
import oracle
import workloads as W

# Attention bar: max |err| <= 2e-2 and sum|out - bf16(ref)| / sum|bf16(ref)| <= 1e-3.
MAX_ABS = 2e-2
MEAN_REL = 1e-3
# Per-row relative L2 bound (a sharper internal check than the max-abs bar).
ROW_REL_L2 = 5e-3


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def bf16_round(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).float().numpy().astype(np.float64)


def mean_rel(got: np.ndarray, ref: np.ndarray) -> float:
    den = np.abs(ref).sum()
    return float(np.abs(got - ref).sum() / den) if den > 0 else float(np.abs(got).sum())


def check_attention(got: np.ndarray, ref: np.ndarray, what: str, bf16_out: bool = True):
    """got: GPU output rows; ref: float64 oracle rows (same shape)."""
    r = bf16_round(ref) if bf16_out else ref
    err = np.abs(got - r)
    assert np.all(np.isfinite(got)), what
    assert err.max() <= MAX_ABS, f"{what}: max abs err {err.max():.3e}"
    mr = mean_rel(got, r)
    assert mr <= MEAN_REL, f"{what}: mean rel err {mr:.3e}"
    num = np.sqrt((err ** 2).sum(axis=-1))
    den = np.sqrt((r ** 2).sum(axis=-1))
    rows = den > 0
    if rows.any():
        worst = (num[rows] / den[rows]).max()
        assert worst <= ROW_REL_L2, f"{what}: worst row rel L2 {worst:.3e}"
    return float(err.max()), mr


@dataclasses.dataclass
class Staged:
    w: W.Workload
    prob: object
    hp: object
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    vert: Optional[torch.Tensor] = None
    slash: Optional[torch.Tensor] = None
    blocks: Optional[torch.Tensor] = None
    dbg_v: Optional[torch.Tensor] = None
    dbg_s: Optional[torch.Tensor] = None
    dbg_scores: Optional[torch.Tensor] = None
    index: Optional[torch.Tensor] = None
    out: Optional[torch.Tensor] = None
    lse: Optional[torch.Tensor] = None


def make(w: W.Workload, out_dtype: int = ms.OUT_BF16, qkv=None) -> Staged:
    q, k, v = qkv if qkv is not None else W.generate(w, device="cuda")
    prob = ms.problem(w.n, w.n_q_heads, w.n_kv_heads, out_dtype=out_dtype)
    return Staged(w, prob, ms.head_params(w.heads), q.contiguous(), k.contiguous(), v.contiguous())


def run_staged(st: Staged, debug: bool = True, lse: bool = True) -> Staged:
    w = st.w
    nv, ns, nbk = ms.ms_selection_sizes(st.prob, st.hp)
    dev = "cuda"
    st.vert = torch.full((max(nv, 1),), -7, dtype=torch.int32, device=dev)
    st.slash = torch.full((max(ns, 1),), -7, dtype=torch.int32, device=dev)
    st.blocks = torch.full((max(nbk, 1),), -7, dtype=torch.int32, device=dev)
    ws = ms.empty_workspace(ms.ms_estimate_workspace_bytes(st.prob, st.hp))
    if debug:
        st.dbg_v = torch.full((w.n_q_heads, w.n), float("nan"), device=dev)
        st.dbg_s = torch.full((w.n_q_heads, w.n), float("nan"), device=dev)
        if any(h.pattern == W.BLOCK_SPARSE for h in w.heads):
            st.dbg_scores = torch.full((w.n_q_heads, w.nb, w.nb), float("nan"), device=dev)
    ms.ms_estimate_vs(st.prob, st.hp, st.q, st.k, st.vert, st.slash, ws, st.dbg_v, st.dbg_s)
    ms.ms_estimate_block(st.prob, st.hp, st.q, st.k, st.blocks, ws, st.dbg_scores)
    st.index = ms.empty_workspace(ms.ms_index_bytes(st.prob, st.hp))
    ms.ms_build_index(st.prob, st.hp, st.vert, st.slash, st.blocks, st.index)
    st.out = torch.empty(st.q.shape, dtype=torch.float32 if st.prob.out_dtype == ms.OUT_F32 else torch.bfloat16,
                         device=dev)
    st.lse = torch.empty((w.n_q_heads, w.n), dtype=torch.float32, device=dev) if lse else None
    aws = ms.empty_workspace(ms.ms_attn_workspace_bytes(st.prob))
    ms.ms_sparse_attn_indexed(st.prob, st.hp, st.q, st.k, st.v, st.index, st.out, aws, st.lse)
    torch.cuda.synchronize()
    return st


def selections(st: Staged):
    """Per head: ('vs', vert, slash) / ('bs', [B_b]) / ('static',) from the GPU outputs."""
    w = st.w
    vert, slash, blocks = st.vert.cpu().numpy(), st.slash.cpu().numpy(), st.blocks.cpu().numpy()
    out = []
    ov = os_ = ob = 0
    for h in w.heads:
        if h.pattern == W.VERTICAL_SLASH:
            out.append(("vs", vert[ov:ov + h.n_vertical].astype(np.int64), slash[os_:os_ + h.n_slash].astype(np.int64)))
            ov += h.n_vertical
            os_ += h.n_slash
        elif h.pattern == W.BLOCK_SPARSE:
            rows = blocks[ob:ob + w.nb * h.top_k_blocks].reshape(w.nb, h.top_k_blocks)
            out.append(("bs", [r[r >= 0].astype(np.int64) for r in rows], rows))
            ob += w.nb * h.top_k_blocks
        else:
            out.append(("static",))
    return out


def oracle_index(w: W.Workload, h: int, sel) -> List:
    hp = w.heads[h]
    return oracle.head_index(hp, sel, w.n)


def kv_of(w: W.Workload, h: int) -> int:
    return h // w.group


def ashape_of(hp):
    return (hp.sink, hp.window) if hp.pattern == W.A_SHAPE else None


def read_index_blocks(prob, hp, index: torch.Tensor, head: int, blocks):
    """CSR entries of some query blocks of one head, copied from the device:
    {b: (ranges [r, 2] int64, cols [c] int64)}."""
    offs, _ = ms.ms_index_layout(prob, hp)
    o_rp, o_r, o_cp, o_c = offs[head]
    nb = ms.index_blocks(prob, hp, head)
    base = index.view(torch.int32)
    rp = base[o_rp // 4:o_rp // 4 + nb + 1].cpu().numpy()
    cp = base[o_cp // 4:o_cp // 4 + nb + 1].cpu().numpy()
    out = {}
    for b in blocks:
        r = base[o_r // 4 + 2 * int(rp[b]):o_r // 4 + 2 * int(rp[b + 1])].cpu().numpy().reshape(-1, 2).astype(np.int64)
        c = base[o_c // 4 + int(cp[b]):o_c // 4 + int(cp[b + 1])].cpu().numpy().astype(np.int64)
        out[b] = (r, c)
    return out


def sample_blocks(nb: int, count: int, seed: int):
    """First, last and random query blocks."""
    rng = np.random.default_rng(seed)
    extra = rng.choice(np.arange(1, nb - 1), size=min(count, nb - 2), replace=False) if nb > 2 else []
    return sorted({0, nb - 1, *[int(x) for x in extra]})
