"""Benchmark: ms per layer of sparse pre-filling attention (estimation + index
conversion + sparse kernel) on one MI355X, and the speedup over the library's
own dense causal kernel on the same GPU.

One step = one ms_sparse_attn call on one layer of synthetic inputs already
resident in HBM.  The headline workload is the 1M-token Vertical-Slash layer
(32 Q / 8 KV heads, d = 128, 1000 verticals + 6096 slashes per head); the
other four workloads (128K mixed 24 VS / 6 BS / 2 A-shape heads, 32K
Block-Sparse, 128K A-shape, 4K Vertical-Slash) and a diagnostic 1M layer with
structured slashes (vs_1m_s) are reported beside it under "side".  Prints ONE
JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload vs_1m|mixed_128k|...]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16/fp16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

# Sources that decide the attention kernels of a call and their launches
# (a recorded traffic figure is reported only while these are unchanged).
ATTN_SOURCES = ("sparse_attn.hip", "group_attn.hip", "api.hip", "internal.h")

WORKLOADS = {"vs_4k": 0, "bs_32k": 1, "ashape_128k": 2, "mixed_128k": 3, "vs_1m": 4, "vs_1m_s": 5, "vs_1m_b32": 6}
# vs_1m_s is a diagnostic beside the five workloads: the 1M layer with a shared
# query mean per KV group, under which the slashes through the planted columns
# win the slash budget (kept fraction ~13% instead of ~31%).  vs_1m_b32 is the
# 1M layer (same inputs) with its heads indexed by 32-row query blocks.


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="vs_1m", choices=sorted(WORKLOADS))
    ap.add_argument("--side", default="mixed_128k,bs_32k,ashape_128k,vs_4k,vs_1m_s,vs_1m_b32",
                    help="comma-separated workloads reported beside the headline ('' = none)")
    ap.add_argument("--side-steps", type=int, default=3, help="at most this many timed steps per side workload")
    ap.add_argument("--dense-steps", type=int, default=1)
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0, help="rough budget of the CPU oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (HBM counter calibration under rocprofv3)")
    return ap.parse_args()


# ---------------------------------------------------------------- kept entries
def _pairs_in_block(lo, hi, row0, torch, rows=64):
    """Causal pairs (i, j), i in [row0, row0+rows), j in [lo, hi), j <= i."""
    L = hi - lo
    x = row0 + 1 - lo

    def G(m):
        m = m.clamp(min=0)
        tri = m * (m + 1) // 2
        over = L * (L + 1) // 2 + (m - L) * L
        return torch.where(m <= L, tri, over)

    return G(x + rows - 1) - G(x - 1)


def kept_entries(ms, prob, hp, heads, index, torch):
    """Exact number of (row, key) pairs the layer attends, summed over heads."""
    offs, _ = ms.ms_index_layout(prob, hp)
    base = index.view(torch.int32)
    total = 0
    for h, (o_rp, o_r, o_cp, o_c) in enumerate(offs):
        nb = ms.index_blocks(prob, hp, h)
        rows = prob.n // nb  # 64, or 32 for a head indexed by 32-row blocks
        rp = base[o_rp // 4:o_rp // 4 + nb + 1].long()
        cp = base[o_cp // 4:o_cp // 4 + nb + 1].long()
        nr, nc = int(rp[-1]), int(cp[-1])
        p = heads[h]
        if p.pattern == 0:  # A-shape: per-row window applied inside the kernel
            i = torch.arange(prob.n, device=index.device, dtype=torch.int64)
            win = torch.minimum(i + 1, torch.full_like(i, p.window))
            sink = (i - p.window + 1).clamp(min=0).clamp(max=p.sink)
            total += int((win + sink).sum())
            continue
        if nr:
            rng = base[o_r // 4:o_r // 4 + 2 * nr].long().view(-1, 2)
            blk = torch.repeat_interleave(torch.arange(nb, device=index.device), rp[1:] - rp[:-1])
            total += int(_pairs_in_block(rng[:, 0], rng[:, 1], blk * rows, torch, rows).sum())
        if nc:
            col = base[o_c // 4:o_c // 4 + nc].long()
            blk = torch.repeat_interleave(torch.arange(nb, device=index.device), cp[1:] - cp[:-1])
            total += int((blk * rows + rows - col).clamp(min=0, max=rows).sum())
    return total


def block_keys(ms, prob, hp, index, torch):
    """Keys each (head, 64-row query block) reads: the sum of its range lengths
    and column counts (the per-head kernel brings each of them into LDS once
    per block; 512 bytes apiece: a bf16 K row and an fp16 V row)."""
    offs, _ = ms.ms_index_layout(prob, hp)
    base = index.view(torch.int32)
    total = cols = 0
    for h, (o_rp, o_r, o_cp, o_c) in enumerate(offs):
        nb = ms.index_blocks(prob, hp, h)
        nr = int(base[o_rp // 4 + nb])
        nc = int(base[o_cp // 4 + nb])
        if nr:
            rng = base[o_r // 4:o_r // 4 + 2 * nr].long().view(-1, 2)
            total += int((rng[:, 1] - rng[:, 0]).clamp(min=0).sum())
        total += nc
        cols += nc
    return total, cols


def gather_stage(ms, torch, W, w, q, k, v, vert, aws, stream):
    """HBM rate of the gathered column loads on a layer of Vertical-Slash
    heads.  The heads are run with their verticals only (the selections the
    estimator just made, no slashes): every key they attend is then a
    gathered column, one bf16 K row and one fp16 V row (512 B) per (query
    block, column), brought in by the column path of the attention kernel.
    The timed call includes the fp16 copy of V the kernel reads."""
    heads = [W.vs(p.n_vertical, 0, block=p.block) for p in w.heads]
    prob, hp = ms.problem(w.n, w.n_q_heads, w.n_kv_heads), ms.head_params(heads)
    index = ms.empty_workspace(ms.ms_index_bytes(prob, hp))
    empty = torch.empty(1, dtype=torch.int32, device="cuda")
    ms.ms_build_index(prob, hp, vert, empty, empty, index)
    out = torch.empty_like(q)
    ms.ms_sparse_attn_indexed(prob, hp, q, k, v, index, out, aws)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    ms.ms_sparse_attn_indexed(prob, hp, q, k, v, index, out, aws)
    e1.record(stream)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1)
    offs, _ = ms.ms_index_layout(prob, hp)
    base = index.view(torch.int32)
    cols = sum(int(base[o[2] // 4 + ms.index_blocks(prob, hp, h)]) for h, o in enumerate(offs))
    del index, out
    return {"ms": t, "col_keys": cols}


def estimate_bytes(w):
    """Algorithmic HBM bytes of the estimation stage: Vertical-Slash reads K of
    each KV head it serves twice (softmax statistics, then scores) plus the last
    64 query rows, and writes and re-reads two fp32 score vectors per head;
    Block-Sparse pools Q of its heads and K of their KV heads once."""
    vs = [h for h, p in enumerate(w.heads) if p.pattern == 1]
    bs = [h for h, p in enumerate(w.heads) if p.pattern == 2]
    row = 128 * 2
    b = 0
    if vs:
        b += 2 * len({h // w.group for h in vs}) * w.n * row + len(vs) * 64 * row + 2 * 2 * len(vs) * w.n * 4
    if bs:
        b += (len(bs) + len({h // w.group for h in bs})) * w.n * row
    return b


def recorded_traffic(workload, srcs):
    """HBM bytes of one attention call on `workload` from the committed
    rocprofv3 counter summary (profiles/traffic_attention_<workload>.md), or
    None when there is none or the sources that decide the attention kernels
    and their launches changed since it was taken."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", f"traffic_attention_{workload}.md")
    if not os.path.exists(path):
        return None, None
    m = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
    if not m:
        return None, None
    rec = json.loads(m.group(1))
    digest = hashlib.sha256(b"".join(open(s, "rb").read() for s in srcs)).hexdigest()
    if rec.get("source_sha256") != digest:
        return None, rec
    return rec["traffic_bytes_per_call"], rec


# ---------------------------------------------------------------- CPU baseline
def cpu_baseline(w, q, k, v, heads, kept_total, budget_s):
    """The float64 oracle, untuned, on a bounded sample of the same layer:
    one head's estimation in full, index conversion and attention on sampled
    query blocks; extrapolated to the layer (estimation x heads of that
    pattern, index x blocks, attention by kept entries)."""
    import numpy as np
    import torch
    import oracle
    import workloads as W

    n, nb = w.n, w.nb
    rng = np.random.default_rng(0)
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    torch.set_num_threads(cores)
    h = next((i for i, p in enumerate(heads) if p.pattern == W.VERTICAL_SLASH), 0)
    p = heads[h]
    kv = h // w.group
    qh = q[h].float().cpu().numpy().astype(np.float64)
    kh = k[kv].float().cpu().numpy().astype(np.float64)
    vh = v[kv].float().cpu().numpy().astype(np.float64)
    t0 = time.perf_counter()
    sel = oracle.estimate_head(p, qh, kh)
    t_est = time.perf_counter() - t0
    n_same = sum(1 for x in heads if x.pattern == p.pattern)
    # sampled blocks: first, last, and random ones, until the budget is spent
    order = [0, nb - 1] + list(rng.permutation(np.arange(1, nb - 1)))
    t_idx = t_att = 0.0
    kept_s = 0
    done = 0
    spent = t_est
    for b in order:
        t1 = time.perf_counter()
        if p.pattern == W.VERTICAL_SLASH:
            bidx = oracle.vs_block_index(sel[1], sel[2], b)
        elif p.pattern == W.BLOCK_SPARSE:
            bidx = oracle.bs_block_index(sel[1][b])
        else:
            bidx = oracle.dense_block_index(b)
        t2 = time.perf_counter()
        oracle.attention_block(qh[b * 64:(b + 1) * 64], kh, vh, bidx, b)
        t3 = time.perf_counter()
        m = oracle.block_mask(bidx, b, n) if n <= 65536 else None
        kept_s += int(m.sum()) if m is not None else _kept_np(bidx, b)
        t_idx += t2 - t1
        t_att += t3 - t2
        done += 1
        spent += t3 - t1
        if done >= 16 and spent > budget_s:
            break
        if done >= 256:
            break
    est_layer = t_est * n_same
    idx_layer = t_idx / done * nb * len(heads)
    att_layer = t_att / max(kept_s, 1) * kept_total
    total_ms = (est_layer + idx_layer + att_layer) * 1e3
    return {
        "value": round(total_ms, 1),
        "unit": "ms/layer",
        "cores": int(cores),
        "kind": "oracle",
        "sample": (f"float64 oracle, head {h}: estimation over all {n} keys ({t_est:.1f} s, x{n_same} heads), "
                   f"index + attention on {done} sampled query blocks of {nb} (first, last, random); "
                   f"attention extrapolated by kept entries ({kept_s} sampled of {kept_total}); "
                   f"wall {spent:.1f} s"),
    }


def _kept_np(bidx, b):
    rng, cols = bidx
    row0 = b * 64
    tot = 0
    for lo, hi in rng.tolist():
        for r in range(64):
            tot += max(0, min(hi, row0 + r + 1) - lo)
    tot += sum(min(64, max(0, row0 + 64 - int(j))) for j in cols)
    return tot


# ---------------------------------------------------------------- main
def run_layer(ms, torch, W, cid, steps, warmup, dense_steps, do_dense, dense_known=None):
    w = W.config(cid)
    q, k, v = W.generate(w, device="cuda")
    prob, hp = ms.problem(w.n, w.n_q_heads, w.n_kv_heads), ms.head_params(w.heads)
    out = torch.empty_like(q)
    ws = ms.empty_workspace(ms.ms_workspace_bytes(prob, hp))
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        ms.ms_sparse_attn(prob, hp, q, k, v, out, ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        ms.ms_sparse_attn(prob, hp, q, k, v, out, ws)
    e1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_step = e0.elapsed_time(e1) / steps

    # Short sequences are bound by launch latency (about 20 kernels per
    # call): the same call captured once in a HIP graph and replayed.
    graph_ms = None
    if w.n <= 32768:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            ms.ms_sparse_attn(prob, hp, q, k, v, out, ws)
        g.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(max(steps, 10)):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        graph_ms = e0.elapsed_time(e1) / max(steps, 10)
        del g

    # Stage split: the attention kernel alone (index already built by the
    # steps above) and estimation + index conversion.
    nv, ns, nbk = ms.ms_selection_sizes(prob, hp)
    vert = torch.empty(max(nv, 1), dtype=torch.int32, device="cuda")
    slash = torch.empty(max(ns, 1), dtype=torch.int32, device="cuda")
    blocks = torch.empty(max(nbk, 1), dtype=torch.int32, device="cuda")
    ews = ms.empty_workspace(ms.ms_estimate_workspace_bytes(prob, hp))
    index = ms.empty_workspace(ms.ms_index_bytes(prob, hp))
    aws = ms.empty_workspace(ms.ms_attn_workspace_bytes(prob))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    ev[0].record(stream)
    ms.ms_estimate_vs(prob, hp, q, k, vert, slash, ews)
    ms.ms_estimate_block(prob, hp, q, k, blocks, ews)
    ev[1].record(stream)
    ms.ms_build_index(prob, hp, vert, slash, blocks, index)
    lse_s = torch.empty((w.n_q_heads, w.n), dtype=torch.float32, device="cuda")
    ev[2].record(stream)
    ms.ms_sparse_attn_indexed(prob, hp, q, k, v, index, out, aws, lse_s)
    ev[3].record(stream)
    torch.cuda.synchronize()
    t_est, t_idx, t_att = (ev[i].elapsed_time(ev[i + 1]) for i in range(3))
    reps = 3 if t_att < 1000.0 else 0   # short kernels: average a few more launches
    if reps:
        ev[2].record(stream)
        for _ in range(reps):
            ms.ms_sparse_attn_indexed(prob, hp, q, k, v, index, out, aws, lse_s)
        ev[3].record(stream)
        torch.cuda.synchronize()
        t_att = ev[2].elapsed_time(ev[3]) / reps
    del ews
    kept = kept_entries(ms, prob, hp, w.heads, index, torch)
    bkeys, ckeys = block_keys(ms, prob, hp, index, torch)
    dense_pairs = w.n * (w.n + 1) // 2 * w.n_q_heads
    del index
    res = {"w": w, "q": q, "k": k, "v": v, "ms": ms_step, "wall_s": t_wall, "t_est": t_est, "t_idx": t_idx,
           "t_att": t_att, "kept": kept, "block_keys": bkeys, "col_keys": ckeys, "dense_pairs": dense_pairs,
           "graph_ms": graph_ms}
    if all(p.pattern == W.VERTICAL_SLASH for p in w.heads) and any(p.n_vertical > 0 for p in w.heads):
        res["gather"] = gather_stage(ms, torch, W, w, q, k, v, vert, aws, stream)
    del ws
    if do_dense and dense_known is not None:
        # the same shapes and inputs as a layer already timed: its dense
        # kernel time and log-sum-exps serve again
        res["dense_ms"] = dense_known["ms"]
        rec = torch.empty(w.n_q_heads, dtype=torch.float32, device="cuda")
        ms.ms_attention_recall(prob, lse_s, dense_known["lse"], rec)
        torch.cuda.synchronize()
        res["recall"] = rec.cpu().tolist()
    elif do_dense:
        dout = torch.empty_like(q)
        d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        # untimed first call: warms the kernel and gives the dense log-sum-exps
        # for the index-quality instrument
        lse_d = torch.empty_like(lse_s)
        ms.ms_dense_attn(prob, q, k, v, dout, aws, lse_d)
        rec = torch.empty(w.n_q_heads, dtype=torch.float32, device="cuda")
        ms.ms_attention_recall(prob, lse_s, lse_d, rec)
        torch.cuda.synchronize()
        res["recall"] = rec.cpu().tolist()
        res["dense_lse"] = lse_d
        d0.record(stream)
        for _ in range(dense_steps):
            ms.ms_dense_attn(prob, q, k, v, dout, aws)
        d1.record(stream)
        torch.cuda.synchronize()
        res["dense_ms"] = d0.elapsed_time(d1) / dense_steps
        del dout
    del out, aws
    return res


def summary(r):
    d = 128
    kept_tf = 4.0 * d * r["kept"] / 1e12
    att_tflops = kept_tf / (r["t_att"] / 1e3)
    s = {
        "ms_per_layer": round(r["ms"], 3),
        "stages_ms": {"estimate": round(r["t_est"], 3), "index": round(r["t_idx"], 3),
                      "attention": round(r["t_att"], 3)},
        "kept_fraction": round(r["kept"] / r["dense_pairs"], 5),
        "flop_ratio_bound": round(r["dense_pairs"] / r["kept"], 3),
        "kept_tflop": round(kept_tf, 3),
        "attention_tflops": round(att_tflops, 1),
        "attention_mfma_frac": round(att_tflops / PEAK_BF16_TFLOPS, 4),
        "effective_tflops": round(kept_tf / (r["ms"] / 1e3), 1),
    }
    if r.get("graph_ms") is not None:
        s["graph_replay_ms_per_layer"] = round(r["graph_ms"], 3)
    # K/V rows the kernels bring in when no row is reused across query blocks
    # (512 B per kept (query block, key) pair: a bf16 K row and an fp16 V row);
    # L2 reuse and heads served together make the HBM traffic smaller.
    att_bytes = 512.0 * r["block_keys"]
    s["attention_kv_rows_gbs"] = round(att_bytes / (r["t_att"] / 1e3) / 1e9, 1)
    s["attention_flop_per_kv_row_byte"] = round(4.0 * d * r["kept"] / att_bytes, 1)
    if "gather" in r:
        g = r["gather"]
        gb = 512.0 * g["col_keys"]
        s["gather"] = {"ms": round(g["ms"], 3), "bytes": gb, "gbs": round(gb / (g["ms"] / 1e3) / 1e9, 1),
                       "frac_of_hbm_peak": round(gb / (g["ms"] / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
                       "what": "the layer's heads with their verticals only: every kept key a gathered column, "
                               "512 B of K/V rows per (query block, column) delivered to the kernel; a head's "
                               "columns are the same for every query block, so L2 serves most of them and the "
                               "rate can exceed the HBM peak"}
    eb = estimate_bytes(r["w"])
    s["estimate_gbs"] = round(eb / (r["t_est"] / 1e3) / 1e9, 1)
    s["estimate_hbm_frac"] = round(s["estimate_gbs"] / PEAK_HBM_GBS, 4)
    if "recall" in r:
        # share of the full causal attention mass the estimated index keeps
        # (mean over rows, per head), summarised over heads and per pattern
        rec = r["recall"]
        names = {0: "a_shape", 1: "vertical_slash", 2: "block_sparse", 3: "dense"}
        s["attention_mass_recall"] = {"mean": round(sum(rec) / len(rec), 5), "min": round(min(rec), 5)}
        for pat, name in names.items():
            vals = [x for x, p in zip(rec, r["w"].heads) if p.pattern == pat]
            if vals:
                s["attention_mass_recall"][name] = round(sum(vals) / len(vals), 5)
    if "dense_ms" in r:
        dense_tf = 4.0 * d * r["dense_pairs"] / 1e12
        s["dense_ms"] = round(r["dense_ms"], 3)
        s["dense_tflops"] = round(dense_tf / (r["dense_ms"] / 1e3), 1)
        s["dense_mfma_frac"] = round(dense_tf / (r["dense_ms"] / 1e3) / PEAK_BF16_TFLOPS, 4)
        s["speedup_vs_dense"] = round(r["dense_ms"] / r["ms"], 3)
        # an equally efficient dense kernel cannot be beaten by more than the
        # FLOP ratio; a larger speedup flags a weak dense baseline
        s["speedup_exceeds_flop_bound"] = s["speedup_vs_dense"] > s["flop_ratio_bound"]
    return s


def main():
    a = parse()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(f"bench.py runs on one GPU only (asked for {a.gpus}); the sparse path has no multi-GPU form here.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import dynamic_sparse_attention_est_amd as ms
    import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    ms.load()
    print(f"[bench] headline {a.workload}: warmup {a.warmup}, steps {a.steps}", file=sys.stderr, flush=True)
    main_r = run_layer(ms, torch, W, WORKLOADS[a.workload], a.steps, a.warmup, a.dense_steps, not a.no_dense)
    main_s = summary(main_r)
    print(f"[bench] {a.workload}: {json.dumps(main_s)}", file=sys.stderr, flush=True)

    cpu = None
    if not a.no_cpu:
        print("[bench] cpu baseline (oracle sample)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(main_r["w"], main_r["q"], main_r["k"], main_r["v"], main_r["w"].heads, main_r["kept"],
                           a.cpu_seconds)
    for key in ("q", "k", "v"):
        main_r.pop(key)
    known = {"ms": main_r["dense_ms"], "lse": main_r.pop("dense_lse")} if "dense_ms" in main_r else None
    torch.cuda.empty_cache()

    side = {}
    for name in [x for x in a.side.split(",") if x and x != a.workload]:
        print(f"[bench] side workload {name}", file=sys.stderr, flush=True)
        # vs_1m_b32 is the headline's layer (same inputs) with other index blocks
        reuse = known if (a.workload, name) == ("vs_1m", "vs_1m_b32") else None
        r2 = run_layer(ms, torch, W, WORKLOADS[name], min(a.steps, a.side_steps), min(a.warmup, 1), a.dense_steps,
                       not a.no_dense, reuse)
        r2.pop("dense_lse", None)
        for key in ("q", "k", "v"):
            r2.pop(key)
        side[name] = summary(r2)
        if reuse is not None:
            side[name]["note"] = "dense time and log-sum-exps of the headline layer (same shapes and inputs)"
        if name == "vs_1m_s":
            side[name]["note"] = ("diagnostic, not one of the five workloads: vs_1m plus a shared query mean "
                                  "(std 0.5) per KV group, so the slashes through the planted columns are selected")
        print(f"[bench] {name}: {json.dumps(side[name])}", file=sys.stderr, flush=True)
        del r2
        torch.cuda.empty_cache()

    if a.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    w = main_r["w"]
    # Roofline of the dominant kernel, the sparse attention of the headline
    # layer (on long sequences the per-head kernel, paced, launched once per
    # 1024 workgroups, plus the fp16 V copy, < 1%): MFMA-bound work of 4*128 flop per kept
    # (row, key) pair, over the attention call's duration measured with HIP
    # events on the library's stream.
    kept_flop = 4.0 * 128 * main_r["kept"]
    compulsory = (2 * w.n_q_heads + 2 * w.n_kv_heads) * w.n * 128 * 2  # Q, K, V read, out written (bf16)
    csrc = os.path.join(ROOT, "dynamic_sparse_attention_est_amd", "csrc")
    traffic, trec = recorded_traffic(a.workload, [os.path.join(csrc, f) for f in ATTN_SOURCES])
    roof = {"bound": "mfma", "achieved": main_s["attention_tflops"], "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": main_s["attention_mfma_frac"], "traffic": traffic,
            "kernel": "sparse attention stage of one call: the attention kernels (on long sequences the "
                      "per-head kernel in paced mode, one launch per 1024 workgroups) and the fp16 V copy "
                      "they read",
            "work": "4*128 flop per kept (row, key) pair, kept pairs counted exactly from the index",
            "flop_per_launch": kept_flop, "launch_ms": round(main_r["t_att"], 3)}
    if traffic is not None:
        roof["hbm_gbs"] = round(traffic / (main_r["t_att"] / 1e3) / 1e9, 1)
        roof["hbm_frac"] = round(roof["hbm_gbs"] / PEAK_HBM_GBS, 4)
        roof["traffic_over_compulsory"] = round(traffic / compulsory, 1)
        roof["flop_per_hbm_byte"] = round(kept_flop / traffic, 1)
        roof["traffic_source"] = f"profiles/traffic_attention_{a.workload}.md"
    elif trec is not None:
        roof["traffic_note"] = "recorded counters are for an older kernel source; not reported"
    roof["compulsory_bytes"] = compulsory
    roof["estimation"] = {"gbs": main_s["estimate_gbs"], "peak": PEAK_HBM_GBS, "frac": main_s["estimate_hbm_frac"],
                          "ms": main_s["stages_ms"]["estimate"]}
    if "gather" in main_s:
        roof["gather"] = {"gbs": main_s["gather"]["gbs"], "peak": PEAK_HBM_GBS,
                          "frac": main_s["gather"]["frac_of_hbm_peak"], "ms": main_s["gather"]["ms"],
                          "note": "gathered K/V rows delivered (L2 and HBM) per second"}
    line = {
        "metric": "ms/layer sparse prefill attn (est+kernel) at 128K & 1M; speedup vs dense",
        "value": round(main_r["ms"], 3),
        "unit": "ms/layer",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(main_r["ms"], 3),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded generators shaped like the pages' workloads; no datasets or weights)",
        "config": {"workload": f"{w.name}: {w.n_q_heads} Q / {w.n_kv_heads} KV heads, n={w.n}, d=128, "
                               + ", ".join(sorted({_head_desc(h) for h in w.heads})),
                   "seq_len": w.n, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads, "batch": 1,
                   "parallelism": "single GPU"},
        "result": main_s,
        "side": side,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


def _head_desc(h):
    if h.pattern == 1:
        return f"VS {h.n_vertical}v/{h.n_slash}s"
    if h.pattern == 2:
        return f"BS top-{h.top_k_blocks}"
    if h.pattern == 0:
        return f"A-shape sink {h.sink}/window {h.window}"
    return "dense"


if __name__ == "__main__":
    main()
