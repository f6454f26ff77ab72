"""Benchmark of the MSA forward path on one MI355X.

One step = msa_forward over one batch of the workload: index scores fused with
the block max-pool, the exp-free Top-k, and block-sparse attention.  Inputs
are seeded synthetic tensors drawn on the device and resident in HBM before
the timed region starts.

Prints ONE JSON line.  ``value`` is tokens/s (queries of the batch per second)
on the largest single-GPU prefill workload: 16384 new queries at positions
1032192 .. 1048575 of a 1,048,576-token causal prefix (B=1, 64/8 heads, head
dim 128, index dim 128, block 128, k=16).  Alongside: mean, median and
minimum step times, algorithmic TFLOP/s and the fraction of the bf16 MFMA
peak, every stage's time and rate (per-chunk launches summed), the attention
as one step, the roofline of the dominant kernel, the CPU oracle timed on a
bounded row sample of the same workload, the 32K and 128K (per-block gain)
prefill workloads, the decode workload (64 sequences against a 256K-token
cache) as HBM GB/s and fraction of peak, and on the 32K workload the forward
value of the index branch's alignment loss, the backward (main branch and
alignment loss) and the block-mask form of the selection.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MSA fwd tokens/s + TFLOP/s (%MFMA peak) prefill; decode HBM GB/s (%peak)"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


# ------------------------------------------------------------ work counts
def positions(w):
    return np.arange(w.seqlen_q, dtype=np.int64) + (w.seqlen_k - w.seqlen_q)


def visible_tokens(w):
    """|T_i| per query: every visible token while the local block index is
    below k, else k-1 full blocks plus the visible part of the local block."""
    t = positions(w)
    local = t // w.block_size
    sparse = (w.topk - 1) * w.block_size + (t % w.block_size) + 1
    return np.where(local < w.topk, t + 1, sparse)


def index_flops(w):
    return 2.0 * w.index_dim * w.heads_kv * w.batch * float((positions(w) + 1).sum())


def attn_flops(w):
    return 4.0 * w.head_dim * w.heads_q * w.batch * float(visible_tokens(w).sum())


def decode_bytes(w):
    """Algorithmic HBM bytes of one decode step: the index-key scan, the
    selected K/V blocks, Q, O, Q_idx and the selection."""
    kidx = w.batch * w.seqlen_k * w.index_dim * 2
    kv = w.batch * w.heads_kv * float(visible_tokens(w).sum()) * w.head_dim * 2 * 2
    q = w.batch * w.seqlen_q * w.heads_q * w.head_dim * 2
    qidx = w.batch * w.seqlen_q * w.heads_kv * w.index_dim * 2
    idx = w.batch * w.heads_kv * w.seqlen_q * w.topk * 4
    return kidx + kv + 2 * q + qidx + idx


# ------------------------------------------------------------ timing
def time_loop(fn, steps, stream):
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def run_workload(w, steps, warmup):
    """Warm up, time `steps` forward steps (an event at every step boundary,
    so the mean, median and minimum come from one timed run), then time each
    internal stage over another `steps` steps through msa_forward_profiled:
    the index scores and the Top-k once per step, the three attention stages
    once per query chunk."""
    import torch

    import block_sparse_gqa_scores_amd as msa
    import synth

    dev = torch.device("cuda", 0)
    t = synth.device_tensors(w, dev)
    d = msa.dims_of(t["q"], t["k"], t["q_idx"], t["k_idx"], topk=w.topk)
    ws_bytes = msa.msa_workspace_bytes(d, msa.ENTRY_FORWARD)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    chunks = msa.msa_attn_chunks(d, msa.ENTRY_FORWARD, ws_bytes)
    out = torch.empty_like(t["q"])
    stream = torch.cuda.current_stream(dev)

    def step(events=None):
        msa.msa_forward(t["q"], t["k"], t["v"], t["q_idx"], t["k_idx"], topk=w.topk, out=out,
                        workspace=ws, stage_events=events)

    for _ in range(warmup):
        step()
    bounds = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    bounds[0].record(stream)
    for k in range(steps):
        step()
        bounds[k + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_step = [bounds[k].elapsed_time(bounds[k + 1]) for k in range(steps)]
    timing = {"mean": bounds[0].elapsed_time(bounds[-1]) / steps, "median": float(np.median(per_step)),
              "min": float(min(per_step)), "wall_s": wall}

    n_ev = msa.n_stage_events(chunks)
    evs = []
    for _ in range(steps):
        pair = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
        for e in pair:
            e.record(stream)  # creates the underlying event
        evs.append(pair)
    torch.cuda.synchronize()
    for pair in evs:
        step([e.cuda_event for e in pair])
    torch.cuda.synchronize()

    def span(p, x):
        return p[x].elapsed_time(p[x + 1])

    stage_ms = {"index_scores": sum(span(p, 0) for p in evs) / steps,
                "block_topk": sum(span(p, 2) for p in evs) / steps}
    for m, name in enumerate(msa.ATTN_STAGES):
        # per step: the sum over the chunks' launches of this stage
        stage_ms[name] = sum(span(p, 4 + 6 * c + 2 * m) for p in evs for c in range(chunks)) / steps
    return t, timing, stage_ms, chunks


def fused_selection(w):
    """msa_forward scores and selects in one kernel for these shapes (msa.h)."""
    return w.seqlen_q * w.heads_kv > 32 and w.topk <= 16


def selection_mask_rates(w, t, steps):
    """The block-mask form of the workload's selection (Sparse Attention Part
    II, section 4.3): time msa_block_mask and msa_mask_blocks on the forward's
    selection; bytes = what each call reads and writes."""
    import torch

    import block_sparse_gqa_scores_amd as msa

    stream = torch.cuda.current_stream()
    _, idx = msa.msa_forward(t["q"], t["k"], t["v"], t["q_idx"], t["k_idx"], topk=w.topk, return_idx=True)
    mask = msa.msa_block_mask(idx, seqlen_k=w.seqlen_k)
    back = torch.empty_like(idx)
    torch.cuda.synchronize()
    rows = w.batch * w.heads_kv * w.seqlen_q
    idx_bytes, mask_bytes = rows * w.topk * 4, rows * (-(-w.n_blk // 32)) * 4
    res = {"workload": f"{w.name} selection ({rows} rows of {w.topk} blocks, {w.n_blk} blocks per row)"}
    for name, fn in (("block_mask", lambda: msa.msa_block_mask(idx, seqlen_k=w.seqlen_k, mask=mask)),
                     ("mask_blocks", lambda: msa.msa_mask_blocks(mask, seqlen_k=w.seqlen_k, topk=w.topk,
                                                                 block_idx=back))):
        fn()
        ms = time_loop(fn, steps, stream)
        res[name] = {"ms": ms, "bytes": idx_bytes + mask_bytes,
                     "GB/s": (idx_bytes + mask_bytes) / (ms * 1e-3) / 1e9}
    torch.cuda.synchronize()
    res["round_trip_exact"] = bool(torch.equal(back, idx))
    return res


def kl_loss_flops(w):
    """Algorithmic FLOPs of the alignment loss: the main-branch logits of every
    head and the index scores, over each row's selected visible tokens."""
    tok = w.batch * float(visible_tokens(w).sum())
    return 2.0 * w.head_dim * w.heads_q * tok + 2.0 * w.index_dim * w.heads_kv * tok


def alignment_loss_rate(w, t, steps):
    """Forward value of the index branch's alignment loss (Sparse Attention
    Part II, section 3.2) on the forward's selection and LSE: time of
    msa_kl_loss_fwd, algorithmic TFLOP/s and the fraction of the MFMA peak."""
    import torch

    import block_sparse_gqa_scores_amd as msa

    stream = torch.cuda.current_stream()
    _, lse, idx = msa.msa_forward(t["q"], t["k"], t["v"], t["q_idx"], t["k_idx"], topk=w.topk,
                                  return_lse=True, return_idx=True)
    d = msa.dims_of(t["q"], t["k"], t["q_idx"], t["k_idx"], topk=w.topk)
    ws = torch.empty(msa.msa_workspace_bytes(d, msa.ENTRY_KL_LOSS_FWD), dtype=torch.uint8, device=lse.device)

    def fn():
        return msa.msa_kl_loss_fwd(t["q"], t["k"], t["q_idx"], t["k_idx"], idx, lse, workspace=ws)

    loss = fn()
    ms = time_loop(fn, steps, stream)
    fl = kl_loss_flops(w)
    tf = fl / (ms * 1e-3) / 1e12
    res = {"workload": w.name, "ms": ms, "algorithmic_flops": fl, "TFLOP/s": tf,
           "mfma_frac": tf / PEAK_BF16_TFLOPS, "loss": float(loss.item())}
    del ws
    return res


def backward_rates(w, t, steps):
    """The backward on the forward's selection (next to the forward, not part
    of its step): msa_sparse_attn_bwd (dq, dk, dv from a seeded dO),
    msa_kl_loss_bwd (gradients of the alignment loss into q_idx, k_idx) and
    msa_backward (both in one call, sharing each query chunk's edge buckets).
    Algorithmic FLOPs per call: the main branch recomputes S and forms dP,
    dV, dK and dq, five products of 2 D H_q sum|T_i| each; the loss backward
    recomputes the main logits (2 D H_q sum|T_i|) and forms z, dk_idx and
    dq_idx (2 D_idx H_kv sum|T_i| each); the combined call's count takes S
    once, although its loss kernels form S again on their own."""
    import torch

    import block_sparse_gqa_scores_amd as msa
    import synth

    stream = torch.cuda.current_stream()
    dout = torch.empty_like(t["q"])
    synth.fill_device(w, "dout", dout)
    out, lse, idx = msa.msa_forward(t["q"], t["k"], t["v"], t["q_idx"], t["k_idx"], topk=w.topk,
                                    return_lse=True, return_idx=True)
    _, lse_idx = msa.msa_kl_loss_fwd(t["q"], t["k"], t["q_idx"], t["k_idx"], idx, lse, return_lse_idx=True)
    d = msa.dims_of(t["q"], t["k"], t["q_idx"], t["k_idx"], topk=w.topk)
    ws = torch.empty(max(msa.msa_workspace_bytes(d, msa.ENTRY_SPARSE_ATTN_BWD),
                         msa.msa_workspace_bytes(d, msa.ENTRY_KL_LOSS_BWD),
                         msa.msa_workspace_bytes(d, msa.ENTRY_BACKWARD)), dtype=torch.uint8, device=lse.device)
    tok = w.batch * float(visible_tokens(w).sum())
    main_fl = 5 * 2.0 * w.head_dim * w.heads_q * tok
    loss_fl = 2.0 * w.head_dim * w.heads_q * tok + 3 * 2.0 * w.index_dim * w.heads_kv * tok
    legs = {
        "sparse_attn_bwd": (lambda: msa.msa_sparse_attn_bwd(t["q"], t["k"], t["v"], idx, out, lse, dout,
                                                             workspace=ws),
                            main_fl),
        "kl_loss_bwd": (lambda: msa.msa_kl_loss_bwd(t["q"], t["k"], t["q_idx"], t["k_idx"], idx, lse, lse_idx,
                                                     1.0, workspace=ws),
                        loss_fl),
        "msa_backward": (lambda: msa.msa_backward(t["q"], t["k"], t["v"], t["q_idx"], t["k_idx"], idx, out, lse, lse_idx,
                                           dout, 1.0, workspace=ws),
                  main_fl + loss_fl - 2.0 * w.head_dim * w.heads_q * tok),
    }
    res = {"workload": w.name}
    for name, (fn, fl) in legs.items():
        fn()
        ms = time_loop(fn, steps, stream)
        tf = fl / (ms * 1e-3) / 1e12
        res[name] = {"ms": ms, "algorithmic_flops": fl, "TFLOP/s": tf, "mfma_frac": tf / PEAK_BF16_TFLOPS}
    del ws, dout
    return res


def stage_work(w):
    """Algorithmic work of each forward stage per step: (bound, amount, unit).
    With the fused selection the Top-k runs inside the index stage and its own
    stage is empty (bound "fused").  The attention stages' work is the whole
    step's, summed over the query chunks they run in."""
    rows = w.batch * w.heads_kv * w.seqlen_q
    edges = w.batch * w.heads_kv * float(np.minimum(positions(w) // w.block_size + 1, w.topk).sum())
    G = w.group
    index = ("mfma", index_flops(w), "FLOP")
    if w.seqlen_q * w.heads_kv <= 32:  # decode: the index-key cache stream bounds the scan
        index = ("hbm", w.batch * (w.seqlen_k * w.index_dim * 2.0 + rows / w.batch * (w.index_dim * 2.0 + w.n_blk * 4.0)), "B")
    partial = ("mfma", attn_flops(w), "FLOP")
    if w.seqlen_q == 1:  # decode: one query per block, the selected K/V bytes bound it
        partial = ("hbm", w.batch * w.heads_kv * float(visible_tokens(w).sum()) * w.head_dim * 4.0
                   + w.batch * w.heads_q * w.head_dim * 2.0, "B")
    return {
        "index_scores": index,
        "block_topk": ("fused", 0.0, "B") if fused_selection(w) else ("hbm", rows * (w.n_blk + w.topk) * 4.0, "B"),
        "attn_build": ("hbm", rows * w.topk * 4.0 * 2 + edges * 4.0, "B"),
        "attn_partial": partial,
        # records of 12-bit codes (1.5 bytes a value) plus 8 bytes of statistics per head
        "attn_merge": ("hbm", edges * G * (1.5 * w.head_dim + 8) + rows * G * w.head_dim * 2.0, "B"),
    }


LAUNCHES = {"index_scores": lambda chunks: 1, "block_topk": lambda chunks: 1,
            "attn_build": lambda chunks: chunks, "attn_partial": lambda chunks: chunks,
            "attn_merge": lambda chunks: chunks}


def rate(bound, amount, ms):
    """Achieved rate of `amount` of work in `ms`: (value, unit, peak)."""
    if bound == "mfma":
        return amount / (ms * 1e-3) / 1e12, "TFLOP/s", PEAK_BF16_TFLOPS
    return amount / (ms * 1e-3) / 1e9, "GB/s", PEAK_HBM_GBS


def stage_rates(w, stage_ms, chunks):
    """Per stage: ms per step, launches per step, and the achieved rate of its
    work over its own time (a one-launch stage over that launch, a per-chunk
    stage over the sum of its chunks' launches)."""
    out = {}
    for name, (bound, amount, _) in stage_work(w).items():
        st = {"ms_per_step": stage_ms[name], "launches_per_step": LAUNCHES[name](chunks), "bound": bound}
        if bound != "fused" and stage_ms[name] > 0:
            r, unit, peak = rate(bound, amount, stage_ms[name])
            st[unit] = r
            st["frac"] = r / peak
        out[name] = st
    return out


def attention_step(w, stage_ms, chunks):
    """The block-sparse attention as one step (bucket build + partial +
    merge, all chunks): algorithmic FLOPs over its whole time."""
    ms = stage_ms["attn_build"] + stage_ms["attn_partial"] + stage_ms["attn_merge"]
    tf = attn_flops(w) / (ms * 1e-3) / 1e12
    return {"ms_per_step": ms, "chunks": chunks, "algorithmic_flops": attn_flops(w), "TFLOP/s": tf,
            "mfma_frac": tf / PEAK_BF16_TFLOPS,
            "what": "bucket build + attention partials + merge, summed over the query chunks"}


def roofline(w, stage_ms, chunks):
    """The dominant kernel's algorithmic work per launch over its average
    launch time (HIP events on the launch stream)."""
    work = stage_work(w)
    dom = max(stage_ms, key=stage_ms.get)
    bound, amount, _ = work[dom]
    n = LAUNCHES[dom](chunks)
    per_launch_ms = stage_ms[dom] / n
    ach, unit, peak = rate(bound, amount / n, per_launch_ms)
    return {"bound": bound, "achieved": ach, "peak": peak, "unit": unit, "frac": ach / peak,
            "traffic": measured_traffic(w, dom, chunks), "kernel": kernel_of_stage(w, dom), "launches_per_step": n,
            "avg_launch_ms": per_launch_ms, "work_per_launch": amount / n}


# Committed counter summaries: HBM bytes per launch of a kernel on a workload,
# valid while the sha256 of the listed sources matches the measured code.
TRAFFIC_FILES = {
    ("prefill_32k", "attn_partial"): ("attn_partial_prefill_32k_traffic.txt",
                                      ("sparse_attn.hip", "edge_buckets.h", "device_common.h")),
    ("chunk_16k_of_1m", "index_scores"): ("index_scan_chunk_16k_of_1m_traffic.txt", ("index_scan.hip", "device_common.h")),
    ("decode_64x256k", "index_scores"): ("index_scan_decode_64x256k_traffic.txt", ("index_scan.hip", "device_common.h")),
    ("prefill_128k_gain", "attn_partial"): ("attn_partial_prefill_128k_gain_traffic.txt",
                                            ("sparse_attn.hip", "edge_buckets.h", "device_common.h")),
}


def source_digest(files):
    import hashlib
    csrc = os.path.join(ROOT, "block_sparse_gqa_scores_amd", "csrc")
    return hashlib.sha256(b"".join(open(os.path.join(csrc, f), "rb").read() for f in files)).hexdigest()


def measured_traffic(w, stage, chunks):
    """HBM bytes per launch from the committed counter summary of this kernel
    (FETCH_SIZE + WRITE_SIZE, each scaled by the copy-kernel calibration), or
    None when there is none, the kernel's source changed since, or the
    attention ran in another number of query chunks than when it was
    measured (a launch then covers another share of the edges)."""
    key = TRAFFIC_FILES.get((w.name, stage))
    if key is None:
        return None
    path = os.path.join(ROOT, "profiles", key[0])
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if source_digest(key[1]) != fields.get("source_sha256"):
        return None
    if "attn_chunks" in fields and int(fields["attn_chunks"]) != chunks:
        return None
    return float(fields["hbm_bytes_per_launch"])


def kernel_of_stage(w, stage):
    if stage == "index_scores":
        if w.seqlen_q * w.heads_kv <= 32:
            return f"index_scan_decode<{w.index_dim}>"
        if fused_selection(w):
            return f"index_select_kernel<{w.index_dim}>"
        return f"index_scan_prefill<{w.index_dim}, 2, 8>"
    return {"block_topk": "block_topk_kernel", "attn_build": "zero/bucket_count/scan/bucket_fill kernels",
            "attn_partial": f"attn_decode_kernel<{w.group}>" if w.seqlen_q == 1 else f"attn_partial_kernel<{w.group}>",
            "attn_merge": f"merge_kernel<{w.group}>"}[stage]


def forward_summary(w, timing, stage_ms, chunks):
    """ms per step (mean, median, min), tokens/s, algorithmic TFLOP/s of the
    whole forward, the stages and the attention step of one workload."""
    fi, fa = index_flops(w), attn_flops(w)
    ms = timing["mean"]
    return {"workload": w.name, "ms_per_step": ms, "ms_per_step_median": timing["median"],
            "ms_per_step_min": timing["min"], "tokens/s": w.batch * w.seqlen_q / (ms * 1e-3),
            "TFLOP/s": (fi + fa) / (ms * 1e-3) / 1e12, "mfma_frac": (fi + fa) / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "algorithmic_flops": {"index": fi, "attention": fa}, "attn_chunks": chunks,
            "stages": stage_rates(w, stage_ms, chunks), "attention": attention_step(w, stage_ms, chunks),
            "roofline": roofline(w, stage_ms, chunks)}


def selection_stats(w, t, tiles=(8, 32, 128)):
    """Block-level against token-level sparsity of one forward's selection:
    for query tiles of T consecutive queries of one (b, g), the distinct
    blocks the tile selects (its union) against its (query, block) edges.
    eff = edges / (union x T) is the fraction of a query-tile kernel's rows
    (every query of the tile against every block of the union) that would
    carry an edge; the edge-bucketed kernels here do work per edge only.
    Also the mean visible tokens per (query, group) row."""
    import torch

    import block_sparse_gqa_scores_amd as msa

    _, idx = msa.msa_forward(t["q"], t["k"], t["v"], t["q_idx"], t["k_idx"], topk=w.topk, return_idx=True)
    B, H, S, K = idx.shape
    valid = idx >= 0
    out = {"edges": int(valid.sum().item()), "rows": B * H * S,
           "visible_tokens_per_row": float(visible_tokens(w).mean())}
    for T in tiles:
        if S % T:
            continue
        x = idx.reshape(B * H, S // T, T * K).long()
        v = x >= 0
        bm = torch.zeros(B * H, S // T, w.n_blk + 1, dtype=torch.bool, device=x.device)
        bm.scatter_(2, torch.where(v, x, w.n_blk), True)
        u = bm[..., :w.n_blk].sum(-1)
        total_u = float(u.sum().item())
        out[f"tile{T}"] = {"union_mean": total_u / u.numel(), "union_median": float(u.float().median().item()),
                           "edges_per_tile": float(v.sum().item()) / u.numel(),
                           "eff": float(v.sum().item()) / (total_u * T)}
        del bm, u, x, v
    del idx
    torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------ CPU baseline
def sample_rows(w, n_random, seed=1):
    """Stratified (b, i, g) rows: first/last query of random query blocks, the
    dense/sparse boundary (t = 2047, 2048), t = 0 or 127 mod 128, and random
    rows."""
    rng = np.random.default_rng(seed)
    off = w.seqlen_k - w.seqlen_q
    qs = set()
    nqb = -(-w.seqlen_q // 128)
    for qb in rng.choice(nqb, size=min(nqb, 64), replace=False):
        qs.update({int(qb) * 128, min(w.seqlen_q - 1, int(qb) * 128 + 127)})
    qs.update(t - off for t in (2047, 2048) if 0 <= t - off < w.seqlen_q)
    qs.update(int(x) for x in rng.integers(0, w.seqlen_q, size=n_random))
    rows = [(int(rng.integers(0, w.batch)), q, g) for q in sorted(qs) for g in range(w.heads_kv)]
    return np.array(rows, dtype=np.int64)


def cpu_model():
    """The host CPU's model name (the "model name" line of /proc/cpuinfo)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, t, budget_s):
    import oracle
    import torch

    h = {k: v.contiguous().view(torch.int16).cpu().numpy().view(np.uint16) for k, v in t.items()}
    p = oracle.Problem.of(w)
    threads = oracle.default_threads()
    # Calibrate on a small sample, then size the sample to the time budget.
    probe = sample_rows(w, 8, seed=2)[: max(threads, 16)]
    t0 = time.perf_counter()
    oracle.forward(p, h["q"], h["k"], h["v"], h["q_idx"], h["k_idx"], rows=probe, threads=threads)
    per_row = (time.perf_counter() - t0) / len(probe)
    n_random = int(max(16, budget_s / max(per_row, 1e-6) / w.heads_kv - 140))
    rows = sample_rows(w, n_random)
    t0 = time.perf_counter()
    oracle.forward(p, h["q"], h["k"], h["v"], h["q_idx"], h["k_idx"], rows=rows, threads=threads)
    dt = time.perf_counter() - t0
    rows_per_s = len(rows) / dt
    return {"value": rows_per_s / w.heads_kv, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{len(rows)} (query, group) rows of {w.name} (stratified, seed 1) in {dt:.1f} s; "
                      f"{rows_per_s:.1f} rows/s; a token is one query with all {w.heads_kv} groups"}


def release():
    import gc

    import torch
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


# ------------------------------------------------------------ main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="chunk_16k_of_1m",
                    help="headline workload (default: the largest single-GPU prefill, 16K queries on a 1M prefix)")
    ap.add_argument("--secondary", default="prefill_32k,prefill_128k_gain,prefill_4k",
                    help="comma-separated forward workloads reported beside the headline ('' for none)")
    ap.add_argument("--legs-workload", default="prefill_32k",
                    help="workload of the alignment-loss, backward and selection-mask legs")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-kl", action="store_true", help="skip the alignment-loss measurement")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward measurement")
    ap.add_argument("--backward-extra", default="prefill_128k_gain",
                    help="comma-separated workloads whose backward is reported beside the legs workload's "
                         "('' for none)")
    ap.add_argument("--no-mask", action="store_true", help="skip the selection-mask measurement")
    ap.add_argument("--copy-probe", type=int, default=0,
                    help="run one plain device copy of this many bytes first (counter calibration)")
    ap.add_argument("--no-copy-rate", action="store_true",
                    help="skip the closing 1 GiB device copy that reports the plain copy rate")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(this path has no multi-GPU mode)", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth

    w = synth.WORKLOADS[args.workload]
    if args.copy_probe:
        synth.copy_probe(args.copy_probe)
    print(f"[bench] workload {w.name}: warmup {args.warmup}, steps {args.steps}", file=sys.stderr, flush=True)
    t, timing, stage_ms, chunks = run_workload(w, args.steps, args.warmup)
    head = forward_summary(w, timing, stage_ms, chunks)
    ms = timing["mean"]
    print(f"[bench] {ms:.3f} ms/step (median {timing['median']:.3f}, min {timing['min']:.3f}); "
          f"stages {json.dumps(stage_ms)}", file=sys.stderr, flush=True)

    res = {
        "metric": METRIC, "value": head["tokens/s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "ms_per_step_median": timing["median"], "ms_per_step_min": timing["min"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seqlen_q": w.seqlen_q, "seqlen_k": w.seqlen_k,
                   "heads_q": w.heads_q, "heads_kv": w.heads_kv, "head_dim": w.head_dim,
                   "index_dim": w.index_dim, "block_size": w.block_size, "topk": w.topk,
                   "parallelism": "single GPU"},
        "tflops": head["TFLOP/s"], "mfma_frac": head["mfma_frac"],
        "algorithmic_flops": head["algorithmic_flops"], "stages": head["stages"], "attn_chunks": chunks,
        "attention": head["attention"], "roofline": head["roofline"], "wall_s_timed": timing["wall_s"],
    }
    res["selection"] = selection_stats(w, t)
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(w, t, args.cpu_seconds)
    del t
    release()
    res["workloads"] = {}
    for name in [x for x in args.secondary.split(",") if x and x != w.name]:
        ws_ = synth.WORKLOADS[name]
        print(f"[bench] secondary workload {name}", file=sys.stderr, flush=True)
        ts, tim_s, st_s, ch_s = run_workload(ws_, args.steps, args.warmup)
        res["workloads"][name] = forward_summary(ws_, tim_s, st_s, ch_s)
        res["workloads"][name]["selection"] = selection_stats(ws_, ts)
        del ts
        release()
    legs = synth.WORKLOADS[args.legs_workload]
    if not (args.no_mask and args.no_kl and args.no_backward):
        tl = synth.device_tensors(legs, torch.device("cuda", 0))
        if not args.no_mask:
            res["selection_mask"] = selection_mask_rates(legs, tl, args.steps)
        if not args.no_kl:
            print("[bench] alignment loss ...", file=sys.stderr, flush=True)
            res["alignment_loss"] = alignment_loss_rate(legs, tl, args.steps)
        if not args.no_backward:
            print("[bench] backward ...", file=sys.stderr, flush=True)
            res["backward"] = backward_rates(legs, tl, max(2, args.steps // 2))
        del tl
        release()
    if not args.no_backward:
        res["backward_workloads"] = {}
        for name in [x for x in args.backward_extra.split(",") if x and x != legs.name]:
            wb = synth.WORKLOADS[name]
            print(f"[bench] backward {name} ...", file=sys.stderr, flush=True)
            tb = synth.device_tensors(wb, torch.device("cuda", 0))
            res["backward_workloads"][name] = backward_rates(wb, tb, max(2, args.steps // 4))
            del tb
            release()
    if not args.no_decode:
        wd = synth.WORKLOADS["decode_64x256k"]
        print(f"[bench] decode workload {wd.name}", file=sys.stderr, flush=True)
        td, tim_d, stage_d, chunks_d = run_workload(wd, args.steps, args.warmup)
        nbytes = decode_bytes(wd)
        msd = tim_d["mean"]
        gbs = nbytes / (msd * 1e-3) / 1e9
        res["decode"] = {"workload": wd.name, "ms_per_step": msd, "ms_per_step_median": tim_d["median"],
                         "ms_per_step_min": tim_d["min"], "algorithmic_bytes": nbytes,
                         "GB/s": gbs, "hbm_frac": gbs / PEAK_HBM_GBS,
                         "tokens/s": wd.batch * wd.seqlen_q / (msd * 1e-3),
                         "stages": stage_rates(wd, stage_d, chunks_d), "roofline": roofline(wd, stage_d, chunks_d),
                         "selection": selection_stats(wd, td, tiles=())}
        del td
        release()
    if not args.no_copy_rate:
        # Reference rate of the same HBM: a plain streaming copy (reads and
        # writes 1 GiB each), for reading the GB/s figures above.
        res["copy_rate"] = {"GB/s": synth.copy_probe(1 << 30, reps=11), "bytes": 1 << 30,
                            "what": "plain device copy, bytes read + written per second"}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
