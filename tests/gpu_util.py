"""Helpers of the GPU parity tests: run the device library through its C ABI
(via the thin binding) and compare with the CPU oracle on the same inputs."""
from __future__ import annotations

import numpy as np
import torch

import block_sparse_gqa_scores_amd as msa
import oracle
import synth

# Output tolerance on bf16 outputs against the fp64 oracle: max-abs 1e-2 and
# mean-abs 1e-3.  The output's own rounding to bf16 is excluded from the
# max-abs bound: for |o| >= 2 half an ulp of bf16 alone is 2^-7 or more.
MAX_ABS = 1e-2
MEAN_ABS = 1e-3
LSE_ABS = 1e-3


def to_u16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half the bf16 spacing at |x| (the largest error of correct rounding)."""
    ax = np.abs(x).astype(np.float64)
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return 2.0 ** (e - 8)


def inputs_for(w: synth.Workload, device="cuda"):
    torch.cuda.synchronize()
    t = synth.device_tensors(w, device)
    torch.cuda.synchronize()
    return t


def run_device(w, t, *, with_bm=True):
    res = {}
    if with_bm:
        # The separate entry points: block scores, then the Top-k on them (the
        # forward may fuse both into one kernel; both paths are compared).
        res["bm"] = msa.msa_index_scores(t["q_idx"], t["k_idx"], topk=w.topk)
        res["idx_split"] = msa.msa_block_topk(res["bm"], seqlen_k=w.seqlen_k, topk=w.topk)
    out, lse, idx = msa.msa_forward(t["q"], t["k"], t["v"], t["q_idx"], t["k_idx"], topk=w.topk,
                                    return_lse=True, return_idx=True)
    res.update(out=out, lse=lse, idx=idx)
    torch.cuda.synchronize()
    return res


def host_inputs(t):
    return {k: to_u16(v) for k, v in t.items()}


def compare(w, dev, ref, rows, *, check_bm=True, label=""):
    """Element-by-element comparison of the listed rows (b, i, g)."""
    G = w.group
    b, i, g = rows[:, 0], rows[:, 1], rows[:, 2]
    msgs = []
    if check_bm and "bm" in dev:
        bm = dev["bm"][torch.from_numpy(b), torch.from_numpy(g), torch.from_numpy(i)].cpu().numpy()
        exp = ref["bm"].astype(np.float32)
        bad = ~((bm == exp) | (np.isneginf(bm) & np.isneginf(exp)))
        if bad.any():
            r = np.argwhere(bad)[0]
            msgs.append(f"{label} block scores differ at {int(bad.sum())} entries; first row {rows[r[0]]}"
                        f" block {r[1]}: {bm[r[0], r[1]]} vs {exp[r[0], r[1]]}")
    for key, what in (("idx", "selection"), ("idx_split", "msa_block_topk selection")):
        if key not in dev:
            continue
        idx = dev[key][torch.from_numpy(b), torch.from_numpy(g), torch.from_numpy(i)].cpu().numpy()
        bad = (idx != ref["sel"]).any(axis=1)
        if bad.any():
            r = int(np.argwhere(bad)[0][0])
            msgs.append(f"{label} {what} differs on {int(bad.sum())} rows; first {rows[r]}: "
                        f"{idx[r].tolist()} vs {ref['sel'][r].tolist()}")
    out = dev["out"].float()
    heads = (g[:, None] * G + np.arange(G)[None, :])
    o = out[torch.from_numpy(b)[:, None], torch.from_numpy(i)[:, None], torch.from_numpy(heads)].cpu().numpy()
    o = o.astype(np.float64)
    err = np.abs(o - ref["out"])
    excess = np.maximum(err - bf16_half_ulp(ref["out"]), 0.0)
    if excess.max() > MAX_ABS or err.mean() > MEAN_ABS:
        r = np.unravel_index(np.argmax(excess), excess.shape)
        msgs.append(f"{label} output error: max {err.max():.3e} (beyond rounding {excess.max():.3e}), "
                    f"mean {err.mean():.3e}; worst row {rows[r[0]]} head {r[1]} d {r[2]}")
    lse = dev["lse"][torch.from_numpy(b)[:, None], torch.from_numpy(heads), torch.from_numpy(i)[:, None]]
    lerr = np.abs(lse.cpu().numpy().astype(np.float64) - ref["lse"])
    if lerr.max() > LSE_ABS:
        msgs.append(f"{label} lse error max {lerr.max():.3e}")
    stats = dict(max_abs=float(err.max()), mean_abs=float(err.mean()), lse_max=float(lerr.max()))
    return msgs, stats


def parity(w, rows=None, threads=0, label=None):
    """Run device and oracle on workload ``w``; returns (messages, stats)."""
    label = label or w.name
    t = inputs_for(w)
    dev = run_device(w, t)
    p = oracle.Problem.of(w)
    rows = p.all_rows() if rows is None else rows
    h = host_inputs(t)
    ref = oracle.forward(p, h["q"], h["k"], h["v"], h["q_idx"], h["k_idx"], rows=rows, threads=threads)
    return compare(w, dev, ref, rows, label=label)
