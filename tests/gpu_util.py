"""Helpers of the GPU parity tests: run the device library through its C ABI
(via the thin binding) and compare with the CPU oracle on the same inputs."""
from __future__ import annotations

import numpy as np
import torch

import block_sparse_gqa_scores_amd as msa
import oracle
import synth

# One tolerance rule for every bf16 result against the fp64 oracle (forward
# outputs and gradients alike), applied by check_close and compare:
#   excess = max(|err| - (half the bf16 spacing at the exact value), 0),
#   max(excess) <= 1e-2 * s and mean(excess) <= 1e-3 * s,
# with s = 1 for the forward output (the absolute bounds 1e-2 and 1e-3; |o| is
# bounded by max |v|) and s = max |ref| of the tensor for gradients, whose
# size is set by the problem (it grows with the rows that meet at a key and
# shrinks with the loss's 1 / (B S_q H_kv)).  The bound is on the arithmetic,
# so each value's own rounding to bf16 is taken out of both the max and the
# mean: a correctly rounded bf16 value in [2^e, 2^(e+1)) is up to 2^(e-8)
# away from the exact one (the max alone exceeds 1e-2 once |x| > 2.56) and
# 2^(e-9) on average, which is already 1e-3 at |x| = 0.5, so a tensor whose
# values sit near 1 would fail a raw-mean bound of 1e-3 even if every value
# were exact before rounding.
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


def check_close(name, got, ref, scale=1.0):
    """The tolerance rule above; returns (max excess, mean error)."""
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    excess = np.maximum(err - bf16_half_ulp(ref), 0.0)
    print(f"{name}: max|ref| {np.abs(ref).max():.4g}, max err {err.max():.3e} (beyond rounding "
          f"{excess.max():.3e}), mean err {err.mean():.3e} (beyond rounding {excess.mean():.3e}); "
          f"scale {scale:.4g}", flush=True)
    assert np.isfinite(got).all(), f"{name}: non-finite values (an element was not written?)"
    assert excess.max() <= MAX_ABS * scale, f"{name}: max error {excess.max():.3e} > {MAX_ABS * scale:.3e}"
    assert excess.mean() <= MEAN_ABS * scale, f"{name}: mean error {excess.mean():.3e} > {MEAN_ABS * scale:.3e}"
    return float(excess.max()), float(excess.mean())


def grad_scale(ref) -> float:
    return max(1.0, float(np.abs(ref).max()))


# Outputs and workspaces are filled with poison before every device call, so
# an element the library fails to write cannot pass on stale memory: all-ones
# bytes are NaN in bf16 and fp32; int32 outputs get 0x7F7F7F7F, which is no
# valid block index and not the -1 padding.
def poisoned(shape, dtype, device="cuda"):
    t = torch.empty(shape, dtype=dtype, device=device)
    t.reshape(-1).view(torch.uint8).fill_(0x7F if dtype == torch.int32 else 0xFF)
    return t


def poisoned_workspace(nbytes, device="cuda"):
    return poisoned((max(int(nbytes), 1),), torch.uint8, device)


def forward_outputs(w, device="cuda"):
    """Poisoned out, lse and block_idx tensors of the forward."""
    return dict(out=poisoned(w.shapes()["q"], torch.bfloat16, device),
                lse=poisoned((w.batch, w.heads_q, w.seqlen_q), torch.float32, device),
                block_idx=poisoned((w.batch, w.heads_kv, w.seqlen_q, w.topk), torch.int32, device))


def workspace_for(w, entry, t, ws_bytes=None):
    d = msa.dims_of(t["q"], t["k"], t.get("q_idx"), t.get("k_idx"), topk=w.topk)
    return poisoned_workspace(msa.msa_workspace_bytes(d, entry) if ws_bytes is None else ws_bytes)


def ws_for_chunks(d, entry, n):
    """The smallest workspace with which `entry` runs in n query chunks
    (host-side search over msa_attn_chunks; None if no size gives n)."""
    lo, hi = msa.msa_workspace_min_bytes(d, entry), msa.msa_workspace_bytes(d, entry)
    if msa.msa_attn_chunks(d, entry, hi) > n:
        return None
    while lo < hi:  # smallest size with at most n chunks
        mid = (lo + hi) // 2
        if msa.msa_attn_chunks(d, entry, mid) <= n:
            hi = mid
        else:
            lo = mid + 1
    return lo if msa.msa_attn_chunks(d, entry, lo) == n else None


def spread_index_queries(w, t, seed=11):
    """Replaces t["q_idx"] by rows with two nonzero channels of value +-1:
    every index score z is then the sum or difference of two k_idx entries,
    an integer in [-6, 6] (exact in fp32), so over the ~k * 128 selected
    tokens the student softmax of z is spread (its largest weight is a few
    1e-3) instead of nearly one-hot as with full integer rows."""
    rng = np.random.default_rng(seed)
    B, Sq, Hkv, D = w.shapes()["q_idx"]
    q = np.zeros((B * Sq * Hkv, D), dtype=np.float32)
    r = np.arange(q.shape[0])
    c1 = rng.integers(0, D, q.shape[0])
    c2 = (c1 + rng.integers(1, D, q.shape[0])) % D
    q[r, c1] = rng.choice([-1.0, 1.0], q.shape[0])
    q[r, c2] = rng.choice([-1.0, 1.0], q.shape[0])
    t["q_idx"] = torch.from_numpy(q.reshape(B, Sq, Hkv, D)).to(torch.bfloat16).to(t["q"].device)
    return t


def student_max_weight(w, h, sel, rows):
    """Largest softmax weight of the index scores over each row's selected
    visible tokens (host numpy on bf16 bit patterns; for the spread check)."""
    qi = synth.bf16_bits_to_f32(h["q_idx"]).astype(np.float64)
    ki = synth.bf16_bits_to_f32(h["k_idx"]).astype(np.float64)
    out = []
    for (b, i, g), s in zip(rows, sel):
        t = i + w.seqlen_k - w.seqlen_q
        toks = np.concatenate([np.arange(j * 128, min((j + 1) * 128, t + 1)) for j in s if j >= 0])
        z = ki[b, toks] @ qi[b, i, g]
        p = np.exp(z - z.max())
        out.append(p.max() / p.sum())
    return np.array(out)


def inputs_for(w: synth.Workload, device="cuda"):
    torch.cuda.synchronize()
    t = synth.device_tensors(w, device)
    torch.cuda.synchronize()
    return t


def run_device(w, t, *, with_bm=True, ws_bytes=None):
    """The forward through the C ABI on poisoned outputs and workspace;
    ws_bytes sizes msa_forward's workspace (None: the designed size)."""
    res = {}
    if with_bm:
        # The separate entry points: block scores, then the Top-k on them (the
        # forward may fuse both into one kernel; both paths are compared).
        bm = poisoned((w.batch, w.heads_kv, w.seqlen_q, w.n_blk), torch.float32)
        res["bm"] = msa.msa_index_scores(t["q_idx"], t["k_idx"], topk=w.topk, block_scores=bm)
        res["idx_split"] = msa.msa_block_topk(
            res["bm"], seqlen_k=w.seqlen_k, topk=w.topk,
            block_idx=poisoned((w.batch, w.heads_kv, w.seqlen_q, w.topk), torch.int32))
    o = forward_outputs(w)
    ws = workspace_for(w, msa.ENTRY_FORWARD, t, ws_bytes)
    out, lse, idx = msa.msa_forward(t["q"], t["k"], t["v"], t["q_idx"], t["k_idx"], topk=w.topk,
                                    workspace=ws, **o)
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
    if not np.isfinite(o).all():
        msgs.append(f"{label} output has non-finite values (an element was not written?)")
    if excess.max() > MAX_ABS or excess.mean() > MEAN_ABS:
        r = np.unravel_index(np.argmax(excess), excess.shape)
        msgs.append(f"{label} output error: max {err.max():.3e} (beyond rounding {excess.max():.3e}), "
                    f"mean {err.mean():.3e} (beyond rounding {excess.mean():.3e}); worst row {rows[r[0]]} "
                    f"head {r[1]} d {r[2]}")
    lse = dev["lse"][torch.from_numpy(b)[:, None], torch.from_numpy(heads), torch.from_numpy(i)[:, None]]
    lerr = np.abs(lse.cpu().numpy().astype(np.float64) - ref["lse"])
    if not (lerr.max() <= LSE_ABS):  # also catches NaN
        msgs.append(f"{label} lse error max {lerr.max():.3e}")
    stats = dict(max_abs=float(err.max()), max_excess=float(excess.max()), mean_abs=float(err.mean()),
                 mean_excess=float(excess.mean()), lse_max=float(lerr.max()))
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


def prepare_backward(w, t):
    """Forward, loss forward and a seeded upstream gradient (t["dout"]) for
    the backward entry points; returns (out, lse, idx, lse_idx)."""
    t["dout"] = torch.empty_like(t["q"])
    synth.fill_device(w, "dout", t["dout"])
    out, lse, idx = msa.msa_forward(t["q"], t["k"], t["v"], t["q_idx"], t["k_idx"], topk=w.topk,
                                    **forward_outputs(w))
    _, lse_idx = msa.msa_kl_loss_fwd(t["q"], t["k"], t["q_idx"], t["k_idx"], idx, lse, return_lse_idx=True)
    return out, lse, idx, lse_idx


def fused_backward(w, t, out, lse, idx, lse_idx, grad=1.0, ws_bytes=None):
    """msa_backward on poisoned gradients and workspace; returns
    (dq, dk, dv, dq_idx, dk_idx)."""
    d = msa.dims_of(t["q"], t["k"], t["q_idx"], t["k_idx"], topk=w.topk)
    nbytes = msa.msa_workspace_bytes(d, msa.ENTRY_BACKWARD) if ws_bytes is None else ws_bytes
    res = msa.msa_backward(t["q"], t["k"], t["v"], t["q_idx"], t["k_idx"], idx, out, lse, lse_idx, t["dout"],
                           grad, workspace=poisoned_workspace(nbytes),
                           dq=poisoned(t["q"].shape, torch.bfloat16), dk=poisoned(t["k"].shape, torch.bfloat16),
                           dv=poisoned(t["v"].shape, torch.bfloat16),
                           dq_idx=poisoned(t["q_idx"].shape, torch.bfloat16),
                           dk_idx=poisoned(t["k_idx"].shape, torch.bfloat16))
    torch.cuda.synchronize()
    return res


def backward_against_oracle(w, t, grads, idx, label):
    """Every row's dq, dq_idx and every key's dk, dv, dk_idx against the
    oracle's gradients (the loss's scaled by 1 / (B S_q H_kv)), by the
    tolerance rule above; the selection is checked bit-exact first."""
    dq, dk, dv, dqi, dki = grads
    p = oracle.Problem.of(w)
    rows = p.all_rows()
    h = {n: to_u16(x) for n, x in t.items()}
    ref = oracle.forward(p, h["q"], h["k"], h["v"], h["q_idx"], h["k_idx"], rows=rows)
    assert (idx.cpu().numpy()[rows[:, 0], rows[:, 2], rows[:, 1]] == ref["sel"]).all(), f"{label}: selection differs"
    rdq, rdk, rdv = oracle.attention_bwd(p, h["q"], h["k"], h["v"], h["dout"], ref["sel"], rows)
    rdqi, rdki, _ = oracle.kl_bwd(p, h["q"], h["k"], h["q_idx"], h["k_idx"], ref["sel"], rows)
    c = 1.0 / (w.batch * w.seqlen_q * w.heads_kv)
    G = w.group
    dqn = dq.float().cpu().numpy()
    gdq = np.stack([dqn[bb, ii, gg * G:(gg + 1) * G] for bb, ii, gg in rows])
    for name, got, r in (("dq", gdq, rdq), ("dk", dk.float().cpu().numpy(), rdk),
                         ("dv", dv.float().cpu().numpy(), rdv)):
        check_close(f"{label} {name}", got, r, grad_scale(r))
    dqin = dqi.float().cpu().numpy()
    check_close(f"{label} dq_idx", dqin[rows[:, 0], rows[:, 1], rows[:, 2]], rdqi * c, float(np.abs(rdqi * c).max()))
    check_close(f"{label} dk_idx", dki.float().cpu().numpy(), rdki * c, float(np.abs(rdki * c).max()))
