"""GPU parity of the query-chunked paths: the attention forward, msa_forward,
the main backward and the alignment-loss backward run the queries in several
chunks when the caller's workspace is smaller than the designed size
(include/msa.h, workspace convention).  Small problems are forced into 2 or 3
chunks of whole 128-query blocks, and into chunks below one block with a
ragged last chunk, then compared element by element with the oracle on every
row and every key:

  - forward: selection bit-exact; out and lse within the tolerance rule of
    gpu_util.check_close; and bit-identical to the one-chunk run (each edge's
    arithmetic does not depend on which chunk it falls in);
  - main backward: dq of every row, dk and dv of every key, including keys
    selected by queries of several chunks (the first / middle / last chunk
    sums) and a key block whose gradient is split over several workgroups
    in every chunk, against the oracle's fp64 gradients;
  - alignment-loss backward: dq_idx of every row and dk_idx of every key.

Outputs and workspaces are poisoned before every call.
"""
import numpy as np
import pytest
import torch

import block_sparse_gqa_scores_amd as msa
import oracle
import synth
from gpu_util import (check_close, compare, forward_outputs, host_inputs, inputs_for, poisoned,
                      poisoned_workspace, run_device, to_u16, ws_for_chunks)

pytestmark = pytest.mark.gpu


def W(name, B, Sq, Sk, Hq, Hkv, Didx=128, topk=16, **kw):
    return synth.Workload(name, B, Sq, Sk, Hq, Hkv, index_dim=Didx, topk=topk, **kw)


# Keys near the end are selected by queries of every chunk (the local blocks
# of the last queries and the blocks the earlier ones pick).
FWD = W("chunked_fwd", 2, 1000, 1300, 16, 2, topk=6)
BWD = W("chunked_bwd", 1, 1000, 1500, 16, 2, topk=5)
KLB = W("chunked_klb", 1, 1000, 1500, 16, 2, Didx=64, topk=5)
SMALL = W("chunked_ragged", 1, 300, 700, 8, 2, topk=4)   # chunks below 128 queries


def dims(w):
    return msa.Dims.make(w.batch, w.seqlen_q, w.seqlen_k, w.heads_q, w.heads_kv, w.head_dim, w.index_dim,
                         w.block_size, w.topk)


def chunk_sizes(w, entry, counts):
    d = dims(w)
    out = []
    for n in counts:
        ws = ws_for_chunks(d, entry, n)
        assert ws is not None, f"no workspace size gives {n} chunks"
        assert msa.msa_attn_chunks(d, entry, ws) == n
        out.append(ws)
    return out


@pytest.mark.parametrize("w,counts", [(FWD, (2, 3)), (SMALL, (4, 7))], ids=["blocks", "ragged"])
def test_forward_chunked_equals_oracle_and_one_chunk(w, counts):
    t = inputs_for(w)
    one = run_device(w, t)
    p = oracle.Problem.of(w)
    h = host_inputs(t)
    rows = p.all_rows()
    ref = oracle.forward(p, h["q"], h["k"], h["v"], h["q_idx"], h["k_idx"], rows=rows)
    for n, ws in zip(counts, chunk_sizes(w, msa.ENTRY_FORWARD, counts)):
        dev = run_device(w, t, with_bm=False, ws_bytes=ws)
        msgs, stats = compare(w, dev, ref, rows, check_bm=False, label=f"{w.name} {n} chunks")
        print(f"{w.name}: {n} chunks ({ws} bytes): {stats}", flush=True)
        assert not msgs, "\n".join(msgs)
        for key in ("out", "lse", "idx"):
            assert torch.equal(dev[key], one[key]), f"{n} chunks: {key} differs from the one-chunk run"


def test_sparse_attn_fwd_chunked():
    """msa_sparse_attn_fwd itself (its own workspace) on the forward's selection."""
    w = FWD
    t = inputs_for(w)
    one = run_device(w, t, with_bm=False)
    for n, ws in zip((2, 3), chunk_sizes(w, msa.ENTRY_SPARSE_ATTN_FWD, (2, 3))):
        o = forward_outputs(w)
        out, lse = msa.msa_sparse_attn_fwd(t["q"], t["k"], t["v"], one["idx"], out=o["out"], lse=o["lse"],
                                           workspace=poisoned_workspace(ws))
        torch.cuda.synchronize()
        assert torch.equal(out, one["out"]) and torch.equal(lse, one["lse"]), f"{n} chunks"


def test_profiled_forward_records_every_chunk():
    """msa_forward_profiled with a 3-chunk workspace: 4 + 6 * 3 events, every
    pair ordered, results identical to msa_forward."""
    w = FWD
    t = inputs_for(w)
    ws = chunk_sizes(w, msa.ENTRY_FORWARD, (3,))[0]
    plain = run_device(w, t, with_bm=False, ws_bytes=ws)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(msa.n_stage_events(3))]
    for e in evs:
        e.record()
    o = forward_outputs(w)
    with pytest.raises(msa.MsaError):  # one chunk's worth of events is too few
        msa.msa_forward(t["q"], t["k"], t["v"], t["q_idx"], t["k_idx"], topk=w.topk,
                        workspace=poisoned_workspace(ws), stage_events=[e.cuda_event for e in evs[:10]], **o)
    msa.msa_forward(t["q"], t["k"], t["v"], t["q_idx"], t["k_idx"], topk=w.topk,
                    workspace=poisoned_workspace(ws), stage_events=[e.cuda_event for e in evs], **o)
    torch.cuda.synchronize()
    for key, name in (("out", "out"), ("lse", "lse"), ("idx", "block_idx")):
        assert torch.equal(o[name], plain[key]), key
    times = [evs[2 * s].elapsed_time(evs[2 * s + 1]) for s in range(len(evs) // 2)]
    assert min(times) >= 0.0
    # chunk c's stages follow chunk c - 1's
    for c in range(1, 3):
        assert evs[4 + 6 * (c - 1) + 5].elapsed_time(evs[4 + 6 * c]) >= 0.0


def _bwd(w, t, idx, out, lse, ws):
    dq, dk, dv = msa.msa_sparse_attn_bwd(
        t["q"], t["k"], t["v"], idx, out, lse, t["dout"], workspace=poisoned_workspace(ws),
        dq=poisoned(t["q"].shape, torch.bfloat16), dk=poisoned(t["k"].shape, torch.bfloat16),
        dv=poisoned(t["v"].shape, torch.bfloat16))
    torch.cuda.synchronize()
    return dq, dk, dv


def test_backward_chunked_every_key():
    w = BWD
    t = inputs_for(w)
    t["dout"] = torch.empty_like(t["q"])
    synth.fill_device(w, "dout", t["dout"])
    o = forward_outputs(w)
    out, lse, idx = msa.msa_forward(t["q"], t["k"], t["v"], t["q_idx"], t["k_idx"], topk=w.topk, **o)
    p = oracle.Problem.of(w)
    h = host_inputs(t)
    h["dout"] = to_u16(t["dout"])
    rows = p.all_rows()
    ref = oracle.forward(p, h["q"], h["k"], h["v"], h["q_idx"], h["k_idx"], rows=rows)
    assert (idx.cpu().numpy()[rows[:, 0], rows[:, 2], rows[:, 1]] == ref["sel"]).all()
    rdq, rdk, rdv = oracle.attention_bwd(p, h["q"], h["k"], h["v"], h["dout"], ref["sel"], rows)
    G = w.group
    # Blocks selected both by queries of the first 128 (always the first
    # chunk) and by the last queries (always the last chunk): their dk, dv
    # are summed across chunks.
    sel = ref["sel"]
    first, last = rows[:, 1] < 128, rows[:, 1] >= w.seqlen_q - 100
    shared = np.intersect1d(sel[first][sel[first] >= 0], sel[last][sel[last] >= 0])
    print(f"blocks selected from the first and the last chunk: {shared.tolist()}", flush=True)
    assert len(shared) > 0
    for n, ws in zip((2, 3), chunk_sizes(w, msa.ENTRY_SPARSE_ATTN_BWD, (2, 3))):
        dq, dk, dv = _bwd(w, t, idx, out, lse, ws)
        dqn = dq.float().cpu().numpy()
        check_close(f"{n} chunks dq", np.stack([dqn[b, i, g * G:(g + 1) * G] for b, i, g in rows]), rdq,
                    float(np.abs(rdq).max()))
        check_close(f"{n} chunks dk", dk.float().cpu().numpy(), rdk, float(np.abs(rdk).max()))
        check_close(f"{n} chunks dv", dv.float().cpu().numpy(), rdv, float(np.abs(rdv).max()))


# G = 32 (one query per 32-row sub-tile) with block 0 chosen by nearly every
# query: its dK, dV walk ~2000 sub-tiles in one chunk and ~1000 / ~700 per
# chunk in two / three, each more than the 512 sub-tiles after which a
# block's gradient is split over several workgroups and its fp32 parts are
# summed (first, middle and last chunk).
SPLIT = W("chunked_split", 1, 2048, 2048, 32, 1, Didx=64, topk=3, gain=True)
# Two sequences and two groups (G = 16): block 0 of every (b, g) takes ~1020
# sub-tiles in one chunk and is split; the work items span all four rows.
SPLIT_B2 = W("split_b2", 2, 2048, 2048, 32, 2, Didx=64, topk=3, gain=True)


@pytest.mark.parametrize("w,counts", [(SPLIT, (1, 2, 3)), (SPLIT_B2, (1,))], ids=["one_group", "b2_g2"])
def test_backward_split_blocks_every_key(w, counts):
    t = inputs_for(w)
    t["dout"] = torch.empty_like(t["q"])
    synth.fill_device(w, "dout", t["dout"])
    o = forward_outputs(w)
    out, lse, idx = msa.msa_forward(t["q"], t["k"], t["v"], t["q_idx"], t["k_idx"], topk=w.topk, **o)
    p = oracle.Problem.of(w)
    h = host_inputs(t)
    h["dout"] = to_u16(t["dout"])
    rows = p.all_rows()
    ref = oracle.forward(p, h["q"], h["k"], h["v"], h["q_idx"], h["k_idx"], rows=rows)
    assert (idx.cpu().numpy()[rows[:, 0], rows[:, 2], rows[:, 1]] == ref["sel"]).all()
    sel = ref["sel"]
    for a, b in ((0, 768), (768, 1536), (1536, 2048)):  # the rows of every chunk below
        m = (rows[:, 1] >= a) & (rows[:, 1] < b)
        assert (sel[m] == 0).any(axis=1).sum() > 0.95 * (b - a), f"block 0 not chosen by rows {a}..{b}"
    rdq, rdk, rdv = oracle.attention_bwd(p, h["q"], h["k"], h["v"], h["dout"], sel, rows)
    G = w.group
    d = dims(w)
    for n in counts:
        ws = msa.msa_workspace_bytes(d, msa.ENTRY_SPARSE_ATTN_BWD) if n == 1 else chunk_sizes(w, msa.ENTRY_SPARSE_ATTN_BWD, (n,))[0]
        dq, dk, dv = _bwd(w, t, idx, out, lse, ws)
        dqn = dq.float().cpu().numpy()
        check_close(f"{n} chunks dq", np.stack([dqn[b, i, g * G:(g + 1) * G] for b, i, g in rows]), rdq,
                    float(np.abs(rdq).max()))
        check_close(f"{n} chunks dk", dk.float().cpu().numpy(), rdk, float(np.abs(rdk).max()))
        check_close(f"{n} chunks dv", dv.float().cpu().numpy(), rdv, float(np.abs(rdv).max()))


def test_alignment_loss_backward_chunked_every_key():
    w = KLB
    t = inputs_for(w)
    o = forward_outputs(w)
    out, lse, idx = msa.msa_forward(t["q"], t["k"], t["v"], t["q_idx"], t["k_idx"], topk=w.topk, **o)
    loss, lse_idx = msa.msa_kl_loss_fwd(t["q"], t["k"], t["q_idx"], t["k_idx"], idx, lse, return_lse_idx=True)
    p = oracle.Problem.of(w)
    h = host_inputs(t)
    rows = p.all_rows()
    ref = oracle.forward(p, h["q"], h["k"], h["v"], h["q_idx"], h["k_idx"], rows=rows)
    rdqi, rdki, _ = oracle.kl_bwd(p, h["q"], h["k"], h["q_idx"], h["k_idx"], ref["sel"], rows)
    c = 1.0 / (w.batch * w.seqlen_q * w.heads_kv)
    rdqi, rdki = rdqi * c, rdki * c
    for n, ws in zip((2, 3), chunk_sizes(w, msa.ENTRY_KL_LOSS_BWD, (2, 3))):
        dqi, dki = msa.msa_kl_loss_bwd(t["q"], t["k"], t["q_idx"], t["k_idx"], idx, lse, lse_idx, 1.0,
                                       dq_idx=poisoned(t["q_idx"].shape, torch.bfloat16),
                                       dk_idx=poisoned(t["k_idx"].shape, torch.bfloat16),
                                       workspace=poisoned_workspace(ws))
        torch.cuda.synchronize()
        dqn = dqi.float().cpu().numpy()
        check_close(f"{n} chunks dq_idx", dqn[rows[:, 0], rows[:, 1], rows[:, 2]], rdqi, float(np.abs(rdqi).max()))
        check_close(f"{n} chunks dk_idx", dki.float().cpu().numpy(), rdki, float(np.abs(rdki).max()))


def test_workspace_below_minimum_is_rejected():
    w = SMALL
    t = inputs_for(w)
    d = dims(w)
    low = msa.msa_workspace_min_bytes(d, msa.ENTRY_FORWARD)
    with pytest.raises(msa.MsaError) as e:
        msa.msa_forward(t["q"], t["k"], t["v"], t["q_idx"], t["k_idx"], topk=w.topk,
                        workspace=poisoned_workspace(low - 256))
    assert e.value.status == 5
    # the minimum itself runs (one query per chunk) and matches the oracle
    dev = run_device(w, t, with_bm=False, ws_bytes=low)
    p = oracle.Problem.of(w)
    h = host_inputs(t)
    rows = p.all_rows()
    ref = oracle.forward(p, h["q"], h["k"], h["v"], h["q_idx"], h["k_idx"], rows=rows)
    msgs, _ = compare(w, dev, ref, rows, check_bm=False, label="minimum workspace")
    assert not msgs, "\n".join(msgs)
