"""GPU parity of the main-branch backward (msa_sparse_attn_bwd through the C
ABI) against the oracle's gradients.

The device side runs its own forward (selection, output, LSE) and then the
backward on a seeded upstream gradient dO; the oracle computes its own
selection and, in fp64, dq of each row and dk, dv summed over the rows.

Tolerance: the one rule of gpu_util.check_close with s = max |ref| of the
tensor (the error beyond the output's own bf16 rounding at most 1e-2 s, the
mean error at most 1e-3 s).  The device feeds P and dS to the matrix cores in
bf16 (relative error 2^-9 per element, averaging out over the 128 keys of a
block and the rows that meet at a key), accumulates in fp32, and keeps each
edge's dq as fp16 scaled by the maximum of its 32-dim quarter (2^-12 of that
maximum).  Outputs and workspaces are poisoned before every call.

Full-size workloads are checked on rows the oracle computes one by one (dq),
on the last key blocks (whose rows are all among the last queries, so their
dk, dv are complete from those rows), and everywhere through identities that
hold at any size: per group, the keys' dk sum to zero and the keys' dv sum to
the group's dO rows (each softmax row sums to one).
"""
import gc

import numpy as np
import pytest
import torch

import block_sparse_gqa_scores_amd as msa
import oracle
import synth
from gpu_util import check_close, forward_outputs, inputs_for, poisoned, poisoned_workspace, to_u16

pytestmark = pytest.mark.gpu


def W(name, B, Sq, Sk, Hq, Hkv, Didx=128, topk=16, **kw):
    return synth.Workload(name, B, Sq, Sk, Hq, Hkv, index_dim=Didx, topk=topk, **kw)


def device_bwd(w, t, ws_bytes=None):
    """Forward, then the backward on poisoned outputs and workspace; ws_bytes
    sizes the backward's workspace (None: the designed size)."""
    out, lse, idx = msa.msa_forward(t["q"], t["k"], t["v"], t["q_idx"], t["k_idx"], topk=w.topk,
                                    **forward_outputs(w))
    d = msa.dims_of(t["q"], t["k"], topk=w.topk)
    nbytes = msa.msa_workspace_bytes(d, msa.ENTRY_SPARSE_ATTN_BWD) if ws_bytes is None else ws_bytes
    dq, dk, dv = msa.msa_sparse_attn_bwd(
        t["q"], t["k"], t["v"], idx, out, lse, t["dout"], workspace=poisoned_workspace(nbytes),
        dq=poisoned(t["q"].shape, torch.bfloat16), dk=poisoned(t["k"].shape, torch.bfloat16),
        dv=poisoned(t["v"].shape, torch.bfloat16))
    torch.cuda.synchronize()
    return idx, dq, dk, dv


def check(name, got, ref):
    return check_close(name, got, ref, float(np.abs(ref).max()))


def compare_all(w, t, idx, dq, dk, dv, rows=None):
    p = oracle.Problem.of(w)
    rows = p.all_rows() if rows is None else rows
    h = {n: to_u16(x) for n, x in t.items()}
    ref = oracle.forward(p, h["q"], h["k"], h["v"], h["q_idx"], h["k_idx"], rows=rows)
    got_sel = idx.cpu().numpy()[rows[:, 0], rows[:, 2], rows[:, 1]]
    assert (got_sel == ref["sel"]).all(), "selection differs"
    rdq, rdk, rdv = oracle.attention_bwd(p, h["q"], h["k"], h["v"], h["dout"], ref["sel"], rows)
    G = w.group
    dqn = dq.float().cpu().numpy()
    gdq = np.stack([dqn[bb, ii, gg * G:(gg + 1) * G] for bb, ii, gg in rows])
    check(f"{w.name} dq", gdq, rdq)
    return rdk, rdv


CASES = [
    W("bwd_4k", 1, 4096, 4096, 8, 2, Didx=64),                 # two query windows
    W("bwd_ragged", 2, 700, 1000, 8, 2, topk=5),               # S_k % 128 != 0, S_q < S_k
    W("bwd_gqa8", 1, 2600, 2600, 64, 8),                       # G = 8
    W("bwd_mha", 1, 600, 777, 4, 4, Didx=64, topk=3),          # G = 1
    W("bwd_g2", 1, 500, 1300, 8, 4, topk=6),                   # G = 2
    W("bwd_g16", 1, 500, 640, 32, 2, topk=2),                  # G = 16
    W("bwd_g32", 2, 300, 300, 32, 1, Didx=64, topk=4),         # G = 32
    W("bwd_topk1", 1, 400, 900, 8, 2, topk=1),                 # local block only
    W("bwd_decode", 3, 1, 5000, 16, 2, Didx=64),               # S_q = 1
    W("bwd_k64", 1, 130, 9000, 4, 1, topk=64),                 # the largest topk
    W("bwd_scale", 1, 300, 1400, 8, 4, topk=4),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_bwd_parity(w):
    t = inputs_for(w)
    synth.fill_device(w, "dout", t.setdefault("dout", torch.empty_like(t["q"])))
    idx, dq, dk, dv = device_bwd(w, t)
    rdk, rdv = compare_all(w, t, idx, dq, dk, dv)
    check(f"{w.name} dk", dk.float().cpu().numpy(), rdk)
    check(f"{w.name} dv", dv.float().cpu().numpy(), rdv)


def test_bwd_deterministic():
    w = W("bwd_det", 1, 1500, 4000, 16, 2, topk=8)
    t = inputs_for(w)
    t["dout"] = torch.empty_like(t["q"])
    synth.fill_device(w, "dout", t["dout"])
    a = device_bwd(w, t)
    b = device_bwd(w, t)
    for x, y, n in zip(a[1:], b[1:], ("dq", "dk", "dv")):
        assert torch.equal(x, y), n


def test_bwd_unselected_keys_get_zero():
    """Keys of blocks no query selects have zero gradients (topk = 2 on a long
    prefix leaves most blocks unselected)."""
    w = W("bwd_zero", 1, 64, 20000, 8, 2, topk=2)
    t = inputs_for(w)
    t["dout"] = torch.empty_like(t["q"])
    synth.fill_device(w, "dout", t["dout"])
    idx, dq, dk, dv = device_bwd(w, t)
    used = np.zeros((2, w.n_blk), dtype=bool)
    sel = idx.cpu().numpy()[0]
    for g in range(2):
        used[g, sel[g][sel[g] >= 0]] = True
    dkn, dvn = dk.float().cpu().numpy()[0], dv.float().cpu().numpy()[0]
    for g in range(2):
        for j in np.flatnonzero(~used[g])[:50]:
            assert not dkn[j * 128:(j + 1) * 128, g].any() and not dvn[j * 128:(j + 1) * 128, g].any()


def test_bwd_without_queries_writes_zero_key_gradients():
    """seqlen_q = 0 with keys present: no row selects anything, dk = dv = 0."""
    dk = torch.full((2, 300, 2, 128), 3.0, dtype=torch.bfloat16, device="cuda")
    dv = torch.full_like(dk, 5.0)
    d = msa.Dims.make(2, 0, 300, 8, 2)
    rc = msa.lib().msa_sparse_attn_bwd(d, None, None, None, None, None, None, None, None,
                                       dk.data_ptr(), dv.data_ptr(), None, 0, None)
    torch.cuda.synchronize()
    assert rc == 0 and not dk.float().any() and not dv.float().any()


def release():
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["prefill_32k", "prefill_128k_gain"])
def test_bwd_workload(name):
    """Full size, in the configuration a training step would call: sampled dq
    rows, the last two key blocks' dk and dv (complete from the last 256
    queries' rows, 32K only), and the sum identities on every group; the
    several-chunk paths are checked on every key in test_gpu_chunks.py)."""
    w = synth.WORKLOADS[name]
    print(f"[{name}] inputs, forward, backward", flush=True)
    t = inputs_for(w)
    t["dout"] = torch.empty_like(t["q"])
    synth.fill_device(w, "dout", t["dout"])
    idx, dq, dk, dv = device_bwd(w, t)
    G = w.group
    # Identities over all keys of each group.
    do_sum = t["dout"].float().reshape(w.seqlen_q, w.heads_kv, G, w.head_dim).sum((0, 2))
    dv_sum = dv.float()[0].sum(0)
    dk_sum = dk.float()[0].sum(0)
    dv_scale = dv.float().abs().sum(1)[0]
    dk_scale = dk.float().abs().sum(1)[0]
    print(f"[{name}] identities: |sum dv - sum dO| max {(dv_sum - do_sum).abs().max().item():.3e} "
          f"(sum |dv| {dv_scale.max().item():.3e}); |sum dk| max {dk_sum.abs().max().item():.3e} "
          f"(sum |dk| {dk_scale.max().item():.3e})", flush=True)
    # bf16 rounding of each key's gradient alone is up to 2^-9 of it.
    assert ((dv_sum - do_sum).abs() <= 4e-3 * dv_scale + 1e-2).all()
    assert (dk_sum.abs() <= 4e-3 * dk_scale + 1e-2).all()
    rng = np.random.default_rng(3)
    qs = np.unique(np.concatenate([rng.integers(0, w.seqlen_q, 24), [0, 127, 2047, 2048]]))
    tail = w.seqlen_q - 256 if name == "prefill_32k" else w.seqlen_q - 8
    qs = np.unique(np.concatenate([qs, np.arange(tail, w.seqlen_q)]))
    rows = np.array([(0, q, g) for q in qs for g in range(w.heads_kv)], dtype=np.int64)
    h = {n: to_u16(x) for n, x in t.items()}
    dkn = dk.float().cpu().numpy() if name == "prefill_32k" else None
    dvn = dv.float().cpu().numpy() if name == "prefill_32k" else None
    dqn = dq.float().cpu().numpy()
    sel_dev = idx.cpu().numpy()
    del t, dq, dk, dv
    release()
    p = oracle.Problem.of(w)
    print(f"[{name}] oracle on {len(rows)} rows", flush=True)
    ref = oracle.forward(p, h["q"], h["k"], h["v"], h["q_idx"], h["k_idx"], rows=rows)
    assert (sel_dev[rows[:, 0], rows[:, 2], rows[:, 1]] == ref["sel"]).all()
    want = name == "prefill_32k"
    rdq, rdk, rdv = oracle.attention_bwd(p, h["q"], h["k"], h["v"], h["dout"], ref["sel"], rows, want_dkv=want,
                                         threads=8)
    check(f"{name} dq", np.stack([dqn[0, q, g * G:(g + 1) * G] for _, q, g in rows]), rdq)
    if want:
        lo = (w.n_blk - 2) * 128
        check(f"{name} dk (last 2 blocks)", dkn[0, lo:], rdk[0, lo:])
        check(f"{name} dv (last 2 blocks)", dvn[0, lo:], rdv[0, lo:])
