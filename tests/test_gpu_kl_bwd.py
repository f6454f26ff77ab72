"""GPU parity of the alignment loss's backward (msa_kl_loss_bwd through the C
ABI) against the oracle's gradients with respect to the index inputs (teacher
detached, Sparse Attention Part II, section 3.2).

The device side runs its own forward (selection and LSE), the loss forward
(which also returns each row's log-sum-exp of the index scores), then the
backward with grad_loss = 1; the oracle computes its own selection and, in
fp64, the unscaled gradients, scaled here by 1 / (B S_q H_kv).

Tolerance: the one rule of gpu_util.check_close with s = max |ref| of the
tensor (the error beyond the output's own bf16 rounding at most 1e-2 s, the
mean error at most 1e-3 s).  The device rounds g to bf16 before the matrix
products (relative 2^-9 per term), accumulates in fp32 and keeps each edge's
dq_idx as fp16 scaled by its 32-dim quarter's maximum (2^-12).  The rows'
index-score log-sum-exps must agree to 1e-6 relative (fp32 against fp64).
Outputs and workspaces are poisoned before every call.
"""
import numpy as np
import pytest
import torch

import block_sparse_gqa_scores_amd as msa
import oracle
import synth
from gpu_util import (check_close, forward_outputs, host_inputs, inputs_for, poisoned, poisoned_workspace,
                      spread_index_queries, student_max_weight, to_u16)

pytestmark = pytest.mark.gpu


def W(name, B, Sq, Sk, Hq, Hkv, Didx=128, topk=16, **kw):
    return synth.Workload(name, B, Sq, Sk, Hq, Hkv, index_dim=Didx, topk=topk, **kw)


def device_kl_bwd(w, t, grad=1.0, ws_bytes=None):
    """Forward, loss forward and loss backward on poisoned outputs and
    workspaces; ws_bytes sizes the backward's workspace (None: designed)."""
    out, lse, idx = msa.msa_forward(t["q"], t["k"], t["v"], t["q_idx"], t["k_idx"], topk=w.topk,
                                    **forward_outputs(w))
    d = msa.dims_of(t["q"], t["k"], t["q_idx"], t["k_idx"], topk=w.topk)
    loss, lse_idx = msa.msa_kl_loss_fwd(
        t["q"], t["k"], t["q_idx"], t["k_idx"], idx, lse,
        lse_idx=poisoned((w.batch, w.heads_kv, w.seqlen_q), torch.float32),
        workspace=poisoned_workspace(msa.msa_workspace_bytes(d, msa.ENTRY_KL_LOSS_FWD)))
    nbytes = msa.msa_workspace_bytes(d, msa.ENTRY_KL_LOSS_BWD) if ws_bytes is None else ws_bytes
    dqi, dki = msa.msa_kl_loss_bwd(t["q"], t["k"], t["q_idx"], t["k_idx"], idx, lse, lse_idx, grad,
                                   dq_idx=poisoned(t["q_idx"].shape, torch.bfloat16),
                                   dk_idx=poisoned(t["k_idx"].shape, torch.bfloat16),
                                   workspace=poisoned_workspace(nbytes))
    torch.cuda.synchronize()
    return idx, lse_idx, dqi, dki


def check(name, got, ref):
    return check_close(name, got, ref, float(np.abs(ref).max()))


def oracle_side(w, h, rows, want_dk=True, threads=0):
    p = oracle.Problem.of(w)
    ref = oracle.forward(p, h["q"], h["k"], h["v"], h["q_idx"], h["k_idx"], rows=rows, threads=threads)
    dqi, dki, lse_z = oracle.kl_bwd(p, h["q"], h["k"], h["q_idx"], h["k_idx"], ref["sel"], rows,
                                    want_dk=want_dk, threads=threads)
    c = 1.0 / (w.batch * w.seqlen_q * w.heads_kv)
    return ref["sel"], dqi * c, (dki * c if dki is not None else None), lse_z


CASES = [
    W("klb_4k", 1, 4096, 4096, 8, 2, Didx=64),                 # two query windows, D_idx 64
    W("klb_ragged", 2, 700, 1000, 8, 2, topk=5),               # S_k % 128 != 0, S_q < S_k
    W("klb_gqa8", 1, 2600, 2600, 64, 8),                       # G = 8
    W("klb_mha", 1, 600, 777, 4, 4, Didx=64, topk=3),          # G = 1
    W("klb_g2", 1, 500, 1300, 8, 4, topk=6),                   # G = 2
    W("klb_g16", 1, 500, 640, 32, 2, topk=2),                  # G = 16
    W("klb_g32", 2, 300, 300, 32, 1, Didx=64, topk=4),         # G = 32
    W("klb_topk1", 1, 400, 900, 8, 2, topk=1),                 # local block only
    W("klb_decode", 3, 1, 5000, 16, 2, Didx=64),               # S_q = 1
    W("klb_k64", 1, 130, 9000, 4, 1, topk=64),                 # the largest topk
    W("klb_gain", 1, 1500, 3000, 16, 2, gain=True, topk=6),    # uneven blocks
    W("klb_hkv12", 1, 400, 900, 12, 12, Didx=64, topk=4),     # H_kv = 12: dk_idx sums groups in two batches
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_kl_bwd_parity(w):
    t = inputs_for(w)
    idx, lse_idx, dqi, dki = device_kl_bwd(w, t)
    h = {n: to_u16(x) for n, x in t.items()}
    rows = oracle.Problem.of(w).all_rows()
    sel, rdqi, rdki, lse_z = oracle_side(w, h, rows)
    got_sel = idx.cpu().numpy()[rows[:, 0], rows[:, 2], rows[:, 1]]
    assert (got_sel == sel).all(), "selection differs"
    li = lse_idx.cpu().numpy()[rows[:, 0], rows[:, 2], rows[:, 1]].astype(np.float64)
    assert np.abs(li - lse_z).max() <= 1e-6 * max(1.0, np.abs(lse_z).max()), np.abs(li - lse_z).max()
    dqin = dqi.float().cpu().numpy()
    check(f"{w.name} dq_idx", dqin[rows[:, 0], rows[:, 1], rows[:, 2]], rdqi)
    check(f"{w.name} dk_idx", dki.float().cpu().numpy(), rdki)


SPREAD = [
    W("klb_spread_g2", 1, 900, 2600, 8, 4, topk=8),           # G = 2
    W("klb_spread_g8", 1, 700, 3000, 64, 8, topk=12),         # G = 8
    W("klb_spread_g8_d64", 2, 300, 2200, 16, 2, Didx=64),     # G = 8, D_idx 64
]


@pytest.mark.parametrize("w", SPREAD, ids=lambda w: w.name)
def test_kl_bwd_parity_spread_student(w):
    """The gradient g = c (P_idx - P) with a spread student (two +-1 channels
    per index row): P_idx of every token, not only the top one, enters dq_idx
    and dk_idx; compared with the oracle on every row and key."""
    t = spread_index_queries(w, inputs_for(w))
    idx, lse_idx, dqi, dki = device_kl_bwd(w, t)
    h = host_inputs(t)
    rows = oracle.Problem.of(w).all_rows()
    sel, rdqi, rdki, lse_z = oracle_side(w, h, rows)
    assert (idx.cpu().numpy()[rows[:, 0], rows[:, 2], rows[:, 1]] == sel).all(), "selection differs"
    pick = rows[:: max(1, len(rows) // 200)]
    mw = student_max_weight(w, h, idx.cpu().numpy()[pick[:, 0], pick[:, 2], pick[:, 1]], pick)
    late = pick[:, 1] + w.seqlen_k - w.seqlen_q >= 1024
    print(f"{w.name}: student max weight median {np.median(mw[late]):.4f}", flush=True)
    assert np.median(mw[late]) < 0.05
    li = lse_idx.cpu().numpy()[rows[:, 0], rows[:, 2], rows[:, 1]].astype(np.float64)
    assert np.abs(li - lse_z).max() <= 1e-6 * max(1.0, np.abs(lse_z).max()), np.abs(li - lse_z).max()
    dqin = dqi.float().cpu().numpy()
    check(f"{w.name} dq_idx", dqin[rows[:, 0], rows[:, 1], rows[:, 2]], rdqi)
    check(f"{w.name} dk_idx", dki.float().cpu().numpy(), rdki)


def test_kl_bwd_grad_scale_and_determinism():
    """grad_loss scales the gradients linearly (2^k exactly); repeated calls
    are bit-identical."""
    w = W("klb_det", 1, 1500, 4000, 16, 2, topk=8)
    t = inputs_for(w)
    a = device_kl_bwd(w, t, 1.0)
    b = device_kl_bwd(w, t, 1.0)
    c = device_kl_bwd(w, t, 4.0)
    assert torch.equal(a[2], b[2]) and torch.equal(a[3], b[3])
    assert torch.equal(c[2].float(), 4 * a[2].float()) and torch.equal(c[3].float(), 4 * a[3].float())


def test_kl_bwd_without_queries_writes_zero_key_gradient():
    dki = torch.full((2, 300, 64), 3.0, dtype=torch.bfloat16, device="cuda")
    d = msa.Dims.make(2, 0, 300, 8, 2, index_dim=64)
    rc = msa.lib().msa_kl_loss_bwd(d, None, None, None, None, None, None, None, 1.0, None,
                                   dki.data_ptr(), None, 0, None)
    torch.cuda.synchronize()
    assert rc == 0 and not dki.float().any()


def test_kl_bwd_prefill_32k():
    """Full size: dq_idx on sampled rows; dk_idx of the last two key blocks,
    whose rows (all groups) are all among the last 256 queries; and, over all
    keys, sum_s dk_idx[s] = 0 (student and teacher both sum to one on every
    row)."""
    w = synth.WORKLOADS["prefill_32k"]
    print("[prefill_32k] inputs, forward, loss, backward", flush=True)
    t = inputs_for(w)
    idx, lse_idx, dqi, dki = device_kl_bwd(w, t)
    tot = dki.float()[0].sum(0)
    scale = dki.float()[0].abs().sum(0)
    print(f"[prefill_32k] |sum dk_idx| max {tot.abs().max().item():.3e} (sum |dk_idx| {scale.max().item():.3e})",
          flush=True)
    assert (tot.abs() <= 4e-3 * scale + 1e-12).all()
    rng = np.random.default_rng(4)
    qs = np.unique(np.concatenate([rng.integers(0, w.seqlen_q, 24), [0, 127, 2047, 2048],
                                   np.arange(w.seqlen_q - 256, w.seqlen_q)]))
    rows = np.array([(0, q, g) for q in qs for g in range(w.heads_kv)], dtype=np.int64)
    h = {n: to_u16(x) for n, x in t.items()}
    dqin, dkin, sel_dev = dqi.float().cpu().numpy(), dki.float().cpu().numpy(), idx.cpu().numpy()
    del t
    print(f"[prefill_32k] oracle on {len(rows)} rows", flush=True)
    sel, rdqi, rdki, _ = oracle_side(w, h, rows, threads=8)
    assert (sel_dev[rows[:, 0], rows[:, 2], rows[:, 1]] == sel).all()
    check("prefill_32k dq_idx", dqin[rows[:, 0], rows[:, 1], rows[:, 2]], rdqi)
    lo = (w.n_blk - 2) * 128
    check("prefill_32k dk_idx (last 2 blocks)", dkin[0, lo:], rdki[0, lo:])
