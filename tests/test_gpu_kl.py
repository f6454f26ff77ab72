"""GPU parity of the alignment loss (Sparse Attention Part II, section 3.2):
msa_kl_loss_fwd through the C ABI against the oracle's per-row KL terms.

The device side runs its own forward (selection and per-head LSE) and then
the loss; the oracle computes its own selection and, from its fp64 softmax,
its own KL terms.  Selections must agree bit for bit; every row term and the
loss must lie within KL_ABS + KL_REL * |KL| of the oracle.

Tolerance.  The device forms each teacher probability from an fp32 logit and
the forward's fp32 LSE (relative error a few 1e-6 after exp2), and the row
term as sum_j (A_j - C_j + S_j (LSE - m_j)), whose pieces reach |z - LSE| of a
few hundred on these index inputs (integer rows of width 64-128): a relative
error of 1e-6 in the probabilities moves the term by up to a few 1e-4.  fp32
accumulation of 16 blocks adds about 1e-6 |KL|.  KL_ABS = 2e-3 and KL_REL =
2e-5 cover both with margin.
"""
import numpy as np
import pytest
import torch

import block_sparse_gqa_scores_amd as msa
import oracle
import synth
from gpu_util import (forward_outputs, host_inputs, inputs_for, poisoned, poisoned_workspace, spread_index_queries,
                      student_max_weight, to_u16)

pytestmark = pytest.mark.gpu

KL_ABS = 2e-3
KL_REL = 2e-5


def W(name, B, Sq, Sk, Hq, Hkv, Didx=128, topk=16, **kw):
    return synth.Workload(name, B, Sq, Sk, Hq, Hkv, index_dim=Didx, topk=topk, **kw)


def device_kl(w, t):
    """Forward, then the loss forward on poisoned outputs and workspace."""
    out, lse, idx = msa.msa_forward(t["q"], t["k"], t["v"], t["q_idx"], t["k_idx"], topk=w.topk,
                                    **forward_outputs(w))
    d = msa.dims_of(t["q"], t["k"], t["q_idx"], t["k_idx"], topk=w.topk)
    loss, rows = msa.msa_kl_loss_fwd(
        t["q"], t["k"], t["q_idx"], t["k_idx"], idx, lse, loss=poisoned((), torch.float32),
        rows=poisoned((w.batch, w.heads_kv, w.seqlen_q), torch.float32),
        workspace=poisoned_workspace(msa.msa_workspace_bytes(d, msa.ENTRY_KL_LOSS_FWD)))
    torch.cuda.synchronize()
    return idx, lse, loss, rows


def check_rows(w, h, idx, kl_dev, rows, label):
    p = oracle.Problem.of(w)
    ref = oracle.forward(p, h["q"], h["k"], h["v"], h["q_idx"], h["k_idx"], rows=rows)
    b, i, g = rows[:, 0], rows[:, 1], rows[:, 2]
    got_sel = idx[b, g, i]
    bad = (got_sel != ref["sel"]).any(axis=1)
    assert not bad.any(), f"{label}: selection differs on {int(bad.sum())} rows"
    exp = oracle.kl_rows(p, h["q"], h["k"], h["q_idx"], h["k_idx"], ref["sel"], rows)
    got = kl_dev[b, g, i].astype(np.float64)
    err = np.abs(got - exp)
    tol = KL_ABS + KL_REL * np.abs(exp)
    r = int(np.argmax(err / tol))
    print(f"{label}: {len(rows)} rows, KL range [{exp.min():.4g}, {exp.max():.4g}], "
          f"max err {err.max():.3e}, worst row {rows[r].tolist()} {got[r]:.6g} vs {exp[r]:.6g}", flush=True)
    assert (err <= tol).all(), f"{label}: KL error {err[r]:.3e} > {tol[r]:.3e} at row {rows[r].tolist()}"
    return exp


CASES = [
    W("kl_4k", 1, 4096, 4096, 8, 2, Didx=64),                  # two query windows
    W("kl_ragged", 2, 700, 1000, 8, 2, topk=5),                # S_k % 128 != 0, S_q < S_k
    W("kl_gqa8", 1, 2600, 2600, 64, 8),                        # G = 8
    W("kl_mha", 1, 600, 777, 4, 4, Didx=64, topk=3),           # G = 1
    W("kl_g2", 1, 500, 1300, 8, 4, topk=6),                    # G = 2
    W("kl_g4", 1, 500, 1300, 8, 2, Didx=64, topk=6),           # G = 4
    W("kl_g16", 1, 500, 640, 32, 2, topk=2),                   # G = 16
    W("kl_g32", 2, 300, 300, 32, 1, Didx=64, topk=4),          # G = 32
    W("kl_topk1", 1, 400, 900, 8, 2, topk=1),                  # local block only
    W("kl_decode", 3, 1, 5000, 16, 2, Didx=64),                # S_q = 1
    W("kl_k64", 1, 130, 9000, 4, 1, topk=64),                  # the largest topk
    W("kl_gain", 1, 1500, 3000, 16, 2, gain=True, topk=6),     # uneven blocks
]


def sample(w, limit=3000, seed=0):
    p = oracle.Problem.of(w)
    rows = p.all_rows()
    if len(rows) <= limit:
        return rows
    rng = np.random.default_rng(seed)
    keep = np.unique(np.concatenate([rng.choice(len(rows), limit, replace=False),
                                     np.arange(len(rows) - 64, len(rows)), np.arange(64)]))
    return rows[keep]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_kl_parity(w):
    t = inputs_for(w)
    idx, lse, loss, kl_dev = device_kl(w, t)
    h = host_inputs(t)
    rows = sample(w)
    check_rows(w, h, idx.cpu().numpy(), kl_dev.cpu().numpy(), rows, w.name)
    # The loss is the mean of the row terms (all rows, in fixed order).
    full = kl_dev.double().mean().item()
    assert abs(loss.item() - full) <= 1e-6 * (1 + abs(full)), (loss.item(), full)
    if len(rows) == w.batch * w.seqlen_q * w.heads_kv:
        exp_loss = oracle.kl_rows(oracle.Problem.of(w), h["q"], h["k"], h["q_idx"], h["k_idx"],
                                  idx.cpu().numpy()[rows[:, 0], rows[:, 2], rows[:, 1]], rows).mean()
        assert abs(loss.item() - exp_loss) <= KL_ABS + KL_REL * abs(exp_loss)


SPREAD = [
    W("kl_spread_g2", 1, 900, 2600, 8, 4, topk=8),            # G = 2
    W("kl_spread_g8", 1, 700, 3000, 64, 8, topk=12),          # G = 8 (16x16x32 index tiles)
    W("kl_spread_g8_d64", 2, 300, 2200, 16, 2, Didx=64),      # G = 8, D_idx 64, whole prefix selected
]


@pytest.mark.parametrize("w", SPREAD, ids=lambda w: w.name)
def test_kl_parity_spread_student(w):
    """A student that is not nearly one-hot (index rows with two +-1 channels,
    spread_index_queries): the non-dominant mass of the index softmax (the
    L, S and C sums of every block, not only the top token) now carries the
    row terms, and every row is compared with the oracle."""
    t = spread_index_queries(w, inputs_for(w))
    idx, lse, loss, kl_dev = device_kl(w, t)
    h = host_inputs(t)
    rows = oracle.Problem.of(w).all_rows()
    sel = idx.cpu().numpy()[rows[:, 0], rows[:, 2], rows[:, 1]]
    pick = rows[:: max(1, len(rows) // 200)]
    mw = student_max_weight(w, h, idx.cpu().numpy()[pick[:, 0], pick[:, 2], pick[:, 1]], pick)
    late = pick[:, 1] + w.seqlen_k - w.seqlen_q >= 1024   # rows that see at least 1024 tokens
    print(f"{w.name}: student max weight median {np.median(mw[late]):.4f}, max {mw[late].max():.4f}", flush=True)
    assert np.median(mw[late]) < 0.05
    exp = check_rows(w, h, idx.cpu().numpy(), kl_dev.cpu().numpy(), rows, w.name)
    assert abs(loss.item() - exp.mean()) <= KL_ABS + KL_REL * abs(exp.mean())
    del sel


def test_kl_caller_selection_unsorted_with_holes():
    """A caller-made selection (unsorted, -1 in the middle) with the LSE of
    msa_sparse_attn_fwd on that same selection."""
    w = W("kl_caller", 2, 200, 2000, 8, 2, topk=6)
    t = inputs_for(w)
    rng = np.random.default_rng(5)
    B, Hkv, Sq, k = 2, 2, 200, 6
    sel = np.full((B, Hkv, Sq, k), -1, dtype=np.int32)
    for b in range(B):
        for g in range(Hkv):
            for i in range(Sq):
                local = (i + 1800) // 128
                others = rng.choice(local, size=min(local, rng.integers(0, k)), replace=False)
                row = np.concatenate([others, [local]])
                sel[b, g, i, rng.choice(k, size=len(row), replace=False)] = row
    idx = torch.from_numpy(sel).cuda()
    _, lse = msa.msa_sparse_attn_fwd(t["q"], t["k"], t["v"], idx, return_lse=True)
    loss, rows_dev = msa.msa_kl_loss_fwd(t["q"], t["k"], t["q_idx"], t["k_idx"], idx, lse, return_rows=True)
    torch.cuda.synchronize()
    p = oracle.Problem.of(w)
    h = host_inputs(t)
    rows = p.all_rows()
    exp = oracle.kl_rows(p, h["q"], h["k"], h["q_idx"], h["k_idx"], sel[rows[:, 0], rows[:, 2], rows[:, 1]], rows)
    got = rows_dev.cpu().numpy()[rows[:, 0], rows[:, 2], rows[:, 1]].astype(np.float64)
    assert (np.abs(got - exp) <= KL_ABS + KL_REL * np.abs(exp)).all(), np.abs(got - exp).max()
    assert abs(loss.item() - exp.mean()) <= KL_ABS + KL_REL * abs(exp.mean())


def test_kl_teacher_equals_student_is_zero():
    """G = 1, q_idx = Q * scale and k_idx = K with Q, K integer-valued: the
    index logits equal the head's scaled logits exactly, so every term is 0
    up to rounding (the identity KL(p || p) = 0 on the device)."""
    w = W("kl_self", 1, 300, 900, 2, 2, topk=4)
    t = inputs_for(w)
    q = torch.randint(-2, 3, t["q"].shape, device="cuda").to(torch.bfloat16)
    k1 = torch.randint(-2, 3, (1, 900, 1, 128), device="cuda").to(torch.bfloat16)
    k = k1.expand(1, 900, 2, 128).contiguous()
    scale = 0.0625  # exact in bf16; logits scale * q.k are exact in fp32
    q_idx = (q.float() * scale).to(torch.bfloat16).contiguous()
    k_idx = k1.reshape(1, 900, 128).contiguous()
    out, lse, idx = msa.msa_forward(q, k, t["v"], q_idx, k_idx, topk=4, softmax_scale=scale,
                                    return_lse=True, return_idx=True)
    loss, rows = msa.msa_kl_loss_fwd(q, k, q_idx, k_idx, idx, lse, softmax_scale=scale, return_rows=True)
    torch.cuda.synchronize()
    assert rows.abs().max().item() < 1e-3 and abs(loss.item()) < 1e-4


def test_kl_deterministic_and_workspace_reuse():
    w = W("kl_det", 1, 1500, 4000, 16, 2, topk=8)
    t = inputs_for(w)
    idx, lse, loss, rows = device_kl(w, t)
    ws = torch.empty(msa.msa_workspace_bytes(msa.dims_of(t["q"], t["k"], t["q_idx"], t["k_idx"], topk=8),
                                             msa.ENTRY_KL_LOSS_FWD), dtype=torch.uint8, device="cuda")
    ws.fill_(0xAB)  # stale contents do not matter
    for _ in range(2):
        l2, r2 = msa.msa_kl_loss_fwd(t["q"], t["k"], t["q_idx"], t["k_idx"], idx, lse, return_rows=True,
                                     workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(l2, loss) and torch.equal(r2, rows)


def test_kl_empty_problem_writes_zero_loss():
    loss = torch.full((4,), 7.0, device="cuda")
    d = msa.Dims.make(0, 0, 0, 8, 2)
    rc = msa.lib().msa_kl_loss_fwd(d, None, None, None, None, None, None, None,
                                   loss.data_ptr(), None, None, 0, None)
    torch.cuda.synchronize()
    assert rc == 0 and loss[0].item() == 0.0 and loss[1].item() == 7.0


def test_kl_prefill_32k_sampled_rows():
    """The 32K workload in the configuration the benchmark times, on rows the
    oracle computes one by one; the loss equals the mean of all row terms."""
    w = synth.WORKLOADS["prefill_32k"]
    print("[prefill_32k] inputs + forward + loss", flush=True)
    t = inputs_for(w)
    idx, lse, loss, kl_dev = device_kl(w, t)
    full = kl_dev.double().mean().item()
    assert abs(loss.item() - full) <= 1e-6 * (1 + abs(full))
    assert torch.isfinite(kl_dev).all() and (kl_dev > -KL_ABS).all()
    h = host_inputs(t)
    del t
    rng = np.random.default_rng(2)
    qs = np.unique(np.concatenate([rng.integers(0, w.seqlen_q, 40), [0, 127, 2047, 2048, w.seqlen_q - 1]]))
    rows = np.array([(0, q, g) for q in qs for g in range(w.heads_kv)], dtype=np.int64)
    print(f"[prefill_32k] oracle on {len(rows)} rows", flush=True)
    check_rows(w, h, idx.cpu().numpy(), kl_dev.cpu().numpy(), rows, "prefill_32k")
