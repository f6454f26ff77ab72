"""Pins of the oracle's gradients: the main branch's dq, dk, dv given dO, and
the alignment term's gradient with respect to the index inputs (teacher held
fixed, Sparse Attention Part II, section 3.2).

Checks against facts the gradient code does not contain: central finite
differences of the (separately pinned) forward functions on fp64 inputs,
torch autograd of dense causal attention and of torch's kl_div when the
selection covers the whole prefix, and identities that hold at any size
(softmax rows sum to one, so the key gradients of a group sum to zero and its
value gradients sum to the group's dO).
"""
import numpy as np
import pytest
import torch

import oracle
import synth


def random_selection(p, rng, rows=None):
    rows = p.all_rows() if rows is None else rows
    sel = np.full((len(rows), p.topk), -1, dtype=np.int32)
    for r, (b, i, g) in enumerate(rows):
        local = (i + p.seqlen_k - p.seqlen_q) // p.block_size
        n = min(local, p.topk - 1, rng.integers(0, p.topk))
        pick = sorted(rng.choice(local, size=n, replace=False).tolist()) if n else []
        sel[r, :n + 1] = pick + [local]
    return rows, sel


def small(rng, B=1, Sq=10, Sk=21, Hq=4, Hkv=2, D=6, Didx=5, bs=4, k=3, scale=0.0):
    p = oracle.Problem(B, Sq, Sk, Hq, Hkv, D, Didx, block_size=bs, topk=k, softmax_scale=scale)
    x = dict(q=rng.normal(size=(B, Sq, Hq, D)), k=rng.normal(size=(B, Sk, Hkv, D)),
             v=rng.normal(size=(B, Sk, Hkv, D)), dout=rng.normal(size=(B, Sq, Hq, D)),
             q_idx=rng.normal(size=(B, Sq, Hkv, Didx)), k_idx=rng.normal(size=(B, Sk, Didx)))
    rows, sel = random_selection(p, rng)
    return p, x, rows, sel


def loss_attn(p, x, rows, sel):
    out, _ = oracle.attention(p, x["q"], x["k"], x["v"], sel, rows)
    G = p.group
    do = np.stack([x["dout"][b, i, g * G:(g + 1) * G] for b, i, g in rows])
    return float((out * do).sum())


def fd(f, arr, idx, eps=1e-6):
    old = arr[idx]
    arr[idx] = old + eps
    up = f()
    arr[idx] = old - eps
    dn = f()
    arr[idx] = old
    return (up - dn) / (2 * eps)


@pytest.mark.parametrize("scale", [0.0, 0.7])
def test_attention_grads_match_finite_differences(oracle_mod, scale):
    """L = sum dO . O over all rows; dL/dq, dL/dk, dL/dv at random coordinates."""
    rng = np.random.default_rng(21)
    p, x, rows, sel = small(rng, scale=scale)
    dq, dk, dv = oracle.attention_bwd(p, x["q"], x["k"], x["v"], x["dout"], sel, rows)
    G = p.group
    f = lambda: loss_attn(p, x, rows, sel)
    for _ in range(12):
        b, i, h, c = (rng.integers(0, n) for n in x["q"].shape)
        r = int(np.flatnonzero((rows[:, 0] == b) & (rows[:, 1] == i) & (rows[:, 2] == h // G))[0])
        assert dq[r, h % G, c] == pytest.approx(fd(f, x["q"], (b, i, h, c)), rel=1e-6, abs=1e-8)
    for _ in range(12):
        idx = tuple(rng.integers(0, n) for n in x["k"].shape)
        assert dk[idx] == pytest.approx(fd(f, x["k"], idx), rel=1e-6, abs=1e-8)
        assert dv[idx] == pytest.approx(fd(f, x["v"], idx), rel=1e-6, abs=1e-8)


def test_kl_grads_match_finite_differences(oracle_mod):
    """L = sum of the KL terms over all rows, teacher fixed: dL/dq_idx and
    dL/dk_idx at random coordinates (the teacher does not depend on them)."""
    rng = np.random.default_rng(22)
    p, x, rows, sel = small(rng)
    dqi, dki, lse_z = oracle.kl_bwd(p, x["q"], x["k"], x["q_idx"], x["k_idx"], sel, rows)
    f = lambda: float(oracle.kl_rows(p, x["q"], x["k"], x["q_idx"], x["k_idx"], sel, rows).sum())
    for _ in range(12):
        b, i, g, c = (rng.integers(0, n) for n in x["q_idx"].shape)
        r = int(np.flatnonzero((rows[:, 0] == b) & (rows[:, 1] == i) & (rows[:, 2] == g))[0])
        assert dqi[r, c] == pytest.approx(fd(f, x["q_idx"], (b, i, g, c)), rel=1e-6, abs=1e-8)
    for _ in range(12):
        idx = tuple(rng.integers(0, n) for n in x["k_idx"].shape)
        assert dki[idx] == pytest.approx(fd(f, x["k_idx"], idx), rel=1e-6, abs=1e-8)


def test_grads_dense_selection_match_torch_autograd(oracle_mod):
    """With every visible block selected: dq, dk, dv equal torch autograd of
    dense causal softmax attention, and the index gradients equal autograd of
    torch's kl_div against the detached group-mean teacher."""
    rng = np.random.default_rng(23)
    B, Sq, Sk, Hq, Hkv, D, Didx, bs = 2, 9, 13, 4, 2, 5, 3, 4
    p = oracle.Problem(B, Sq, Sk, Hq, Hkv, D, Didx, block_size=bs, topk=-(-Sk // bs))
    x = dict(q=rng.normal(size=(B, Sq, Hq, D)), k=rng.normal(size=(B, Sk, Hkv, D)),
             v=rng.normal(size=(B, Sk, Hkv, D)), dout=rng.normal(size=(B, Sq, Hq, D)),
             q_idx=rng.normal(size=(B, Sq, Hkv, Didx)), k_idx=rng.normal(size=(B, Sk, Didx)))
    rows = p.all_rows()
    sel = np.full((len(rows), p.topk), -1, dtype=np.int32)
    for r, (b, i, g) in enumerate(rows):
        local = (i + Sk - Sq) // bs
        sel[r, :local + 1] = np.arange(local + 1)
    dq, dk, dv = oracle.attention_bwd(p, x["q"], x["k"], x["v"], x["dout"], sel, rows)
    dqi, dki, _ = oracle.kl_bwd(p, x["q"], x["k"], x["q_idx"], x["k_idx"], sel, rows)

    T = {n: torch.tensor(a, requires_grad=True) for n, a in x.items()}
    G = Hq // Hkv
    mask = torch.arange(Sk)[None, :] > (torch.arange(Sq)[:, None] + Sk - Sq)
    L = 0.0
    kl_total = 0.0
    for b in range(B):
        for g in range(Hkv):
            heads = []
            for hh in range(G):
                h = g * G + hh
                s = (T["q"][b, :, h] @ T["k"][b, :, g].T / np.sqrt(D)).masked_fill(mask, -np.inf)
                pr = torch.softmax(s, -1)
                L = L + (pr @ T["v"][b, :, g] * T["dout"][b, :, h]).sum()
                heads.append(pr)
            teacher = torch.stack(heads).mean(0).detach()
            logz = torch.log_softmax((T["q_idx"][b, :, g] @ T["k_idx"][b].T).masked_fill(mask, -np.inf), -1)
            for i in range(Sq):
                vis = ~mask[i]
                kl_total = kl_total + torch.nn.functional.kl_div(logz[i, vis], teacher[i, vis], reduction="sum")
    L.backward()
    kl_total.backward()
    got_dq = np.zeros_like(x["q"])
    for r, (b, i, g) in enumerate(rows):
        got_dq[b, i, g * G:(g + 1) * G] = dq[r]
    np.testing.assert_allclose(got_dq, T["q"].grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, T["k"].grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, T["v"].grad.numpy(), rtol=1e-10, atol=1e-12)
    got_dqi = np.zeros_like(x["q_idx"])
    for r, (b, i, g) in enumerate(rows):
        got_dqi[b, i, g] = dqi[r]
    np.testing.assert_allclose(got_dqi, T["q_idx"].grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dki, T["k_idx"].grad.numpy(), rtol=1e-10, atol=1e-12)


def test_gradient_sum_identities(oracle_mod):
    """Each row's softmax sums to one over its tokens, so summed over keys the
    key gradient of a group is 0, its value gradient is the sum of the group's
    dO rows, and the index-key gradient is 0 (student and teacher both sum to
    one).  Checked on bf16 inputs with sparse random selections."""
    rng = np.random.default_rng(24)
    w = synth.Workload("bwd_id", 2, 60, 200, 8, 2, head_dim=16, index_dim=8, block_size=16, topk=4)
    p = oracle.Problem.of(w)
    h = {n: synth.host_tensor(w, n) for n in ("q", "k", "v", "q_idx", "k_idx")}
    dout = synth.f32_to_bf16_bits(rng.normal(size=h["q"].shape).astype(np.float32))
    rows, sel = random_selection(p, rng)
    dq, dk, dv = oracle.attention_bwd(p, h["q"], h["k"], h["v"], dout, sel, rows)
    G = p.group
    do = synth.bf16_bits_to_f32(dout).astype(np.float64)
    for b in range(2):
        for g in range(2):
            assert np.abs(dk[b, :, g].sum(0)).max() < 1e-9
            np.testing.assert_allclose(dv[b, :, g].sum(0), do[b, :, g * G:(g + 1) * G].sum((0, 1)), atol=1e-9)
    _, dki, _ = oracle.kl_bwd(p, h["q"], h["k"], h["q_idx"], h["k_idx"], sel, rows)
    assert np.abs(dki.sum(1)).max() < 1e-6 * max(1.0, np.abs(dki).max())


def test_bf16_and_fp64_entries_agree(oracle_mod):
    """The bf16 entry points read their inputs exactly as fp64 ones would."""
    rng = np.random.default_rng(25)
    w = synth.Workload("bwd_same", 1, 20, 40, 4, 2, head_dim=8, index_dim=4, block_size=8, topk=3)
    p = oracle.Problem.of(w)
    h = {n: synth.host_tensor(w, n) for n in ("q", "k", "v", "q_idx", "k_idx")}
    dout = synth.f32_to_bf16_bits(rng.normal(size=h["q"].shape).astype(np.float32))
    f = {n: synth.bf16_bits_to_f32(a).astype(np.float64) for n, a in h.items()}
    rows, sel = random_selection(p, rng)
    a = oracle.attention_bwd(p, h["q"], h["k"], h["v"], dout, sel, rows)
    b = oracle.attention_bwd(p, f["q"], f["k"], f["v"], synth.bf16_bits_to_f32(dout).astype(np.float64), sel, rows)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    a = oracle.kl_bwd(p, h["q"], h["k"], h["q_idx"], h["k_idx"], sel, rows)
    b = oracle.kl_bwd(p, f["q"], f["k"], f["q_idx"], f["k_idx"], sel, rows)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
