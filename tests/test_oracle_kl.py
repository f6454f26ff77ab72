"""Pins of the oracle's alignment-loss term (Sparse Attention Part II,
section 3.2): KL(teacher || student) per (query, group) row over the visible
tokens of the row's selected blocks, teacher = mean over the group's heads of
each head's softmax there, student = softmax of the raw index token scores.

Each test checks the oracle against something its code does not contain:
closed forms of the KL for a uniform teacher or a two-point mixture teacher,
the identity KL(p || p) = 0, torch's dense softmax and kl_div when the
selection covers the whole prefix, and invariances (head order inside a group,
tokens outside the selection or past the query).
"""
import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle
import synth


def bits(x):
    return synth.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def random_selection(p, rng):
    """A valid selection per row: the local block, up to k-1 distinct earlier
    blocks, ascending, padded with -1."""
    rows = p.all_rows()
    sel = np.full((len(rows), p.topk), -1, dtype=np.int32)
    for r, (b, i, g) in enumerate(rows):
        local = (i + p.seqlen_k - p.seqlen_q) // p.block_size
        n = min(local, p.topk - 1, rng.integers(0, p.topk))
        pick = sorted(rng.choice(local, size=n, replace=False).tolist()) if n else []
        sel[r, :n + 1] = pick + [local]
    return rows, sel


def token_set(p, i, sel_row):
    t = i + p.seqlen_k - p.seqlen_q
    toks = []
    for j in sel_row:
        if j >= 0:
            toks += [s for s in range(j * p.block_size, (j + 1) * p.block_size) if s <= t]
    return np.array(toks)


def normal_bits(rng, shape, sd=1.0):
    return bits(rng.normal(0.0, sd, size=shape))


@pytest.mark.parametrize("B,Sq,Sk,Hq,Hkv,bs,k,Didx", [
    (2, 37, 53, 4, 2, 8, 3, 4), (1, 64, 64, 2, 2, 16, 4, 3), (1, 1, 41, 8, 1, 8, 5, 6)])
def test_kl_uniform_teacher_closed_form(oracle_mod, B, Sq, Sk, Hq, Hkv, bs, k, Didx):
    """Q = 0 makes every head uniform over the token set T, so the teacher is
    uniform; with q_idx = 1 and k_idx rows c_s * 1 the index score is
    Didx * c_s and KL(U || softmax z) = logsumexp(z_T) - mean(z_T) - ln |T|."""
    p = oracle.Problem(B, Sq, Sk, Hq, Hkv, 8, Didx, block_size=bs, topk=k)
    rng = np.random.default_rng(11)
    q = bits(np.zeros((B, Sq, Hq, 8)))
    kk = normal_bits(rng, (B, Sk, Hkv, 8))
    c = rng.integers(-3, 4, size=(B, Sk))
    q_idx = bits(np.ones((B, Sq, Hkv, Didx)))
    k_idx = bits(np.repeat(c[..., None], Didx, axis=-1).astype(float))
    rows, sel = random_selection(p, rng)
    kl = oracle.kl_rows(p, q, kk, q_idx, k_idx, sel, rows)
    for r, (b, i, g) in enumerate(rows):
        z = Didx * c[b, token_set(p, i, sel[r])].astype(float)
        exp = logsumexp(z) - z.mean() - np.log(len(z))
        assert kl[r] == pytest.approx(exp, abs=1e-12, rel=1e-12)


def test_kl_mixture_teacher_closed_form(oracle_mod):
    """Group 0: head 0 has Q = 0 (uniform), head 1 aligns with token 0 only
    (its other logits sit 45 below), so the teacher is (U + delta_0) / 2; the
    student is uniform (q_idx = 0).  KL = sum P ln(n P) in closed form.  Group
    1 has both heads at Q = 0: teacher = student, KL = 0.  A wrong head-to-group
    map or a product instead of a mean of the heads fails one of the two."""
    B, Sq, Sk, Hq, Hkv, D, bs, k = 1, 40, 40, 4, 2, 8, 8, 3
    p = oracle.Problem(B, Sq, Sk, Hq, Hkv, D, 4, block_size=bs, topk=k, softmax_scale=1.0 / np.sqrt(D))
    q = np.zeros((B, Sq, Hq, D))
    q[:, :, 1, :] = 8.0
    kk = -np.ones((B, Sk, Hkv, D))
    kk[:, 0, 0, :] = 1.0
    rng = np.random.default_rng(12)
    rows, sel = random_selection(p, rng)
    for r, (b, i, g) in enumerate(rows):  # keep block 0 selected
        if sel[r, 0] != 0:
            sel[r] = np.array(sorted(set([0] + [x for x in sel[r] if x >= 0][-(k - 1):])) + [-1] * k)[:k]
    kl = oracle.kl_rows(p, bits(q), bits(kk), bits(np.zeros((B, Sq, Hkv, 4))), bits(np.zeros((B, Sk, 4))),
                        sel, rows)
    for r, (b, i, g) in enumerate(rows):
        n = len(token_set(p, i, sel[r]))
        if g == 1 or n == 1:
            assert abs(kl[r]) < 1e-12
            continue
        P = np.full(n, 0.5 / n)
        P[0] += 0.5
        assert kl[r] == pytest.approx(float(np.sum(P * np.log(n * P))), abs=1e-12)


def test_kl_student_equal_to_teacher_is_zero(oracle_mod):
    """G = 1, one group, q_idx = Q, k_idx = K and scale 1: the student's
    logits are the head's logits, so KL(p || p) = 0 on every row."""
    B, Sq, Sk, D, bs, k = 2, 48, 70, 16, 8, 4
    p = oracle.Problem(B, Sq, Sk, 1, 1, D, D, block_size=bs, topk=k, softmax_scale=1.0)
    rng = np.random.default_rng(13)
    q = normal_bits(rng, (B, Sq, 1, D), 0.5)
    kk = normal_bits(rng, (B, Sk, 1, D), 0.5)
    rows, sel = random_selection(p, rng)
    kl = oracle.kl_rows(p, q, kk, q.reshape(B, Sq, 1, D), kk.reshape(B, Sk, D), sel, rows)
    assert np.max(np.abs(kl)) < 1e-12


@pytest.mark.parametrize("Sq,Sk,Hq,Hkv,scale", [(24, 24, 8, 2, 0.0), (17, 45, 4, 4, 0.3)])
def test_kl_dense_selection_matches_torch(oracle_mod, Sq, Sk, Hq, Hkv, scale):
    """With every visible block selected, the teacher is the group mean of
    torch's dense causal softmax and the term is torch's kl_div against the
    causal log_softmax of the index scores."""
    B, D, Didx, bs = 2, 8, 5, 8
    p = oracle.Problem(B, Sq, Sk, Hq, Hkv, D, Didx, block_size=bs, topk=-(-Sk // bs), softmax_scale=scale)
    rng = np.random.default_rng(14)
    q, kk = normal_bits(rng, (B, Sq, Hq, D)), normal_bits(rng, (B, Sk, Hkv, D))
    qi, ki = normal_bits(rng, (B, Sq, Hkv, Didx), 2.0), normal_bits(rng, (B, Sk, Didx), 2.0)
    rows = p.all_rows()
    sel = np.full((len(rows), p.topk), -1, dtype=np.int32)
    for r, (b, i, g) in enumerate(rows):
        local = (i + Sk - Sq) // bs
        sel[r, :local + 1] = np.arange(local + 1)
    kl = oracle.kl_rows(p, q, kk, qi, ki, sel, rows).reshape(B, Sq, Hkv)

    f = lambda x: torch.from_numpy(synth.bf16_bits_to_f32(x).astype(np.float64))
    Q, K, QI, KI = f(q), f(kk), f(qi), f(ki)
    G = Hq // Hkv
    sc = scale if scale else 1.0 / np.sqrt(D)
    mask = torch.arange(Sk)[None, :] > (torch.arange(Sq)[:, None] + Sk - Sq)
    for b in range(B):
        for g in range(Hkv):
            heads = [torch.softmax((Q[b, :, g * G + hh] @ K[b, :, g].T * sc).masked_fill(mask, -np.inf), -1)
                     for hh in range(G)]
            teacher = torch.stack(heads).mean(0)
            log_student = torch.log_softmax((QI[b, :, g] @ KI[b].T).masked_fill(mask, -np.inf), -1)
            for i in range(Sq):
                vis = ~mask[i]
                ref = torch.nn.functional.kl_div(log_student[i, vis], teacher[i, vis], reduction="sum")
                assert kl[b, i, g] == pytest.approx(float(ref), abs=1e-10, rel=1e-10)


def test_kl_invariances(oracle_mod):
    """KL >= 0; permuting the heads inside a group changes nothing; tokens of
    unselected blocks and tokens past the query do not enter; changing a
    selected visible token does."""
    B, Sq, Sk, Hq, Hkv, D, Didx, bs, k = 1, 30, 62, 6, 2, 8, 4, 8, 3
    p = oracle.Problem(B, Sq, Sk, Hq, Hkv, D, Didx, block_size=bs, topk=k)
    rng = np.random.default_rng(15)
    q, kk = normal_bits(rng, (B, Sq, Hq, D)), normal_bits(rng, (B, Sk, Hkv, D))
    qi, ki = normal_bits(rng, (B, Sq, Hkv, Didx)), normal_bits(rng, (B, Sk, Didx))
    rows, sel = random_selection(p, rng)
    kl = oracle.kl_rows(p, q, kk, qi, ki, sel, rows)
    assert kl.min() >= -1e-12 and kl.max() > 1e-3

    perm = np.array([2, 0, 1, 4, 5, 3])  # within groups {0,1,2} and {3,4,5}
    assert np.allclose(oracle.kl_rows(p, q[:, :, perm], kk, qi, ki, sel, rows), kl, atol=1e-13, rtol=1e-12)
    cross = np.array([3, 1, 2, 0, 4, 5])
    assert not np.allclose(oracle.kl_rows(p, q[:, :, cross], kk, qi, ki, sel, rows), kl, atol=1e-6)

    # Row (0, i, 0) with its selection: perturb an unselected block, an
    # invisible token of the local block, then a selected visible token.
    r = next(r for r, (b, i, g) in enumerate(rows)
             if g == 0 and (i + Sk - Sq) % bs < bs - 1 and 2 <= (sel[r] >= 0).sum() < (i + Sk - Sq) // bs + 1)
    i = rows[r, 1]
    t = i + Sk - Sq
    unsel = next(j for j in range(t // bs) if j not in sel[r])
    one = rows[r:r + 1]
    base = oracle.kl_rows(p, q, kk, qi, ki, sel[r:r + 1], one)[0]
    assert base > 0
    for s in (unsel * bs + 3, t + 1):
        k2, ki2 = kk.copy(), ki.copy()
        k2[0, s] = bits(rng.normal(size=(Hkv, D)))
        ki2[0, s] = bits(rng.normal(size=Didx) * 5)
        assert oracle.kl_rows(p, q, k2, qi, ki2, sel[r:r + 1], one)[0] == base
    ki3 = ki.copy()
    ki3[0, t] = bits(synth.bf16_bits_to_f32(ki[0, t]) + 3.0)
    assert oracle.kl_rows(p, q, kk, qi, ki3, sel[r:r + 1], one)[0] != base


def test_kl_rejects_selection_without_local_block(oracle_mod):
    p = oracle.Problem(1, 16, 16, 2, 1, 8, 4, block_size=8, topk=2)
    z = bits(np.zeros((1, 16, 2, 8)))
    sel = np.tile(np.array([[0, -1]], dtype=np.int32), (16, 1))
    with pytest.raises(ValueError):
        oracle.kl_rows(p, z, bits(np.zeros((1, 16, 1, 8))), bits(np.zeros((1, 16, 1, 4))),
                       bits(np.zeros((1, 16, 4))), sel)
