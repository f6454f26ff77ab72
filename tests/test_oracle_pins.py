"""Pins of the CPU oracle to facts other than its own code.

Each test checks the oracle against something the pages or plain mathematics
fix: closed forms, a brute-force rank definition of the selection that uses no
sort, torch's dense scaled-dot-product attention (a library routine) where the
selection covers the whole prefix, the sparse-vs-dense error bound of Sparse
Attention Part II section 2, and invariants of section 3.2 (local block always
kept, at most k blocks and k * block_size tokens per query and group).
"""
import itertools

import numpy as np
import pytest
import torch

import oracle
import synth

NEG_INF = -np.inf


def bits(x):
    return synth.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def positions(p):
    return np.arange(p.seqlen_q) + p.seqlen_k - p.seqlen_q


# ------------------------------------------------------------ block scores
@pytest.mark.parametrize("Sq,Sk,bs,Didx", [(40, 40, 8, 4), (13, 50, 8, 6), (1, 37, 16, 8), (64, 64, 16, 4)])
def test_block_scores_closed_form_constant_rows(oracle_mod, Sq, Sk, bs, Didx):
    """q_idx row (b,i,g) = a_big constant, k_idx row s = c_bs constant: the token
    score is Didx * a * c, so the block score is Didx * a * max c (a > 0) or
    Didx * a * min c (a < 0) over the visible part of the block; -inf beyond the
    local block (section 3.2: max token score per block, visible tokens only)."""
    B, Hkv = 2, 3
    p = oracle.Problem(B, Sq, Sk, Hkv * 2, Hkv, 8, Didx, block_size=bs, topk=3)
    rng = np.random.default_rng(1)
    a = rng.choice([-3, -2, -1, 1, 2, 3], size=(B, Sq, Hkv))
    c = rng.integers(-3, 4, size=(B, Sk))
    q_idx = bits(np.repeat(a[..., None], Didx, axis=-1))
    k_idx = bits(np.repeat(c[..., None], Didx, axis=-1))
    bm = oracle.block_scores(p, q_idx, k_idx)
    t = positions(p)
    exp = np.full((B, Sq, Hkv, p.n_blk), NEG_INF)
    for b, i, g in itertools.product(range(B), range(Sq), range(Hkv)):
        for j in range(t[i] // bs + 1):
            vis = c[b, j * bs: min((j + 1) * bs, t[i] + 1)]
            ext = vis.max() if a[b, i, g] > 0 else vis.min()
            exp[b, i, g, j] = Didx * a[b, i, g] * ext
    np.testing.assert_array_equal(bm, exp.reshape(-1, p.n_blk))


def test_block_scores_one_hot_channel_picks_a_column(oracle_mod):
    """q_idx = one-hot on channel c0 makes the token score k_idx[s, c0]: a
    transposed operand or a wrong channel stride changes the result."""
    p = oracle.Problem(1, 24, 24, 2, 2, 8, 5, block_size=8, topk=2)
    rng = np.random.default_rng(2)
    k = rng.integers(-3, 4, size=(1, 24, 5))
    q = np.zeros((1, 24, 2, 5))
    q[:, :, 0, 1] = 1.0
    q[:, :, 1, 4] = -2.0
    bm = oracle.block_scores(p, bits(q), bits(k)).reshape(24, 2, 3)
    for i in range(24):
        for j in range(3):
            vis = slice(j * 8, min(j * 8 + 8, i + 1))
            if j * 8 > i:
                assert bm[i, 0, j] == NEG_INF and bm[i, 1, j] == NEG_INF
                continue
            assert bm[i, 0, j] == k[0, vis, 1].max()
            assert bm[i, 1, j] == -2.0 * k[0, vis, 4].min()


def test_block_scores_planted_spike(oracle_mod):
    """One k_idx row of +3 against q_idx of +3 scores 9 * Didx, above every
    other token (|score| <= 9 * Didx with equality only there)."""
    p = oracle.Problem(1, 64, 64, 4, 1, 8, 16, block_size=8, topk=3)
    rng = np.random.default_rng(3)
    k = rng.integers(-2, 3, size=(1, 64, 16)).astype(float)
    k[0, 21] = 3.0
    q = np.full((1, 64, 1, 16), 3.0)
    bm = oracle.block_scores(p, bits(q), bits(k))
    assert np.all(bm[21:, 2] == 9 * 16)
    assert np.all(bm[:21, 2] < 9 * 16)
    sel = oracle.select(p, bm)
    for i in range(64):
        li = i // 8
        if li > 2:
            assert 2 in sel[i], "the block holding the spike must be selected"


# --------------------------------------------------------------- selection
def rank_select(bm_row, local, k):
    """Brute-force rank definition, no sort: block j < local is kept iff fewer
    than k-1 earlier blocks beat it (higher score, or equal score and lower
    index); the local block is always kept (section 3.2; ties: section 4.2)."""
    kept = []
    for j in range(local):
        beaten = sum(1 for jj in range(local)
                     if bm_row[jj] > bm_row[j] or (bm_row[jj] == bm_row[j] and jj < j))
        if beaten < k - 1:
            kept.append(j)
    kept.append(local)
    return kept


@pytest.mark.parametrize("k", [1, 2, 5, 16])
def test_select_matches_rank_definition_with_ties(oracle_mod, k):
    Sk, bs = 300, 4
    p = oracle.Problem(1, Sk, Sk, 1, 1, 8, 8, block_size=bs, topk=k)
    rng = np.random.default_rng(10 + k)
    bm = rng.integers(-4, 5, size=(Sk, p.n_blk)).astype(np.float64)  # many ties
    t = positions(p)
    for i in range(Sk):
        bm[i, t[i] // bs + 1:] = NEG_INF
    sel = oracle.select(p, bm)
    for i in range(Sk):
        exp = rank_select(bm[i], t[i] // bs, k)
        got = [j for j in sel[i] if j >= 0]
        assert got == exp, (i, got, exp)
        assert list(sel[i][len(exp):]) == [-1] * (k - len(exp))


def test_select_all_equal_scores_keeps_lowest_indices(oracle_mod):
    """k_idx = 0 makes every block score 0: the tie rule keeps blocks
    0 .. k-2 plus the local block."""
    p = oracle.Problem(1, 200, 200, 2, 2, 8, 4, block_size=8, topk=6)
    q = bits(np.ones((1, 200, 2, 4)))
    kz = bits(np.zeros((1, 200, 4)))
    sel = oracle.select(p, oracle.block_scores(p, q, kz))
    for r, (b, i, g) in enumerate(p.all_rows()):
        local = i // 8
        exp = list(range(min(5, local))) + [local]
        assert [j for j in sel[r] if j >= 0] == exp


def test_select_local_block_never_competes(oracle_mod):
    """The local block's own score, high or low, does not change which
    earlier blocks are chosen (section 3.2: the local block has a slot of its own)."""
    p = oracle.Problem(1, 64, 64, 1, 1, 8, 8, block_size=4, topk=4)
    rng = np.random.default_rng(4)
    bm = rng.normal(size=(64, 16))
    t = positions(p)
    for i in range(64):
        bm[i, t[i] // 4 + 1:] = NEG_INF
    hi, lo = bm.copy(), bm.copy()
    for i in range(64):
        hi[i, t[i] // 4] = 1e9
        lo[i, t[i] // 4] = -1e9
    np.testing.assert_array_equal(oracle.select(p, hi), oracle.select(p, lo))


def test_select_invariants_on_a_workload_shape(oracle_mod):
    """Local block kept; count = min(k, l+1); ascending, unique; at most
    k * block_size tokens (section 3.2: 16 blocks of 128 cap the tokens per query and group)."""
    w = synth.WORKLOADS["prefill_4k"].with_(seqlen_q=512, seqlen_k=2304)
    p = oracle.Problem.of(w)
    rows = p.all_rows()[::7]
    bm = oracle.block_scores(p, synth.host_tensor(w, "q_idx"), synth.host_tensor(w, "k_idx"), rows)
    sel = oracle.select(p, bm, rows)
    for (b, i, g), s in zip(rows, sel):
        t = i + p.seqlen_k - p.seqlen_q
        local = t // 128
        valid = [j for j in s if j >= 0]
        assert valid[-1] == local and len(valid) == min(16, local + 1)
        assert valid == sorted(set(valid))
        assert all(j == -1 for j in s[len(valid):])
        assert sum(min(128, t + 1 - 128 * j) for j in valid) <= 16 * 128


# --------------------------------------------------------------- attention
def dense_reference(p, q, k, v):
    """Dense causal GQA attention (bottom-right aligned) by torch SDPA in fp64."""
    f = lambda a: torch.from_numpy(synth.bf16_bits_to_f32(a).astype(np.float64))
    Q = f(q).permute(0, 2, 1, 3)
    K = f(k).permute(0, 2, 1, 3)
    V = f(v).permute(0, 2, 1, 3)
    t = positions(p)
    mask = torch.from_numpy(np.arange(p.seqlen_k)[None, :] <= t[:, None])
    scale = p.softmax_scale or None
    O = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=scale,
                                                         enable_gqa=True)
    return O.permute(0, 2, 1, 3).numpy()  # [B, Sq, Hq, D]


def random_problem(seed, B, Sq, Sk, Hq, Hkv, D, Didx, bs, k, scale=0.0):
    p = oracle.Problem(B, Sq, Sk, Hq, Hkv, D, Didx, block_size=bs, topk=k, softmax_scale=scale)
    rng = np.random.default_rng(seed)
    q = bits(rng.normal(size=(B, Sq, Hq, D)))
    kk = bits(rng.normal(size=(B, Sk, Hkv, D)))
    v = bits(rng.normal(size=(B, Sk, Hkv, D)))
    qi = bits(rng.integers(-3, 4, size=(B, Sq, Hkv, Didx)))
    ki = bits(rng.integers(-3, 4, size=(B, Sk, Didx)))
    return p, q, kk, v, qi, ki


def to_bshd(p, out):
    """Oracle rows (b,i,g) x G x D -> [B, Sq, Hq, D]."""
    return out.reshape(p.batch, p.seqlen_q, p.heads_kv * p.group, p.head_dim)


@pytest.mark.parametrize("B,Sq,Sk,Hq,Hkv,bs,k,scale", [
    (2, 37, 37, 4, 2, 8, 5, 0.0),      # every block selectable: k * bs >= S_k
    (1, 20, 53, 8, 2, 16, 4, 0.0),     # chunk at the end of a longer prefix
    (1, 64, 64, 3, 1, 8, 8, 0.3),      # multi-query, explicit scale
    (2, 9, 9, 2, 2, 4, 3, 0.0),        # ragged last block
])
def test_attention_equals_dense_when_selection_covers_prefix(oracle_mod, B, Sq, Sk, Hq, Hkv, bs, k, scale):
    """When k blocks cover every visible block the selection is the whole
    causal prefix, so MSA reduces to dense causal GQA attention."""
    p, q, kk, v, qi, ki = random_problem(7, B, Sq, Sk, Hq, Hkv, 16, 4, bs, k, scale)
    assert k * bs >= Sk
    res = oracle.forward(p, q, kk, v, qi, ki)
    np.testing.assert_allclose(to_bshd(p, res["out"]), dense_reference(p, q, kk, v), rtol=0, atol=1e-12)


def test_attention_dense_regime_of_long_rows(oracle_mod):
    """Queries whose local block index is below k see every earlier block
    (all of 0..l kept), so they match dense attention even when S_k > k * bs."""
    p, q, kk, v, qi, ki = random_problem(8, 1, 96, 96, 4, 2, 16, 4, 8, 4)
    res = oracle.forward(p, q, kk, v, qi, ki)
    dense = dense_reference(p, q, kk, v)
    got = to_bshd(p, res["out"])
    n_dense = 4 * 8  # t < k * bs
    np.testing.assert_allclose(got[:, :n_dense], dense[:, :n_dense], rtol=0, atol=1e-12)
    assert np.abs(got[:, n_dense:] - dense[:, n_dense:]).max() > 1e-6  # sparse rows differ


def test_attention_constant_values(oracle_mod):
    """Identical value vectors give that vector under any normalised
    weighting (Sparse Attention Part II, section 2)."""
    p, q, kk, v, qi, ki = random_problem(9, 1, 50, 50, 4, 2, 16, 4, 8, 3)
    row = np.random.default_rng(0).normal(size=16)
    v = bits(np.broadcast_to(row, (1, 50, 2, 16)))
    res = oracle.forward(p, q, kk, v, qi, ki)
    np.testing.assert_allclose(res["out"], np.broadcast_to(synth.bf16_bits_to_f32(bits(row)), res["out"].shape),
                               rtol=0, atol=1e-12)


def test_attention_zero_query_is_mean_over_selected_tokens(oracle_mod):
    """Q = 0 gives equal weights: O = mean of V over the visible tokens of the
    selected blocks, LSE = log(#tokens)."""
    p, q, kk, v, qi, ki = random_problem(11, 1, 70, 90, 4, 2, 16, 4, 8, 3)
    q = bits(np.zeros((1, 70, 4, 16)))
    res = oracle.forward(p, q, kk, v, qi, ki)
    V = synth.bf16_bits_to_f32(v).astype(np.float64)
    for r, (b, i, g) in enumerate(res["rows"]):
        t = i + 90 - 70
        toks = [s for j in res["sel"][r] if j >= 0 for s in range(8 * j, 8 * j + 8) if s <= t]
        exp = V[b, toks, g].mean(axis=0)
        for hh in range(2):
            np.testing.assert_allclose(res["out"][r, hh], exp, rtol=0, atol=1e-12)
            assert abs(res["lse"][r, hh] - np.log(len(toks))) < 1e-12


def test_attention_lse_with_constant_keys(oracle_mod):
    """All keys equal to k0: every logit is scale * q.k0, so
    LSE = scale * q.k0 + log(#tokens)."""
    p, q, kk, v, qi, ki = random_problem(12, 1, 40, 40, 2, 1, 16, 4, 8, 2)
    k0 = np.random.default_rng(5).normal(size=16)
    kk = bits(np.broadcast_to(k0, (1, 40, 1, 16)))
    res = oracle.forward(p, q, kk, v, qi, ki)
    Q = synth.bf16_bits_to_f32(q).astype(np.float64)
    K0 = synth.bf16_bits_to_f32(bits(k0)).astype(np.float64)
    for r, (b, i, g) in enumerate(res["rows"]):
        n = sum(min(8, i + 1 - 8 * j) for j in res["sel"][r] if j >= 0)
        for hh in range(2):
            exp = (Q[b, i, hh] @ K0) / 4.0 + np.log(n)
            assert abs(res["lse"][r, hh] - exp) < 1e-12


def test_attention_sparse_vs_dense_error_bound(oracle_mod):
    """||o - o_sparse|| <= 2 B delta, delta = dense softmax mass outside the
    selection, B = max value norm (Sparse Attention Part II, section 2)."""
    p, q, kk, v, qi, ki = random_problem(13, 1, 120, 120, 4, 2, 16, 4, 8, 3)
    res = oracle.forward(p, q, kk, v, qi, ki)
    Q = synth.bf16_bits_to_f32(q).astype(np.float64)
    K = synth.bf16_bits_to_f32(kk).astype(np.float64)
    V = synth.bf16_bits_to_f32(v).astype(np.float64)
    dense = dense_reference(p, q, kk, v)
    Bnorm = np.linalg.norm(V, axis=-1).max()
    for r, (b, i, g) in enumerate(res["rows"]):
        t = i
        inside = np.zeros(t + 1, dtype=bool)
        for j in res["sel"][r]:
            if j >= 0:
                inside[8 * j: min(8 * j + 8, t + 1)] = True
        for hh in range(2):
            h = g * 2 + hh
            a = K[b, : t + 1, g] @ Q[b, i, h] / 4.0
            w = np.exp(a - a.max())
            w /= w.sum()
            delta = w[~inside].sum()
            err = np.linalg.norm(res["out"][r, hh] - dense[b, i, h])
            assert err <= 2 * Bnorm * delta + 1e-12


def test_attention_brute_force_mask_tiny(oracle_mod):
    """Tiny case against an explicit 0/1 token mask built from the selection
    and a dense masked softmax (S=64, bs=8, k=3, D=8, Didx=4, Hq=4, Hkv=2)."""
    p, q, kk, v, qi, ki = random_problem(14, 1, 64, 64, 4, 2, 8, 4, 8, 3)
    res = oracle.forward(p, q, kk, v, qi, ki)
    Q = synth.bf16_bits_to_f32(q).astype(np.float64)[0]
    K = synth.bf16_bits_to_f32(kk).astype(np.float64)[0]
    V = synth.bf16_bits_to_f32(v).astype(np.float64)[0]
    sel = res["sel"].reshape(64, 2, 3)
    blk_of = np.arange(64) // 8
    for h in range(4):
        g = h // 2
        M = np.zeros((64, 64), dtype=bool)
        for i in range(64):
            M[i] = np.isin(blk_of, sel[i, g][sel[i, g] >= 0]) & (np.arange(64) <= i)
        S = np.where(M, Q[:, h] @ K[:, g].T / np.sqrt(8), -np.inf)
        P = np.exp(S - S.max(axis=1, keepdims=True))
        P /= P.sum(axis=1, keepdims=True)
        O = P @ V[:, g]
        np.testing.assert_allclose(to_bshd(p, res["out"])[0, :, h], O, rtol=0, atol=1e-12)


def test_oracle_rejects_bad_rows_and_selections(oracle_mod):
    p, q, kk, v, qi, ki = random_problem(15, 1, 16, 16, 2, 1, 8, 4, 8, 2)
    with pytest.raises(ValueError):
        oracle.block_scores(p, qi, ki, rows=np.array([[0, 16, 0]]))
    bad = np.array([[0, -1]], dtype=np.int32)  # local block missing
    with pytest.raises(ValueError):
        oracle.attention(p, q, kk, v, bad, rows=np.array([[0, 12, 0]]))
