"""GPU parity: the HIP path through the C ABI against the CPU oracle, element
by element, on seeded inputs that span several tiles and ragged tails.

Block scores and selections must be bit-exact (index inputs are integers
stored exactly in bf16, so every fp32 score is exact); outputs must meet the
tolerance rule of gpu_util (beyond each value's own bf16 rounding: max 1e-2,
mean 1e-3 against the fp64 oracle); LSE within 1e-3.  Outputs and workspaces
are poisoned before every call.
"""
import numpy as np
import pytest
import torch

import block_sparse_gqa_scores_amd as msa
import oracle
import synth
from gpu_util import check_close, compare, host_inputs, inputs_for, parity, run_device, to_u16

pytestmark = pytest.mark.gpu


def W(name, B, Sq, Sk, Hq, Hkv, Didx=128, topk=16, **kw):
    return synth.Workload(name, B, Sq, Sk, Hq, Hkv, index_dim=Didx, topk=topk, **kw)


def test_device_generator_matches_host_generator():
    """The device fill kernel and the numpy generator agree bit for bit."""
    for w in (W("gen", 2, 300, 1000, 8, 2, Didx=64), W("gen_gain", 1, 10, 3000, 4, 2, gain=True)):
        t = inputs_for(w)
        rng = np.random.default_rng(0)
        for name, x in t.items():
            n = x.numel()
            e = np.unique(np.concatenate([np.arange(min(n, 4096)), rng.integers(0, n, 20000)]))
            got = to_u16(x).reshape(-1)[e]
            exp = synth.host_bits(w, name, e.astype(np.uint64))
            assert np.array_equal(got, exp), (w.name, name, int((got != exp).sum()))


SMALL = [
    W("prefill_4k_full", 1, 4096, 4096, 8, 2, Didx=64),                 # the 4K workload, every row
    W("ragged_chunk", 2, 700, 1000, 8, 2, topk=5),                      # S_k % 128 != 0, S_q < S_k
    W("gqa8_sparse", 1, 2600, 2600, 64, 8),                             # G = 8, past the dense regime
    W("mha", 1, 600, 777, 4, 4, Didx=64, topk=3),                       # G = 1
    W("g16", 1, 500, 640, 32, 2, topk=2),                               # G = 16
    W("g32", 2, 300, 300, 32, 1, Didx=64, topk=4),                      # G = 32, one group
    W("topk1", 1, 400, 900, 8, 2, topk=1),                              # local block only
    W("hkv12", 1, 400, 900, 12, 12, Didx=64, topk=4),                   # H_kv = 12, not a power of two
    W("decode_small", 3, 1, 5000, 16, 2, Didx=64),                      # S_q = 1: decode kernels
    W("decode_mha", 2, 1, 3000, 4, 4, topk=8),                          # decode, G = 1
    W("decode_g2", 2, 1, 2500, 8, 4, Didx=64, topk=5),                  # decode, G = 2
    W("decode_g4", 3, 1, 4100, 8, 2),                                   # decode, G = 4
    W("decode_g16", 2, 1, 3300, 32, 2, topk=6),                         # decode, G = 16
    W("decode_g32", 2, 1, 2049, 32, 1, Didx=64),                        # decode, G = 32
    W("decode_short", 4, 1, 300, 16, 2),                                # 3 blocks < k: unused entries
    W("decode_r32", 2, 4, 3001, 64, 8),                                 # 32 rows per sequence
    W("scale", 1, 300, 1400, 8, 4, topk=4),
    W("gain", 1, 1500, 3000, 16, 2, gain=True, topk=6),                 # uneven block scores
    W("k64", 1, 130, 9000, 4, 1, topk=64),                              # the largest topk
    W("dense_k1", 2, 300, 300, 8, 2, topk=1),                           # dense rows: block 0 only
    W("dense_k64", 1, 900, 900, 4, 1, Didx=64, topk=64),                # every row dense, k = 64
    W("dense_g32", 1, 260, 390, 32, 1, topk=3),                         # dense tiles of one query (G = 32)
]


def sampled_rows(w, step=5, around=(2040, 2110), tail=100):
    """All groups of every step-th query, the queries around the dense/sparse
    boundary (t = 2047 / 2048) and the last ``tail`` queries."""
    off = w.seqlen_k - w.seqlen_q
    qs = set(range(0, w.seqlen_q, step)) | set(range(w.seqlen_q - tail, w.seqlen_q))
    qs |= {t - off for t in range(*around) if 0 <= t - off < w.seqlen_q}
    qs = sorted(q for q in qs if 0 <= q < w.seqlen_q)
    return np.array([(b, i, g) for b in range(w.batch) for i in qs for g in range(w.heads_kv)],
                    dtype=np.int64)


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_forward_parity_small(w):
    rows = sampled_rows(w) if w.heads_q * w.seqlen_q * w.seqlen_k > 1e11 else None
    msgs, stats = parity(w, rows=rows)
    print(w.name, stats, flush=True)
    assert not msgs, "\n".join(msgs)


def test_explicit_softmax_scale():
    w = W("explicit_scale", 1, 300, 1000, 8, 2, topk=4)
    t = inputs_for(w)
    out, lse = msa.msa_forward(t["q"], t["k"], t["v"], t["q_idx"], t["k_idx"], topk=4,
                               softmax_scale=0.05, return_lse=True)
    p = oracle.Problem.of(w, softmax_scale=0.05)
    h = host_inputs(t)
    ref = oracle.forward(p, h["q"], h["k"], h["v"], h["q_idx"], h["k_idx"])
    o = out.float().cpu().numpy().reshape(ref["out"].shape).astype(np.float64)
    check_close("explicit scale out", o, ref["out"])
    l = lse.cpu().numpy().transpose(0, 2, 1).reshape(ref["lse"].shape)
    assert np.abs(l - ref["lse"]).max() < 1e-3


@pytest.mark.parametrize("shape", [(2, 700, 1100, 4, 4, 64, 5), (1, 1500, 2600, 64, 8, 128, 8)],
                         ids=["mha", "g8"])
def test_sharp_softmax_forward(shape):
    """q and k scaled by 6 (logits with a standard deviation near 36, nearly
    one-hot rows) and the integer q_idx by 4: block scores and selections
    bit-exact, out and lse within the tolerance rule, on every row."""
    B, Sq, Sk, Hq, Hkv, Didx, k = shape
    w = W(f"sharp_{Hq}x{Hkv}", B, Sq, Sk, Hq, Hkv, Didx=Didx, topk=k)
    t = inputs_for(w)
    with torch.no_grad():
        t["q"].mul_(6)
        t["k"].mul_(6)
        t["q_idx"].mul_(4)
    dev = run_device(w, t)
    p = oracle.Problem.of(w)
    rows = p.all_rows()
    h = host_inputs(t)
    ref = oracle.forward(p, h["q"], h["k"], h["v"], h["q_idx"], h["k_idx"], rows=rows)
    msgs, stats = compare(w, dev, ref, rows, label=w.name)
    print(w.name, stats, flush=True)
    assert not msgs, "\n".join(msgs)


def test_massive_ties_take_the_exact_path():
    """k_idx = 0: every block score is 0, so the tie rule alone decides
    (blocks 0..k-2 plus the local block), on rows wider than the survivor
    buffer (more than 256 candidates)."""
    w = W("ties", 1, 64, 40000, 4, 2, Didx=64, topk=16)
    t = inputs_for(w)
    t["k_idx"].zero_()
    dev = run_device(w, t)
    idx = dev["idx"].cpu().numpy()
    local = (np.arange(64) + 40000 - 64) // 128
    for i in range(64):
        exp = list(range(15)) + [local[i]]
        assert (idx[0, :, i] == exp).all()
    assert (dev["bm"].cpu().numpy()[0, :, :, : local[0]] == 0).all()


def test_few_distinct_scores():
    """k_idx in {0, 1}: heavy ties, but the survivors fit the fast path."""
    w = W("fewvals", 1, 200, 30000, 8, 2, topk=16)
    t = inputs_for(w)
    t["k_idx"].copy_((t["k_idx"] > 2).to(torch.bfloat16))
    t["q_idx"].copy_((t["q_idx"] > 2).to(torch.bfloat16))
    dev = run_device(w, t)
    p = oracle.Problem.of(w)
    h = host_inputs(t)
    ref = oracle.forward(p, h["q"], h["k"], h["v"], h["q_idx"], h["k_idx"])
    msgs, _ = compare(w, dev, ref, p.all_rows())
    assert not msgs, "\n".join(msgs)


def test_sparse_attn_fwd_with_caller_selection():
    """msa_sparse_attn_fwd on a caller-made selection: unsorted, -1 entries
    in the middle, local block anywhere."""
    w = W("caller_sel", 2, 200, 2000, 8, 2, topk=6)
    t = inputs_for(w)
    rng = np.random.default_rng(3)
    B, Hkv, Sq, k = 2, 2, 200, 6
    sel = np.full((B, Hkv, Sq, k), -1, dtype=np.int32)
    for b in range(B):
        for g in range(Hkv):
            for i in range(Sq):
                local = (i + 1800) // 128
                others = rng.choice(local, size=min(local, rng.integers(0, k)), replace=False)
                row = np.concatenate([others, [local]])
                slots = rng.choice(k, size=len(row), replace=False)
                sel[b, g, i, slots] = row
    idx = torch.from_numpy(sel).cuda()
    out, lse = msa.msa_sparse_attn_fwd(t["q"], t["k"], t["v"], idx, return_lse=True)
    torch.cuda.synchronize()
    p = oracle.Problem.of(w)
    h = host_inputs(t)
    rows = p.all_rows()
    sel_rows = sel[rows[:, 0], rows[:, 2], rows[:, 1]]
    ref_out, ref_lse = oracle.attention(p, h["q"], h["k"], h["v"], sel_rows, rows)
    o = out.float().cpu().numpy()
    G = w.group
    got = np.stack([o[b, i, g * G:(g + 1) * G] for b, i, g in rows]).astype(np.float64)
    check_close("caller selection out", got, ref_out)
    l = lse.cpu().numpy()
    got_l = np.stack([l[b, g * G:(g + 1) * G, i] for b, i, g in rows])
    assert np.abs(got_l - ref_lse).max() < 1e-3


@pytest.mark.parametrize("shape", [("dense_sel_g8", 1, 1100, 1300, 16, 2, 12),  # offset 200: tiles straddle blocks
                                   ("dense_sel_g1", 2, 700, 700, 4, 4, 8)],
                         ids=lambda s: s[0])
def test_dense_rows_take_only_their_selection(shape):
    """Rows whose local block is below topk go through the query-stationary
    dense tiles.  On a caller's selection each row takes only the blocks it
    names: here random subsets of its prefix (any size, unsorted, -1 entries),
    some rows their local block alone."""
    name, B, Sq, Sk, Hq, Hkv, k = shape
    w = W(name, B, Sq, Sk, Hq, Hkv, topk=k)
    assert (Sq - 1 + Sk - Sq) // 128 < k  # every row is a dense row
    t = inputs_for(w)
    rng = np.random.default_rng(5)
    sel = np.full((B, Hkv, Sq, k), -1, dtype=np.int32)
    for b in range(B):
        for g in range(Hkv):
            for i in range(Sq):
                local = (i + Sk - Sq) // 128
                n_other = 0 if i % 7 == 0 else int(rng.integers(0, local + 1))
                others = rng.choice(local, size=min(local, n_other), replace=False)
                row = np.concatenate([others, [local]])
                slots = rng.choice(k, size=len(row), replace=False)
                sel[b, g, i, slots] = row
    idx = torch.from_numpy(sel).cuda()
    out, lse = msa.msa_sparse_attn_fwd(t["q"], t["k"], t["v"], idx, return_lse=True)
    torch.cuda.synchronize()
    p = oracle.Problem.of(w)
    h = host_inputs(t)
    rows = p.all_rows()
    sel_rows = sel[rows[:, 0], rows[:, 2], rows[:, 1]]
    ref_out, ref_lse = oracle.attention(p, h["q"], h["k"], h["v"], sel_rows, rows)
    o = out.float().cpu().numpy()
    G = w.group
    got = np.stack([o[b, i, g * G:(g + 1) * G] for b, i, g in rows]).astype(np.float64)
    check_close(f"{name} out", got, ref_out)
    l = lse.cpu().numpy()
    got_l = np.stack([l[b, g * G:(g + 1) * G, i] for b, i, g in rows])
    assert np.abs(got_l - ref_lse).max() < 1e-3


def test_deterministic():
    w = W("determinism", 1, 1500, 4000, 16, 2, topk=8)
    t = inputs_for(w)
    a = run_device(w, t)
    b = run_device(w, t)
    for key in ("bm", "idx", "out", "lse"):
        assert torch.equal(a[key], b[key]), key


def test_empty_problem_launches_nothing():
    d = msa.Dims.make(0, 0, 0, 8, 2)
    assert msa.lib().msa_forward(d, None, None, None, None, None, None, None, None, None, 0, None) == 0


def test_profiled_forward_matches_forward():
    """msa_forward_profiled only adds event records: identical results."""
    w = W("profiled", 1, 700, 3000, 16, 2, topk=8)
    t = inputs_for(w)
    a = run_device(w, t)
    d = msa.dims_of(t["q"], t["k"], t["q_idx"], t["k_idx"], topk=8)
    chunks = msa.msa_attn_chunks(d, msa.ENTRY_FORWARD)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(msa.n_stage_events(chunks))]
    for e in evs:
        e.record()
    out, lse, idx = msa.msa_forward(t["q"], t["k"], t["v"], t["q_idx"], t["k_idx"], topk=8,
                                    return_lse=True, return_idx=True,
                                    stage_events=[e.cuda_event for e in evs])
    torch.cuda.synchronize()
    assert torch.equal(out, a["out"]) and torch.equal(lse, a["lse"]) and torch.equal(idx, a["idx"])
    for s in range(len(evs) // 2):
        assert evs[2 * s].elapsed_time(evs[2 * s + 1]) >= 0.0
