"""GPU parity of the combined backward (msa_backward through the C ABI):
both gradients in one call, the two passes sharing each query chunk's edge
buckets.

The combined call runs the main backward's kernels and the loss backward's,
in the same summation orders, so at one query chunk each output must equal
the separate entry point's bit for bit (msa_sparse_attn_bwd,
msa_kl_loss_bwd), on every shape those tests cover.  With several query chunks (forced through a small workspace) the
outputs are compared with the oracle's gradients on every row and key, by
the one tolerance rule of gpu_util.check_close.  Outputs and workspaces are
poisoned before every call.
"""
import pytest
import torch

import block_sparse_gqa_scores_amd as msa
import synth
from gpu_util import (backward_against_oracle, fused_backward as fused, inputs_for, poisoned_workspace,
                      prepare_backward as prepare, spread_index_queries)

pytestmark = pytest.mark.gpu


def W(name, B, Sq, Sk, Hq, Hkv, Didx=128, topk=16, **kw):
    return synth.Workload(name, B, Sq, Sk, Hq, Hkv, index_dim=Didx, topk=topk, **kw)


def separate(w, t, out, lse, idx, lse_idx, grad=1.0):
    d = msa.dims_of(t["q"], t["k"], t["q_idx"], t["k_idx"], topk=w.topk)
    dq, dk, dv = msa.msa_sparse_attn_bwd(
        t["q"], t["k"], t["v"], idx, out, lse, t["dout"],
        workspace=poisoned_workspace(msa.msa_workspace_bytes(d, msa.ENTRY_SPARSE_ATTN_BWD)))
    dqi, dki = msa.msa_kl_loss_bwd(
        t["q"], t["k"], t["q_idx"], t["k_idx"], idx, lse, lse_idx, grad,
        workspace=poisoned_workspace(msa.msa_workspace_bytes(d, msa.ENTRY_KL_LOSS_BWD)))
    torch.cuda.synchronize()
    return dq, dk, dv, dqi, dki


NAMES = ("dq", "dk", "dv", "dq_idx", "dk_idx")

CASES = [
    W("fb_4k", 1, 4096, 4096, 8, 2, Didx=64),                  # two query windows, D_idx 64
    W("fb_ragged", 2, 700, 1000, 8, 2, topk=5),                # S_k % 128 != 0, S_q < S_k
    W("fb_gqa8", 1, 2600, 2600, 64, 8),                        # G = 8
    W("fb_mha", 1, 600, 777, 4, 4, Didx=64, topk=3),           # G = 1
    W("fb_g2", 1, 500, 1300, 8, 4, topk=6),                    # G = 2
    W("fb_g16", 1, 500, 640, 32, 2, topk=2),                   # G = 16
    W("fb_g32", 2, 300, 300, 32, 1, Didx=64, topk=4),          # G = 32
    W("fb_decode", 3, 1, 5000, 16, 2, Didx=64),                # S_q = 1
    W("fb_gain", 1, 1500, 3000, 16, 2, gain=True, topk=6),     # uneven blocks
    W("fb_hkv10", 1, 400, 900, 20, 10, topk=4),                # H_kv = 10 (G = 2): groups past the first eight
    W("fb_split", 1, 2048, 2048, 32, 1, Didx=64, topk=3, gain=True),  # block 0's dK, dV split over workgroups
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_fused_equals_separate(w):
    t = inputs_for(w)
    out, lse, idx, lse_idx = prepare(w, t)
    d = msa.dims_of(t["q"], t["k"], t["q_idx"], t["k_idx"], topk=w.topk)
    nbytes = msa.msa_workspace_bytes(d, msa.ENTRY_BACKWARD)
    assert msa.msa_attn_chunks(d, msa.ENTRY_BACKWARD, nbytes) == 1
    got = fused(w, t, out, lse, idx, lse_idx, grad=0.75)
    ref = separate(w, t, out, lse, idx, lse_idx, grad=0.75)
    for name, a, b in zip(NAMES, got, ref):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{w.name} {name} differs"


def test_fused_spread_student_equals_separate():
    """With a spread student (two +-1 channels per index row) every token's
    P_idx enters g; the combined call still equals the separate ones."""
    w = W("fb_spread_g8", 1, 700, 3000, 64, 8, topk=12)
    t = spread_index_queries(w, inputs_for(w))
    out, lse, idx, lse_idx = prepare(w, t)
    got = fused(w, t, out, lse, idx, lse_idx)
    ref = separate(w, t, out, lse, idx, lse_idx)
    for name, a, b in zip(NAMES, got, ref):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{w.name} {name} differs"


@pytest.mark.parametrize("chunks", [2, 3])
def test_fused_chunked_against_oracle(chunks):
    """A workspace that fits only part of the queries runs the combined call in
    several chunks (dk, dv and dk_idx carry fp32 sums across them); every
    row's dq, dq_idx and every key's dk, dv, dk_idx against the oracle."""
    w = W("fb_chunks", 1, 1024, 1536, 16, 2, Didx=64, topk=6)
    t = inputs_for(w)
    out, lse, idx, lse_idx = prepare(w, t)
    d = msa.dims_of(t["q"], t["k"], t["q_idx"], t["k_idx"], topk=w.topk)
    lo, hi = msa.msa_workspace_min_bytes(d, msa.ENTRY_BACKWARD), msa.msa_workspace_bytes(d, msa.ENTRY_BACKWARD)
    nbytes = next(b for b in range(lo, hi + 1, max(1, (hi - lo) // 4096))
                  if msa.msa_attn_chunks(d, msa.ENTRY_BACKWARD, b) <= chunks)
    assert msa.msa_attn_chunks(d, msa.ENTRY_BACKWARD, nbytes) == chunks
    grads = fused(w, t, out, lse, idx, lse_idx, ws_bytes=nbytes)
    backward_against_oracle(w, t, grads, idx, f"{chunks} chunks")


def test_fused_without_queries_writes_zero_key_gradients():
    """seqlen_q = 0 with keys present: dk = dv = dk_idx = 0."""
    dk = torch.full((2, 300, 2, 128), 3.0, dtype=torch.bfloat16, device="cuda")
    dv = torch.full_like(dk, 5.0)
    dki = torch.full((2, 300, 64), 7.0, dtype=torch.bfloat16, device="cuda")
    d = msa.Dims.make(2, 0, 300, 8, 2, index_dim=64)
    rc = msa.lib().msa_backward(d, None, None, None, None, None, None, None, None, None, None, 1.0, None,
                                dk.data_ptr(), dv.data_ptr(), None, dki.data_ptr(), None, 0, None)
    torch.cuda.synchronize()
    assert rc == 0 and not dk.float().any() and not dv.float().any() and not dki.float().any()


SHARP = [W("fb_sharp_mha", 2, 700, 1100, 4, 4, Didx=64, topk=5),
         W("fb_sharp_g8", 1, 1500, 2600, 64, 8, topk=8)]


@pytest.mark.parametrize("w", SHARP, ids=lambda w: w.name)
def test_sharp_softmax_against_oracle(w):
    """Sharp main and index softmaxes (q and k scaled by 6, the integer q_idx
    by 4): a block that holds almost none of a row's mass in both gives
    gradient records whose largest magnitude is subnormal, which must encode
    as zeros rather than inf or NaN.  Every row and key against the oracle."""
    t = inputs_for(w)
    with torch.no_grad():
        t["q"].mul_(6)
        t["k"].mul_(6)
        t["q_idx"].mul_(4)
    out, lse, idx, lse_idx = prepare(w, t)
    grads = fused(w, t, out, lse, idx, lse_idx)
    backward_against_oracle(w, t, grads, idx, w.name)


def test_zero_upstream_gradient():
    """dO = 0: dq, dk, dv are exactly zero, and dq_idx, dk_idx (which do not
    depend on dO) equal the call with the seeded dO bit for bit."""
    w = W("fb_zero_dout", 1, 1300, 2300, 64, 8, topk=8)
    t = inputs_for(w)
    out, lse, idx, lse_idx = prepare(w, t)
    ref = fused(w, t, out, lse, idx, lse_idx)
    t["dout"].zero_()
    got = fused(w, t, out, lse, idx, lse_idx)
    for name, g in zip(NAMES[:3], got[:3]):
        assert not g.float().abs().max().item(), f"{name} is not zero"
    for name, a, b in zip(NAMES[3:], got[3:], ref[3:]):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{name} depends on dO"


def test_uniform_attention_against_oracle():
    """q = 0: every visible token gets the same weight (the main scores are
    all zero) while the selection still follows the index branch; forward
    selection and every gradient against the oracle."""
    w = W("fb_uniform", 2, 600, 1000, 4, 4, Didx=64, topk=5)
    t = inputs_for(w)
    t["q"].zero_()
    out, lse, idx, lse_idx = prepare(w, t)
    grads = fused(w, t, out, lse, idx, lse_idx)
    backward_against_oracle(w, t, grads, idx, w.name)
