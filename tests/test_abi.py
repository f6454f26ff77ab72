"""The C-ABI library loads, exports what include/msa.h declares, and rejects
bad arguments on the host before any HIP call (no GPU needed: only error
paths are exercised, nothing is launched).  Every call below must fail
validation: the pointers are fake addresses that are never dereferenced."""
import ctypes
import os
import re

import pytest

import block_sparse_gqa_scores_amd as msa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
A = ctypes.c_void_p(0x10000)       # a 16-byte aligned, never dereferenced address
MIS = ctypes.c_void_p(0x10008)     # misaligned
NULL = None


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "msa.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(msa_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol():
    L = msa.lib()
    names = declared_symbols()
    assert set(names) == set(msa.EXPORTED)
    for n in names:
        assert hasattr(L, n), n


def dims(**kw):
    base = dict(batch=1, seqlen_q=256, seqlen_k=512, num_heads_q=8, num_heads_kv=2, head_dim=128,
                index_dim=128, block_size=128, topk=16, causal=1, softmax_scale=0.0)
    base.update(kw)
    return msa.Dims.make(**base)


def fwd(d, q=A, k=A, v=A, qi=A, ki=A, out=A, lse=NULL, idx=NULL, ws=A, nbytes=None):
    if nbytes is None:
        nbytes = 1 << 40
    return msa.lib().msa_forward(None if d is None else ctypes.byref(d), q, k, v, qi, ki, out, lse,
                                 idx, ws, nbytes, None)


def attn(d, q=A, k=A, v=A, idx=A, out=A, lse=NULL, ws=A, nbytes=1 << 40):
    return msa.lib().msa_sparse_attn_fwd(ctypes.byref(d), q, k, v, idx, out, lse, ws, nbytes, None)


def scores(d, qi=A, ki=A, bm=A):
    return msa.lib().msa_index_scores(ctypes.byref(d), qi, ki, bm, None)


def topk(d, bm=A, idx=A):
    return msa.lib().msa_block_topk(ctypes.byref(d), bm, idx, None)


def bmask(d, idx=A, mask=A):
    return msa.lib().msa_block_mask(None if d is None else ctypes.byref(d), idx, mask, None)


def mblocks(d, mask=A, idx=A):
    return msa.lib().msa_mask_blocks(None if d is None else ctypes.byref(d), mask, idx, None)


def kl(d, q=A, k=A, qi=A, ki=A, idx=A, lse=A, rows=A, loss=A, lsei=A, ws=A, nbytes=1 << 40):
    return msa.lib().msa_kl_loss_fwd(None if d is None else ctypes.byref(d), q, k, qi, ki, idx, lse,
                                     rows, loss, lsei, ws, nbytes, None)


def klb(d, q=A, k=A, qi=A, ki=A, idx=A, lse=A, lsei=A, grad=1.0, dqi=A, dki=A, ws=A, nbytes=1 << 40):
    return msa.lib().msa_kl_loss_bwd(None if d is None else ctypes.byref(d), q, k, qi, ki, idx, lse,
                                     lsei, grad, dqi, dki, ws, nbytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(batch=-1), 2), (dict(seqlen_q=600), 2), (dict(num_heads_q=7), 2), (dict(topk=0), 2),
    (dict(block_size=0), 2), (dict(num_heads_kv=0), 2), (dict(head_dim=0), 2),
    (dict(softmax_scale=float("nan")), 2), (dict(softmax_scale=-0.5), 2),
    (dict(causal=0), 3), (dict(head_dim=64), 3), (dict(block_size=64), 3), (dict(topk=65), 3),
    (dict(index_dim=96), 3), (dict(num_heads_q=6, num_heads_kv=2), 3),
])
def test_forward_rejects_dims(kw, status):
    assert fwd(dims(**kw)) == status


def test_entry_specific_checks():
    # index_dim only matters to the index branch; head_dim only to the main branch
    assert scores(dims(index_dim=96)) == 3
    assert topk(dims(block_size=64)) == 3 and topk(dims(topk=0)) == 2
    assert attn(dims(index_dim=96, head_dim=64)) == 3
    assert scores(dims(head_dim=64, index_dim=64, seqlen_q=600)) == 2


def test_null_and_misaligned_pointers():
    d = dims()
    assert fwd(None) == 1
    assert fwd(d, q=NULL) == 1
    assert fwd(d, ki=NULL) == 1
    assert fwd(d, ws=NULL, nbytes=0) == 1
    assert fwd(d, v=MIS) == 4
    assert fwd(d, lse=MIS) == 4
    assert fwd(d, idx=MIS) == 4
    assert attn(d, idx=NULL) == 1
    assert attn(d, out=MIS) == 4
    assert scores(d, bm=NULL) == 1
    assert scores(d, qi=MIS) == 4
    assert topk(d, idx=NULL) == 1
    assert topk(d, bm=MIS) == 4
    assert bmask(None) == 1 and mblocks(None) == 1
    assert bmask(d, idx=NULL) == 1 and bmask(d, mask=NULL) == 1
    assert mblocks(d, mask=NULL) == 1 and mblocks(d, idx=NULL) == 1
    assert bmask(d, idx=MIS) == 4 and mblocks(d, mask=MIS) == 4
    assert kl(None) == 1
    for kw in ("q", "k", "qi", "ki", "idx", "lse"):
        assert kl(d, **{kw: NULL}) == 1, kw
        assert kl(d, **{kw: MIS}) == 4, kw
    assert kl(d, rows=MIS) == 4 and kl(d, loss=MIS) == 4 and kl(d, ws=MIS) == 4
    assert kl(d, lsei=MIS) == 4
    assert klb(None) == 1
    for kw in ("q", "k", "qi", "ki", "idx", "lse", "lsei", "dqi", "dki"):
        assert klb(d, **{kw: NULL}) == 1, kw
        assert klb(d, **{kw: MIS}) == 4, kw
    assert klb(d, ws=NULL, nbytes=0) == 1 and klb(d, ws=MIS) == 4
    assert klb(d, grad=float("nan")) == 2 and klb(d, grad=float("inf")) == 2
    assert kl(d, ws=NULL, nbytes=0) == 1


def bwd(d, q=A, k=A, v=A, idx=A, out=A, lse=A, do=A, dq=A, dk=A, dv=A, ws=A, nbytes=1 << 40):
    return msa.lib().msa_sparse_attn_bwd(None if d is None else ctypes.byref(d), q, k, v, idx, out, lse,
                                         do, dq, dk, dv, ws, nbytes, None)


def test_bwd_entry_checks():
    d = dims()
    assert bwd(None) == 1
    for kw in ("q", "k", "v", "idx", "out", "lse", "do", "dq", "dk", "dv"):
        assert bwd(d, **{kw: NULL}) == 1, kw
        assert bwd(d, **{kw: MIS}) == 4, kw
    assert bwd(d, ws=NULL, nbytes=0) == 1 and bwd(d, ws=MIS) == 4
    full = msa.msa_workspace_bytes(d, msa.ENTRY_SPARSE_ATTN_BWD)
    need = msa.msa_workspace_min_bytes(d, msa.ENTRY_SPARSE_ATTN_BWD)
    rows = d.batch * d.num_heads_kv * d.seqlen_q
    G = d.num_heads_q // d.num_heads_kv
    assert full >= rows * d.topk * G * (128 * 3 // 2 + 16)  # 12-bit dq record + scales per edge and head
    assert 0 < need <= full
    assert bwd(d, nbytes=need - 1) == 5
    # the main branch only: index_dim does not matter (the workspace check is reached)
    assert bwd(dims(index_dim=96), nbytes=need - 1) == 5
    for kw, status in ((dict(head_dim=64), 3), (dict(num_heads_q=6), 3), (dict(causal=0), 3),
                       (dict(softmax_scale=-1.0), 2), (dict(topk=65), 3)):
        assert bwd(dims(**kw)) == status, kw
    e = dims(batch=0)
    assert bwd(e, q=NULL, k=NULL, v=NULL, idx=NULL, out=NULL, lse=NULL, do=NULL, dq=NULL, dk=NULL,
               dv=NULL, ws=NULL, nbytes=0) == 0


def test_kl_bwd_entry_checks():
    d = dims()
    full = msa.msa_workspace_bytes(d, msa.ENTRY_KL_LOSS_BWD)
    need = msa.msa_workspace_min_bytes(d, msa.ENTRY_KL_LOSS_BWD)
    rows = d.batch * d.num_heads_kv * d.seqlen_q
    assert full >= rows * d.topk * (2 * d.index_dim + 16)
    assert 0 < need < full
    assert klb(d, nbytes=need - 1) == 5
    for kw, status in ((dict(index_dim=96), 3), (dict(head_dim=64), 3), (dict(causal=0), 3)):
        assert klb(dims(**kw)) == status, kw
    assert klb(dims(batch=0), q=NULL, k=NULL, qi=NULL, ki=NULL, idx=NULL, lse=NULL, lsei=NULL, dqi=NULL,
               dki=NULL, ws=NULL, nbytes=0) == 0


def fb(d, q=A, k=A, v=A, qi=A, ki=A, idx=A, out=A, lse=A, lsei=A, do=A, grad=1.0, dq=A, dk=A, dv=A, dqi=A, dki=A,
       ws=A, nbytes=1 << 40):
    return msa.lib().msa_backward(None if d is None else ctypes.byref(d), q, k, v, qi, ki, idx, out, lse, lsei, do,
                                  grad, dq, dk, dv, dqi, dki, ws, nbytes, None)


def test_fused_bwd_entry_checks():
    d = dims()
    assert fb(None) == 1
    for kw in ("q", "k", "v", "qi", "ki", "idx", "out", "lse", "lsei", "do", "dq", "dk", "dv", "dqi", "dki"):
        assert fb(d, **{kw: NULL}) == 1, kw
        assert fb(d, **{kw: MIS}) == 4, kw
    assert fb(d, ws=NULL, nbytes=0) == 1 and fb(d, ws=MIS) == 4
    assert fb(d, grad=float("inf")) == 2
    full = msa.msa_workspace_bytes(d, msa.ENTRY_BACKWARD)
    need = msa.msa_workspace_min_bytes(d, msa.ENTRY_BACKWARD)
    # both passes' records: at least the two separate entry points' smallest workspaces' records
    assert full >= msa.msa_workspace_bytes(d, msa.ENTRY_SPARSE_ATTN_BWD)
    assert full >= msa.msa_workspace_bytes(d, msa.ENTRY_KL_LOSS_BWD)
    assert 0 < need <= full
    assert fb(d, nbytes=need - 1) == 5
    assert msa.msa_attn_chunks(d, msa.ENTRY_BACKWARD, full) == 1
    assert msa.msa_attn_chunks(d, msa.ENTRY_BACKWARD, need) >= 1
    assert msa.msa_attn_chunks(d, msa.ENTRY_BACKWARD, need - 1) == 0
    for kw, status in ((dict(index_dim=96), 3), (dict(head_dim=64), 3), (dict(causal=0), 3),
                       (dict(softmax_scale=-1.0), 2), (dict(topk=65), 3)):
        assert fb(dims(**kw)) == status, kw
    assert fb(dims(batch=0), **{k: NULL for k in ("q", "k", "v", "qi", "ki", "idx", "out", "lse", "lsei", "do",
                                                    "dq", "dk", "dv", "dqi", "dki", "ws")}, nbytes=0) == 0


def test_kl_entry_checks_both_branches():
    for kw, status in ((dict(index_dim=96), 3), (dict(head_dim=64), 3), (dict(num_heads_q=6), 3),
                       (dict(softmax_scale=-1.0), 2), (dict(causal=0), 3), (dict(topk=0), 2)):
        assert kl(dims(**kw)) == status, kw
    d = dims()
    need = msa.msa_workspace_bytes(d, msa.ENTRY_KL_LOSS_FWD)
    rows = d.batch * d.num_heads_kv * d.seqlen_q
    # 20 bytes of records per selected block of every row, besides the edge lists
    assert need >= rows * d.topk * (16 + 4 + 4)
    assert kl(d, nbytes=need - 1) == 5
    with pytest.raises(msa.MsaError):
        msa.msa_workspace_bytes(dims(index_dim=96), msa.ENTRY_KL_LOSS_FWD)


def _al(x):
    return (x + 255) // 256 * 256


def test_workspace_checks():
    d = dims()
    need = msa.msa_workspace_bytes(d, msa.ENTRY_FORWARD)
    rows = d.batch * d.num_heads_kv * d.seqlen_q
    attn_ws = msa.msa_workspace_bytes(d, msa.ENTRY_SPARSE_ATTN_FWD)
    # k <= 16 with more than 32 rows: scores and selection are fused, so the
    # forward workspace holds the selection and the attention scratch only.
    assert need == _al(rows * d.topk * 4) + attn_ws
    # A wider Top-k stages the block scores in the workspace first.
    d2 = dims(topk=32)
    attn2 = msa.msa_workspace_bytes(d2, msa.ENTRY_SPARSE_ATTN_FWD)
    assert msa.msa_workspace_bytes(d2, msa.ENTRY_FORWARD) == (
        _al(rows * d2.n_blk * 4) + _al(rows * 32 * 4) + attn2)
    # So does decode (at most 32 rows), which scores with the decode kernel.
    d3 = dims(seqlen_q=1, seqlen_k=4096)
    attn3 = msa.msa_workspace_bytes(d3, msa.ENTRY_SPARSE_ATTN_FWD)
    assert msa.msa_workspace_bytes(d3, msa.ENTRY_FORWARD) == (
        _al(2 * d3.n_blk * 4) + _al(2 * 16 * 4) + attn3)
    min_f = msa.msa_workspace_min_bytes(d, msa.ENTRY_FORWARD)
    min_a = msa.msa_workspace_min_bytes(d, msa.ENTRY_SPARSE_ATTN_FWD)
    # The minimum differs from the designed size only in the attention part.
    assert 0 < min_a < attn_ws and min_f == need - attn_ws + min_a
    assert fwd(d, nbytes=min_f - 1) == 5
    assert attn(d, nbytes=min_a - 1) == 5
    assert msa.msa_workspace_bytes(d, msa.ENTRY_INDEX_SCORES) == 0
    assert msa.msa_workspace_bytes(d, msa.ENTRY_BLOCK_TOPK) == 0
    with pytest.raises(msa.MsaError):
        msa.msa_workspace_bytes(dims(causal=0), msa.ENTRY_FORWARD)
    with pytest.raises(msa.MsaError):
        msa.msa_workspace_bytes(d, 17)


def test_empty_problems_are_ok_without_pointers():
    for kw in (dict(batch=0), dict(seqlen_q=0)):
        d = dims(**kw)
        assert fwd(d, q=NULL, k=NULL, v=NULL, qi=NULL, ki=NULL, out=NULL, ws=NULL, nbytes=0) == 0
        assert attn(d, q=NULL, k=NULL, v=NULL, idx=NULL, out=NULL, ws=NULL, nbytes=0) == 0
        assert scores(d, qi=NULL, ki=NULL, bm=NULL) == 0
        assert topk(d, bm=NULL, idx=NULL) == 0
        assert bmask(d, idx=NULL, mask=NULL) == 0 and mblocks(d, mask=NULL, idx=NULL) == 0
        assert kl(d, q=NULL, k=NULL, qi=NULL, ki=NULL, idx=NULL, lse=NULL, rows=NULL, loss=NULL,
                  ws=NULL, nbytes=0) == 0
        assert msa.msa_workspace_bytes(d, msa.ENTRY_KL_LOSS_FWD) == 0
        assert msa.msa_workspace_bytes(d, msa.ENTRY_FORWARD) == 0


def test_mask_entries_check_dims():
    assert bmask(dims(topk=0)) == 2 and mblocks(dims(topk=0)) == 2
    assert bmask(dims(block_size=64)) == 3 and mblocks(dims(causal=0)) == 3
    assert bmask(dims(topk=65)) == 3 and mblocks(dims(seqlen_q=600)) == 2


def test_size_limits():
    # rows * topk must stay below 2^31 (32-bit slot ids)
    assert fwd(dims(batch=1 << 10, seqlen_q=1 << 17, seqlen_k=1 << 17, topk=16)) == 3


def test_noalloc_host_checks():
    """msa_forward_noalloc makes msa_forward's host checks before any HIP call,
    and rejects a problem whose smallest workspace exceeds its static scratch
    (only failure paths here: nothing may be launched)."""
    L = msa.lib()

    def call(d, q=A, k=A, v=A, qi=A, ki=A, out=A, lse=NULL, idx=NULL):
        return L.msa_forward_noalloc(None if d is None else ctypes.byref(d), q, k, v, qi, ki, out, lse, idx, None)

    assert call(None) == 1
    assert call(dims(causal=0)) == 3 and call(dims(topk=0)) == 2
    assert call(dims(), q=NULL) == 1 and call(dims(), out=MIS) == 4 and call(dims(), lse=MIS) == 4
    assert call(dims(batch=0), q=NULL, k=NULL, v=NULL, qi=NULL, ki=NULL, out=NULL) == 0
    # topk 32 stages block scores: 8 x 32768 rows x 256 blocks x 4 bytes = 256 MiB alone
    big = dims(seqlen_q=32768, seqlen_k=32768, num_heads_q=64, num_heads_kv=8, topk=32)
    assert msa.msa_workspace_min_bytes(big, msa.ENTRY_FORWARD) > msa.NOALLOC_SCRATCH_BYTES
    assert call(big) == 5


def test_status_strings():
    for code, name in msa.STATUS_NAMES.items():
        assert msa.msa_status_str(code) == name
    assert msa.msa_status_str(99) == "MSA_ERR_UNKNOWN"


def test_profiled_entry_rejects_bad_events():
    d = dims()
    L = msa.lib()
    ev = (ctypes.c_void_p * 10)(*([0x20000] * 10))
    args = (ctypes.byref(d), A, A, A, A, A, A, NULL, NULL, A, 1 << 40, None)
    assert L.msa_forward_profiled(*args, None, 10) == 1
    assert L.msa_forward_profiled(*args, ev, 3) == 2
    assert msa.n_stage_events(1) == 10
    assert L.msa_forward_profiled(*args, ev, 9) == 2      # one chunk records 10 events
    holes = (ctypes.c_void_p * 10)(*([0x20000] * 9 + [0]))
    assert L.msa_forward_profiled(*args, holes, 10) == 1
    bad = dims(causal=0)
    assert L.msa_forward_profiled(ctypes.byref(bad), *args[1:], ev, 10) == 3


def test_attn_chunks():
    assert msa.msa_attn_chunks(dims()) == 1
    assert msa.msa_attn_chunks(dims(causal=0)) == 0
    assert msa.msa_attn_chunks(dims(batch=0)) == 0
    # partials of 262144 queries x 8 groups x 16 blocks exceed one chunk's budget
    big = dims(seqlen_q=262144, seqlen_k=262144, num_heads_q=64, num_heads_kv=8)
    assert msa.msa_attn_chunks(big) >= 2
    assert msa.msa_attn_chunks(dims(), msa.ENTRY_INDEX_SCORES, 1 << 30) == 0
    assert msa.msa_attn_chunks(dims(), msa.ENTRY_KL_LOSS_FWD) == 1


@pytest.mark.parametrize("entry", [msa.ENTRY_SPARSE_ATTN_FWD, msa.ENTRY_FORWARD, msa.ENTRY_SPARSE_ATTN_BWD,
                                   msa.ENTRY_KL_LOSS_BWD])
def test_chunks_follow_the_workspace(entry):
    """The query chunk is the largest that fits ws_bytes: the designed size
    runs one chunk here, the minimum one query per chunk, and sizes between
    give whole 128-query blocks, more chunks for less memory."""
    d = dims(seqlen_q=1000, seqlen_k=1300, topk=6)
    full = msa.msa_workspace_bytes(d, entry)
    low = msa.msa_workspace_min_bytes(d, entry)
    assert msa.msa_attn_chunks(d, entry, full) == 1
    assert msa.msa_attn_chunks(d, entry, low) == 1000
    assert msa.msa_attn_chunks(d, entry, low - 1) == 0
    assert msa.msa_attn_chunks(d, entry, full * 4) == 1   # never larger than the designed chunks
    seen = []
    for frac in (0.9, 0.7, 0.5, 0.35, 0.2):
        n = msa.msa_attn_chunks(d, entry, int(low + frac * (full - low)))
        assert 1 <= n <= 1000
        # chunks of 128 m queries (m = 1 .. 7) give 8, 4, 3, 2 or 2 chunks;
        # more than 8 means chunks below one 128-query block
        assert n in (1, 2, 3, 4, 8) or n > 8, n
        seen.append(n)
    assert seen == sorted(seen) and seen[-1] >= 2
