"""GPU parity of the block-mask selection format (Sparse Attention Part II,
section 4.3) against the oracle: masks bit for bit, traversals element for
element, on selections from the forward path, on random selections with
out-of-range entries, and on random masks (stray bits past the last block,
rows with more set bits than the output holds, empty rows)."""
import numpy as np
import pytest
import torch

import block_sparse_gqa_scores_amd as msa
import oracle
import synth
from gpu_util import inputs_for

pytestmark = pytest.mark.gpu


def as_u32(t):
    return t.cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("w", [
    synth.Workload("mask_small", 2, 700, 1000, 8, 2, topk=5),
    synth.Workload("mask_gqa8", 1, 2600, 2600, 64, 8),
    synth.Workload("mask_decode", 3, 1, 5000, 16, 2, index_dim=64),
    synth.Workload("mask_k64", 1, 130, 9000, 4, 1, topk=64),
], ids=lambda w: w.name)
def test_mask_of_forward_selection(w):
    t = inputs_for(w)
    _, idx = msa.msa_forward(t["q"], t["k"], t["v"], t["q_idx"], t["k_idx"], topk=w.topk, return_idx=True)
    mask = msa.msa_block_mask(idx, seqlen_k=w.seqlen_k)
    back = msa.msa_mask_blocks(mask, seqlen_k=w.seqlen_k, topk=w.topk)
    torch.cuda.synchronize()
    sel = idx.cpu().numpy()
    assert np.array_equal(as_u32(mask), oracle.block_mask(sel, w.n_blk))
    assert torch.equal(back, idx)


@pytest.mark.parametrize("n_blk,topk", [(1, 1), (31, 4), (32, 16), (33, 16), (257, 16), (8192, 64)])
def test_mask_of_random_selections(n_blk, topk):
    rng = np.random.default_rng(n_blk + topk)
    B, H, S = 2, 3, min(257, n_blk * 128)  # dims keep seqlen_q <= seqlen_k
    sel = rng.integers(-3, n_blk + 40, size=(B, H, S, topk)).astype(np.int32)  # includes out-of-range entries
    dev = msa.msa_block_mask(torch.from_numpy(sel).cuda(), seqlen_k=n_blk * 128)
    torch.cuda.synchronize()
    assert np.array_equal(as_u32(dev), oracle.block_mask(sel, n_blk))


@pytest.mark.parametrize("n_blk,topk", [(1, 1), (31, 4), (33, 16), (100, 7), (257, 16), (8192, 64)])
def test_traversal_of_random_masks(n_blk, topk):
    rng = np.random.default_rng(7 * n_blk + topk)
    B, H, S = 2, 3, min(300, n_blk * 128)
    nw = oracle.mask_words(n_blk)
    density = rng.choice([0.0, 0.01, 0.1, 0.6], size=(B, H, S, 1))
    bits = rng.random((B, H, S, nw * 32)) < density  # stray bits past n_blk included
    words = np.packbits(bits.reshape(B, H, S, nw, 4, 8)[..., ::-1], axis=-1).reshape(B, H, S, nw, 4)
    words = (words[..., 3].astype(np.uint32) << 24) | (words[..., 2].astype(np.uint32) << 16) | \
            (words[..., 1].astype(np.uint32) << 8) | words[..., 0].astype(np.uint32)
    dev = msa.msa_mask_blocks(torch.from_numpy(words.view(np.int32)).cuda(), seqlen_k=n_blk * 128, topk=topk)
    torch.cuda.synchronize()
    clean = words.copy()
    if n_blk % 32:
        clean[..., nw - 1] &= np.uint32((1 << (n_blk % 32)) - 1)  # bits past the last block are ignored
    assert np.array_equal(dev.cpu().numpy(), oracle.mask_blocks(clean, topk))


def test_mask_round_trip_at_full_size():
    """The 32K workload: every row's selection survives mask and traversal,
    and every mask word matches the oracle's."""
    w = synth.WORKLOADS["prefill_32k"]
    t = inputs_for(w)
    _, idx = msa.msa_forward(t["q"], t["k"], t["v"], t["q_idx"], t["k_idx"], topk=w.topk, return_idx=True)
    del t
    mask = msa.msa_block_mask(idx, seqlen_k=w.seqlen_k)
    back = msa.msa_mask_blocks(mask, seqlen_k=w.seqlen_k, topk=w.topk)
    torch.cuda.synchronize()
    assert torch.equal(back, idx)
    assert np.array_equal(as_u32(mask), oracle.block_mask(idx.cpu().numpy(), w.n_blk))
