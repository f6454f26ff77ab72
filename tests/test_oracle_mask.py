"""Pins of the oracle's block-mask format (Sparse Attention Part II, section
4.3) to the section's worked example, its storage formula and the plain
definition of a bit set."""
import numpy as np
import pytest

import oracle


def test_worked_example_word_is_73():
    """Blocks 0, 3 and 6 of the first query block survive: the low eight bits
    read 01001001, which is 73; the traversal visits 0, 3, 6."""
    m = oracle.block_mask(np.array([[0, 3, 6, -1]]), n_blk=8)
    assert m.shape == (1, 1) and int(m[0, 0]) == 0b01001001 == 73
    assert oracle.popcount(73) == 3
    assert [oracle.nth_set_bit(73, r) for r in range(3)] == [0, 3, 6]
    assert oracle.mask_blocks_by_scan(m[0], 8, 4) == [0, 3, 6, -1]
    assert oracle.mask_blocks(m, 4).tolist() == [[0, 3, 6, -1]]


@pytest.mark.parametrize("t_r,t_c", [(1, 8), (3, 32), (5, 33), (2, 64), (7, 100), (4, 8192)])
def test_storage_is_4_tr_ceil_tc_over_32_bytes(t_r, t_c):
    m = oracle.block_mask(np.full((t_r, 1), -1), n_blk=t_c)
    assert m.dtype == np.uint32 and m.nbytes == 4 * t_r * int(np.ceil(t_c / 32))


def test_word_and_bit_of_each_block():
    """Block j lives in word floor(j / 32) at bit j mod 32, and nowhere else."""
    n_blk = 100
    for j in range(n_blk):
        m = oracle.block_mask(np.array([[j]]), n_blk)[0]
        expect = np.zeros(4, dtype=np.uint32)
        expect[j // 32] = np.uint32(1) << np.uint32(j % 32)
        assert np.array_equal(m, expect), j


def test_unused_bits_stay_zero_and_out_of_range_entries_are_ignored():
    n_blk = 37  # second word uses bits 0..4 only
    m = oracle.block_mask(np.array([[36, 37, 63, -1, 5]]), n_blk)[0]
    assert int(m[1]) == 1 << 4 and int(m[0]) == 1 << 5


def test_traversal_equals_definition_on_random_masks():
    """The vectorised traversal equals a scan of every block position against
    its word and bit, and both equal the sorted list of set positions."""
    rng = np.random.default_rng(3)
    for n_blk in (1, 31, 32, 33, 95, 256):
        nw = oracle.mask_words(n_blk)
        for density in (0.02, 0.3, 0.9):
            bitsv = rng.random((20, nw * 32)) < density
            bitsv[:, n_blk:] = False
            words = np.zeros((20, nw), dtype=np.uint32)
            for r in range(20):
                for j in np.nonzero(bitsv[r])[0]:
                    words[r, j // 32] |= np.uint32(1) << np.uint32(j % 32)
            for cap in (1, 5, 16, 64):
                got = oracle.mask_blocks(words, cap)
                for r in range(20):
                    pos = np.nonzero(bitsv[r])[0][:cap].tolist()
                    want = pos + [-1] * (cap - len(pos))
                    assert got[r].tolist() == want
                    assert oracle.mask_blocks_by_scan(words[r], n_blk, cap) == want


def test_round_trip_of_selections():
    """A selection (ascending, distinct, -1 padded) survives mask and traversal."""
    rng = np.random.default_rng(4)
    n_blk, k = 300, 16
    sel = np.full((50, k), -1, dtype=np.int32)
    for r in range(50):
        n = rng.integers(1, k + 1)
        sel[r, :n] = np.sort(rng.choice(n_blk, size=n, replace=False))
    m = oracle.block_mask(sel, n_blk)
    assert np.array_equal(oracle.mask_blocks(m, k), sel)
    assert [sum(oracle.popcount(w) for w in row) for row in m] == (sel >= 0).sum(1).tolist()
