"""Host side of the seeded input generator (no method arithmetic here)."""
import numpy as np
import torch

import synth


def test_splitmix64_known_answers():
    # First outputs of Vigna's splitmix64.c seeded with state 0: the state
    # advances by the golden gamma before mixing, as synth.splitmix64 does.
    gamma = 0x9E3779B97F4A7C15
    z = np.array([0, gamma], dtype=np.uint64)
    out = synth.splitmix64(z)
    assert int(out[0]) == 0xE220A8397B1DCDAF
    assert int(out[1]) == 0x6E789E6AA1B965F4


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.normal(size=100000).astype(np.float32) * 10 ** rng.uniform(-5, 5, 100000).astype(np.float32),
                        np.array([1.00390625, 1.01171875, -2.00390625, 0.0, -0.0], dtype=np.float32)])
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_distributions():
    e = np.arange(1 << 18, dtype=np.uint64)
    ints = synth.integer(0, 4, e)
    assert set(np.unique(ints)) == set(range(-3, 4))
    counts = np.bincount((ints + 3).astype(int))
    assert counts.min() > 0.97 * len(e) / 7 and counts.max() < 1.03 * len(e) / 7
    z = synth.normal(0, 1, e)
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1) < 0.01


def test_gain_keeps_index_values_exact_integers():
    w = synth.WORKLOADS["prefill_128k_gain"]
    e = np.arange(0, w.seqlen_k * w.index_dim, 997, dtype=np.uint64)
    v = synth.values_f64(w, "k_idx", e)
    assert np.all(v == np.rint(v)) and np.abs(v).max() <= 256
    b = synth.host_bits(w, "k_idx", e)
    np.testing.assert_array_equal(synth.bf16_bits_to_f32(b), v.astype(np.float32))


def test_workloads_shapes():
    w = synth.WORKLOADS["chunk_16k_of_1m"]
    assert w.seqlen_k - w.seqlen_q == 1032192 and w.n_blk == 8192
    d = synth.WORKLOADS["decode_64x256k"]
    assert d.batch == 64 and d.seqlen_q == 1 and d.n_blk == 2048 and d.group == 8
