"""Parity on seeded random shapes.  Forward: batch, sequence lengths (decode,
short and ragged prefill), G, D_idx, k and the key-gain workload drawn from a
fixed generator, each compared with the oracle on every row (block scores and
selections bit-exact, output and LSE within the tolerance rule), through the
fused and the separate index entry points alike.  Backward: small prefill
shapes and larger ones that split key blocks over workgroups, msa_backward's
five gradients against the oracle on every row and key."""
import numpy as np
import pytest

import synth
from gpu_util import backward_against_oracle, fused_backward, inputs_for, parity, prepare_backward

pytestmark = pytest.mark.gpu


def random_workloads(n, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    for c in range(n):
        hkv = int(rng.choice([1, 2, 4]))
        g = int(rng.choice([1, 2, 4, 8, 16, 32]))
        while g * hkv > 64:
            g //= 2
        didx = int(rng.choice([64, 128]))
        topk = int(rng.choice([1, 2, 3, 5, 8, 11, 16, 17, 24, 64]))
        sk = int(rng.integers(1, 3500))
        kind = rng.random()
        if kind < 0.25:
            sq = 1                                     # decode
        elif kind < 0.4:
            sq = int(rng.integers(2, min(33, sk + 1)))  # a few rows per sequence
        else:
            sq = int(rng.integers(1, sk + 1))
        b = int(rng.choice([1, 2, 3]))
        gain = bool(rng.random() < 0.2)
        name = f"rand{c}_b{b}_q{sq}_k{sk}_g{g}x{hkv}_d{didx}_k{topk}" + ("_gain" if gain else "")
        out.append(synth.Workload(name, b, sq, sk, g * hkv, hkv, index_dim=didx, topk=topk, gain=gain))
    return out


@pytest.mark.parametrize("w", random_workloads(24), ids=lambda w: w.name)
def test_random_shape_parity(w):
    msgs, stats = parity(w)
    print(w.name, stats, flush=True)
    assert not msgs, "\n".join(msgs)


def random_backward_workloads(n, seed=7):
    """Prefill shapes small enough for the oracle's gradients on every row and
    key (the decode shape has its own cases in the backward tests)."""
    rng = np.random.default_rng(seed)
    out = []
    for c in range(n):
        hkv = int(rng.choice([1, 2, 4]))
        g = int(rng.choice([1, 2, 4, 8, 16]))
        while g * hkv > 32:
            g //= 2
        didx = int(rng.choice([64, 128]))
        topk = int(rng.choice([1, 3, 6, 16, 20]))
        sk = int(rng.integers(200, 1600))
        sq = int(rng.integers(2, sk + 1))
        b = int(rng.choice([1, 2]))
        gain = bool(rng.random() < 0.25)
        name = f"rbwd{c}_b{b}_q{sq}_k{sk}_g{g}x{hkv}_d{didx}_k{topk}" + ("_gain" if gain else "")
        out.append(synth.Workload(name, b, sq, sk, g * hkv, hkv, index_dim=didx, topk=topk, gain=gain))
    return out


@pytest.mark.parametrize("w", random_backward_workloads(10), ids=lambda w: w.name)
def test_random_shape_backward_parity(w):
    """msa_backward (main-branch and alignment-loss gradients in one pass)
    against the oracle on every row and key."""
    t = inputs_for(w)
    out, lse, idx, lse_idx = prepare_backward(w, t)
    grads = fused_backward(w, t, out, lse, idx, lse_idx)
    backward_against_oracle(w, t, grads, idx, w.name)


def big_backward_workloads(n, seed=11):
    """Larger prefill shapes (G >= 8, S_q G > 16384, mostly with the per-block
    gain) whose main backward builds a segmented work list, and most of them
    split a key block that nearly every query selects over several
    workgroups; the large buckets take the counting sort."""
    rng = np.random.default_rng(seed)
    out = []
    for c in range(n):
        g = int(rng.choice([8, 16, 32]))
        hkv = int(rng.choice([1, 2])) if g <= 16 else 1
        sq = int(rng.integers(max(1100, 17000 // g + 1), 2601))
        sk = int(rng.integers(sq, 3001))
        topk = int(rng.choice([2, 3, 6]))
        didx = int(rng.choice([64, 128]))
        b = int(rng.choice([1, 2])) if g * hkv * sq <= 40000 else 1
        gain = bool(rng.random() < 0.75)
        name = f"bbwd{c}_b{b}_q{sq}_k{sk}_g{g}x{hkv}_d{didx}_k{topk}" + ("_gain" if gain else "")
        out.append(synth.Workload(name, b, sq, sk, g * hkv, hkv, index_dim=didx, topk=topk, gain=gain))
    return out


@pytest.mark.parametrize("w", big_backward_workloads(6), ids=lambda w: w.name)
def test_big_shape_backward_parity(w):
    """msa_backward on the larger shapes against the oracle on every row and
    key."""
    t = inputs_for(w)
    out, lse, idx, lse_idx = prepare_backward(w, t)
    grads = fused_backward(w, t, out, lse, idx, lse_idx)
    backward_against_oracle(w, t, grads, idx, w.name)
