"""GPU test of msa_forward_noalloc (include/msa.h), through the C ABI: the
forward on the library's static scratch against msa_forward on a caller
workspace of the designed size, on two calls in a row, the second with a
smaller input.

msa_forward's results do not depend on the query chunking (each edge's
arithmetic is independent of its chunk), so the two entry points must agree
bit for bit even when the 256 MiB scratch forces many chunks (the 32K
workload: one chunk with the designed workspace, dozens in the scratch).
Both calls are also compared with the oracle (sampled rows of the first, all
rows of the second).  Outputs are poisoned before every call.
"""
import numpy as np
import pytest
import torch

import block_sparse_gqa_scores_amd as msa
import oracle
import synth
from gpu_util import compare, forward_outputs, host_inputs, inputs_for, run_device

pytestmark = pytest.mark.gpu


def noalloc(w, t):
    o = forward_outputs(w)
    msa.msa_forward_noalloc(t["q"], t["k"], t["v"], t["q_idx"], t["k_idx"], topk=w.topk, **o)
    torch.cuda.synchronize()
    return {"out": o["out"], "lse": o["lse"], "idx": o["block_idx"]}


def sampled(w, n=48, seed=5):
    rng = np.random.default_rng(seed)
    qs = np.unique(np.concatenate([rng.integers(0, w.seqlen_q, n), [0, 2047, 2048, w.seqlen_q - 1]]))
    return np.array([(b, q, g) for b in range(w.batch) for q in qs for g in range(w.heads_kv)], dtype=np.int64)


def test_noalloc_matches_forward_on_two_calls():
    big = synth.WORKLOADS["prefill_32k"]
    small = synth.Workload("noalloc_small", 2, 700, 1000, 8, 2, topk=5)
    d = msa.Dims.make(big.batch, big.seqlen_q, big.seqlen_k, big.heads_q, big.heads_kv, topk=big.topk)
    chunks = msa.msa_attn_chunks(d, msa.ENTRY_FORWARD, msa.NOALLOC_SCRATCH_BYTES)
    print(f"32K in the scratch: {chunks} query chunks", flush=True)
    assert chunks > 1
    for w, rows_of in ((big, sampled), (small, lambda w: oracle.Problem.of(w).all_rows())):
        print(f"[{w.name}] noalloc and forward", flush=True)
        t = inputs_for(w)
        got = noalloc(w, t)
        ref_dev = run_device(w, t, with_bm=False)
        for key in ("out", "lse", "idx"):
            assert torch.equal(got[key], ref_dev[key]), f"{w.name}: {key} differs from msa_forward"
        p = oracle.Problem.of(w)
        h = host_inputs(t)
        rows = rows_of(w)
        ref = oracle.forward(p, h["q"], h["k"], h["v"], h["q_idx"], h["k_idx"], rows=rows)
        msgs, stats = compare(w, got, ref, rows, check_bm=False, label=f"{w.name} noalloc")
        print(w.name, stats, flush=True)
        assert not msgs, "\n".join(msgs)
        del t


def test_noalloc_empty_problem_and_repeat():
    """An empty problem returns OK; a repeated call gives identical results
    (the scratch keeps the last call's contents, which nothing reads)."""
    d = msa.Dims.make(0, 0, 0, 8, 2)
    assert msa.lib().msa_forward_noalloc(d, None, None, None, None, None, None, None, None, None) == 0
    w = synth.Workload("noalloc_repeat", 1, 300, 1300, 16, 2, topk=6)
    t = inputs_for(w)
    a = noalloc(w, t)
    b = noalloc(w, t)
    for key in ("out", "lse", "idx"):
        assert torch.equal(a[key], b[key]), key
