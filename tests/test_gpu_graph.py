"""HIP graph capture of the forward, through the C ABI.  The library
allocates nothing during a call, synchronises nothing, and clears the
counters it reads back with its own kernels (no hipMemsetAsync), so a call
can be recorded into a graph: msa_forward on a caller workspace and
msa_forward_noalloc on the library's static scratch are captured with
torch.cuda.graph, and every replay must equal the eager call bit for bit.
Between replays the outputs are poisoned and other library calls run
eagerly on other inputs (overwriting the workspace and the static scratch),
so a replay that relied on leftover contents would fail."""
import pytest
import torch

import block_sparse_gqa_scores_amd as msa
import synth
from gpu_util import inputs_for

pytestmark = pytest.mark.gpu

W = synth.Workload("graph_fwd", 2, 1500, 2600, 16, 2, topk=8)
OTHER = synth.Workload("graph_other", 1, 900, 1900, 16, 2, topk=5)  # eager work between replays


def outputs(w, t):
    return (torch.empty_like(t["q"]),
            torch.empty((w.batch, w.heads_q, w.seqlen_q), dtype=torch.float32, device="cuda"),
            torch.empty((w.batch, w.heads_kv, w.seqlen_q, w.topk), dtype=torch.int32, device="cuda"))


def poison(bufs):
    out, lse, idx = bufs
    out.view(torch.int16).fill_(-1)  # bf16 NaN pattern
    lse.fill_(float("nan"))
    idx.fill_(-7)


@pytest.mark.parametrize("entry", ["noalloc", "workspace"])
def test_forward_graph_replays_equal_eager(entry):
    t, t2 = inputs_for(W), inputs_for(OTHER)
    d, d2 = (msa.dims_of(x["q"], x["k"], x["q_idx"], x["k_idx"], topk=w.topk) for x, w in ((t, W), (t2, OTHER)))
    ws = torch.empty(max(msa.msa_workspace_bytes(d, msa.ENTRY_FORWARD), msa.msa_workspace_bytes(d2, msa.ENTRY_FORWARD)),
                     dtype=torch.uint8, device="cuda")

    def call(w, x, bufs):
        out, lse, idx = bufs
        if entry == "noalloc":
            msa.msa_forward_noalloc(x["q"], x["k"], x["v"], x["q_idx"], x["k_idx"], topk=w.topk,
                                    out=out, lse=lse, block_idx=idx)
        else:
            msa.msa_forward(x["q"], x["k"], x["v"], x["q_idx"], x["k_idx"], topk=w.topk,
                            out=out, lse=lse, block_idx=idx, workspace=ws)

    eager = outputs(W, t)
    call(W, t, eager)
    other = outputs(OTHER, t2)
    call(OTHER, t2, other)
    torch.cuda.synchronize()

    replayed = outputs(W, t)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(W, t, replayed)
    torch.cuda.synchronize()

    names = ("out", "lse", "block_idx")
    for rep in range(3):
        poison(replayed)
        call(OTHER, t2, other)  # eager: rewrites the workspace / scratch with another problem
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(names, replayed, eager):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)), \
                f"{entry}: replay {rep} {name} differs from the eager call"
