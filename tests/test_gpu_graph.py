"""HIP graph capture of the forward and the backward, through the C ABI.  The library
allocates nothing during a call, synchronises nothing, and clears the
counters it reads back with its own kernels (no hipMemsetAsync), so a call
can be recorded into a graph: msa_forward on a caller workspace and
msa_forward_noalloc on the library's static scratch, and msa_backward, are
captured with torch.cuda.graph, and every replay must equal the eager call
bit for bit.
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


def test_backward_graph_replays_equal_eager():
    """msa_backward (both gradients, with a segmented work list: G = 8 and
    2600 queries) captured and replayed against the eager call."""
    from gpu_util import prepare_backward
    w = synth.Workload("graph_bwd", 1, 2600, 2600, 64, 8, topk=8, gain=True)
    t = inputs_for(w)
    out, lse, idx, lse_idx = prepare_backward(w, t)
    d = msa.dims_of(t["q"], t["k"], t["q_idx"], t["k_idx"], topk=w.topk)
    ws = torch.empty(msa.msa_workspace_bytes(d, msa.ENTRY_BACKWARD), dtype=torch.uint8, device="cuda")

    def grads():
        return (torch.empty_like(t["q"]), torch.empty_like(t["k"]), torch.empty_like(t["v"]),
                torch.empty_like(t["q_idx"]), torch.empty_like(t["k_idx"]))

    def call(g, dout, grad_loss):
        msa.msa_backward(t["q"], t["k"], t["v"], t["q_idx"], t["k_idx"], idx, out, lse, lse_idx, dout, grad_loss,
                         dq=g[0], dk=g[1], dv=g[2], dq_idx=g[3], dk_idx=g[4], workspace=ws)

    dout = t["dout"]
    other_dout = -0.5 * dout
    eager = grads()
    call(eager, dout, 0.75)
    other = grads()
    call(other, other_dout, 2.0)
    torch.cuda.synchronize()
    replayed = grads()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(replayed, dout, 0.75)
    torch.cuda.synchronize()
    for rep in range(3):
        for x in replayed:
            x.view(torch.int16).fill_(-1)
        call(other, other_dout, 2.0)
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv", "dq_idx", "dk_idx"), replayed, eager):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"replay {rep} {name} differs"
