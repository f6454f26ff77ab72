"""Host checks of bench.py: its algorithmic work counts against closed forms of
the definitions they follow, and its refusal of more than one GPU.

The closed forms restate the counting rules independently of bench.py's
vectorised sums: a causal query at position t scores t + 1 index keys (the
index branch sees every earlier token, Sparse Attention Part II, section
3.2), and attends to every visible token while its local block index is below
k, else to k - 1 full blocks plus the visible part of its own block (the
reserved local block of the same section).  The printed totals are the ones
derived for these workloads from the same definitions (1.0995e12 index FLOP
and 2.0664e12 attention FLOP on the 32K prefill; 4 834 099 200 bytes per
decode step).
"""
import os
import subprocess
import sys

import pytest

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def index_closed(w):
    """2 D_idx H_kv B sum_{t = t0}^{t0 + S_q - 1} (t + 1), t0 = S_k - S_q."""
    t0 = w.seqlen_k - w.seqlen_q
    s = (t0 + w.seqlen_q) * (t0 + w.seqlen_q + 1) // 2 - t0 * (t0 + 1) // 2
    return 2 * w.index_dim * w.heads_kv * w.batch * s


def attn_closed(w):
    """4 D H_q B sum_i |T_i|, summed block by block: positions t = 128 j + r."""
    bs, k = w.block_size, w.topk
    total = 0
    t0, t1 = w.seqlen_k - w.seqlen_q, w.seqlen_k  # positions [t0, t1)
    for j in range(t0 // bs, (t1 - 1) // bs + 1):
        lo, hi = max(t0, j * bs), min(t1, (j + 1) * bs)  # positions of block j in range
        n = hi - lo
        rsum = (lo - j * bs + hi - 1 - j * bs) * n // 2  # sum of t mod bs over them
        if j < k:  # every token up to t is visible: sum of (t + 1)
            total += (lo + hi - 1) * n // 2 + n
        else:      # (k - 1) full blocks + (t mod bs) + 1
            total += n * ((k - 1) * bs + 1) + rsum
    return 4 * w.head_dim * w.heads_q * w.batch * total


@pytest.mark.parametrize("name", ["prefill_4k", "prefill_32k", "prefill_128k_gain", "chunk_16k_of_1m",
                                  "decode_64x256k"])
def test_work_counts_match_closed_forms(name):
    w = synth.WORKLOADS[name]
    assert bench.index_flops(w) == pytest.approx(index_closed(w), rel=1e-12)
    assert bench.attn_flops(w) == pytest.approx(attn_closed(w), rel=1e-12)


def test_printed_totals():
    w = synth.WORKLOADS["prefill_32k"]
    assert bench.index_flops(w) == pytest.approx(1.0995e12, rel=1e-4)
    assert bench.attn_flops(w) == pytest.approx(2.0664e12, rel=1e-4)
    assert bench.attn_flops(synth.WORKLOADS["prefill_4k"]) == pytest.approx(2.524e10, rel=1e-3)
    assert bench.index_flops(synth.WORKLOADS["chunk_16k_of_1m"]) == pytest.approx(3.4910e13, rel=1e-4)
    assert bench.attn_flops(synth.WORKLOADS["chunk_16k_of_1m"]) == pytest.approx(1.0654e12, rel=1e-4)
    assert bench.decode_bytes(synth.WORKLOADS["decode_64x256k"]) == 4834099200


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_multi_chunk_stage_accounting():
    """With the attention in 3 query chunks, each stage is rated over its own
    time: the one-launch index scan over that launch, the per-chunk stages
    over the sum of their launches; no rate exceeds its peak for plausible
    times, and the roofline's per-launch work times launches is the step's."""
    w = synth.WORKLOADS["prefill_128k_gain"]
    stage_ms = {"index_scores": 11.8, "block_topk": 0.004, "attn_build": 0.3, "attn_partial": 12.0,
                "attn_merge": 6.5}
    chunks = 3
    st = bench.stage_rates(w, stage_ms, chunks)
    assert st["index_scores"]["launches_per_step"] == 1 and st["attn_partial"]["launches_per_step"] == 3
    assert st["index_scores"]["TFLOP/s"] == pytest.approx(bench.index_flops(w) / 11.8e-3 / 1e12)
    assert st["attn_partial"]["TFLOP/s"] == pytest.approx(bench.attn_flops(w) / 12.0e-3 / 1e12)
    for name, x in st.items():
        if "frac" in x:
            assert 0 < x["frac"] < 1, name
    att = bench.attention_step(w, stage_ms, chunks)
    assert att["ms_per_step"] == pytest.approx(0.3 + 12.0 + 6.5)
    assert att["TFLOP/s"] == pytest.approx(bench.attn_flops(w) / 18.8e-3 / 1e12)
    r = bench.roofline(w, stage_ms, chunks)
    assert r["kernel"].startswith("attn_partial_kernel") and r["launches_per_step"] == 3
    assert r["avg_launch_ms"] == pytest.approx(4.0)
    assert r["work_per_launch"] * 3 == pytest.approx(bench.attn_flops(w))
    assert r["frac"] < 1
    # the fused selection has no Top-k stage of its own
    assert st["block_topk"]["bound"] == "fused" and "frac" not in st["block_topk"]


def test_decode_stages_are_rated_in_bytes():
    w = synth.WORKLOADS["decode_64x256k"]
    st = bench.stage_rates(w, {"index_scores": 0.64, "block_topk": 0.005, "attn_build": 0.0,
                               "attn_partial": 0.11, "attn_merge": 0.01}, 1)
    assert st["index_scores"]["bound"] == "hbm" and st["attn_partial"]["bound"] == "hbm"
    assert 0 < st["index_scores"]["frac"] < 1 and 0 < st["attn_partial"]["frac"] < 1


def test_partial_traffic_needs_the_measured_chunk_count():
    """A committed traffic figure of the partial kernel is bytes per launch at
    the chunk count it was measured with; another count (a launch covering
    another share of the edges) reports none."""
    w = synth.WORKLOADS["prefill_32k"]
    measured = bench.measured_traffic(w, "attn_partial", 1)
    if measured is None:
        pytest.skip("the committed summary does not match the current kernel sources")
    assert measured > 0
    assert bench.measured_traffic(w, "attn_partial", 2) is None
