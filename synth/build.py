"""Builds ``libmsa_synth.so`` (device fill kernels of the synthetic inputs)."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
from block_sparse_gqa_scores_amd.build import hipcc  # noqa: E402  (compiler lookup only)

LIB = os.path.join(HERE, "libmsa_synth.so")


def build(verbose: bool = False) -> str:
    cmd = [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-x", "hip", os.path.join(HERE, "synth_fill.hip"), "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        print(r.stdout)
        raise RuntimeError("hipcc failed for synth_fill.hip")
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
