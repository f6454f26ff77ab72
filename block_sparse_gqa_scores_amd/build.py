"""Builds ``libmsa.so`` (the gfx950 HIP library) in-tree with hipcc.

Every call recompiles from source.  Objects go to ``_build/`` at the repo root.
"""
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmsa.so")
BUILD_DIR = os.path.join(ROOT, "_build", "msa")

SOURCES = ["index_scan.hip", "block_topk.hip", "sparse_attn.hip", "kl_loss.hip", "attn_bwd.hip", "kl_bwd.hip",
           "block_mask.hip", "noalloc.hip", "plan.cpp", "msa_api.cpp"]
ARCH = "gfx950"
# Packed fp32 vector ops are kept out of the generated code on purpose.
HIP_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I" + INCLUDE, "-I" + CSRC]


def hipcc() -> str:
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, extra_flags=()) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    procs, objs = [], []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [cc, *HIP_FLAGS, *extra_flags, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        objs.append(obj)
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        lines = [l for l in out.splitlines() if "packed-fp32-ops" not in l]
        if p.returncode != 0:
            failed.append(src)
            print("\n".join(lines), flush=True)
        elif verbose and lines:
            print("\n".join(lines), flush=True)
    if failed:
        raise RuntimeError("hipcc failed for " + ", ".join(failed))
    cmd = [cc, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
