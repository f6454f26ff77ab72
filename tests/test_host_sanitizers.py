"""Sanitizer builds of the host code, run on the CPU (no GPU):

  - the C ABI's host half (include/msa.h entry points in msa_api.cpp and the
    workspace / chunk planning in plan.cpp), built with g++ under
    AddressSanitizer + UndefinedBehaviorSanitizer against launch stubs
    (tests/sanitize/launch_stubs.cpp) and driven by
    tests/sanitize/abi_check.cpp: every argument check, the planning over a
    sweep of shapes up to the 1M-token prefix, and valid calls that reach
    the (stubbed) launchers;
  - the CPU oracle (oracle/msa_oracle.cpp) under ASan + UBSan and, since it
    runs rows on several threads, under ThreadSanitizer, driven by
    tests/sanitize/oracle_check.cpp on small ragged problems.

Each build stops at the first sanitizer report (-fno-sanitize-recover) and
the drivers exit non-zero on a failed expectation.  The device code is not
part of these builds; it is compiled for gfx950 by the package build.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_gqa_scores_amd", "csrc")
SAN = os.path.join(ROOT, "tests", "sanitize")
ROCM_INCLUDE = "/opt/rocm/include"

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")

ASAN_UBSAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def build_and_run(tmp_path, name, flags, sources, includes=(), defines=(), env=None):
    exe = str(tmp_path / name)
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-pthread", *flags, *[f"-D{d}" for d in defines],
           *[f"-I{i}" for i in includes], *sources, "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert b.returncode == 0, b.stderr[-4000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env={**os.environ, **(env or {})})
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "Sanitizer" not in out, out[-4000:]
    return out


@pytest.mark.skipif(not os.path.isdir(ROCM_INCLUDE), reason="needs the HIP headers")
def test_abi_host_code_under_asan_ubsan(tmp_path):
    out = build_and_run(
        tmp_path, "abi_check", ASAN_UBSAN,
        [os.path.join(CSRC, "msa_api.cpp"), os.path.join(CSRC, "plan.cpp"),
         os.path.join(SAN, "launch_stubs.cpp"), os.path.join(SAN, "abi_check.cpp")],
        includes=[ROCM_INCLUDE, os.path.join(ROOT, "include"), CSRC], defines=["__HIP_PLATFORM_AMD__"],
        env={"ASAN_OPTIONS": "detect_leaks=1"})
    assert "abi host check ok" in out


def test_oracle_under_asan_ubsan(tmp_path):
    out = build_and_run(tmp_path, "oracle_check", ASAN_UBSAN,
                        [os.path.join(ROOT, "oracle", "msa_oracle.cpp"), os.path.join(SAN, "oracle_check.cpp")],
                        env={"ASAN_OPTIONS": "detect_leaks=1"})
    assert "oracle host check ok" in out


def test_oracle_under_tsan(tmp_path):
    out = build_and_run(tmp_path, "oracle_check_tsan", ["-fsanitize=thread"],
                        [os.path.join(ROOT, "oracle", "msa_oracle.cpp"), os.path.join(SAN, "oracle_check.cpp")])
    assert "oracle host check ok" in out
