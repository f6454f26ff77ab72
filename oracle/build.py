"""Builds the CPU oracle (``liboracle.so``) with the host C++ compiler.

The oracle is test infrastructure; building it is part of building the
project, using it is reserved to the tests, the smoke check and the
benchmark's CPU-baseline leg.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "msa_oracle.cpp")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["g++", "-std=c++17", "-O2", "-fPIC", "-shared", "-pthread", SRC, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
