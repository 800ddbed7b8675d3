"""Builds liboracle.so (the plain CPU reference) with the host C compiler.

No fast-math and no floating-point contraction: the reference must perform
exactly the IEEE single-precision operations its source spells out.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose=False):
    src = os.path.join(HERE, "fa_oracle.c")
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-fno-tree-vectorize", "-pthread",
           "-o", LIB + ".tmp", src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
