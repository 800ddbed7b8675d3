"""Builds libfa.so, the C-ABI library of the gfx950 forward and backward kernels, with hipcc.

Flags:
  --offload-arch=gfx950           MI355X only (CDNA4)
  -fno-honor-nans                 NaN inputs are outside the contract; lets
                                  fmax compile to a bare v_max (no canonicalise).
                                  Infinities are still honoured (-inf masks).
  -target-feature -packed-fp32-ops  no packed f32 VALU instructions
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libfa.so")
SOURCES = [os.path.join(HERE, "csrc", "fa_fwd.hip"), os.path.join(HERE, "csrc", "fa_bwd.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-fno-honor-nans", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include")]


def build(verbose=False, extra_flags=()):
    cmd = [HIPCC, *FLAGS, *extra_flags, "-o", LIB + ".tmp", *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True, extra_flags=sys.argv[1:]))
