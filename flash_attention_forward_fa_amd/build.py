"""Builds libfa.so, the C-ABI library of the gfx950 forward and backward kernels, with hipcc.

Flags:
  --offload-arch=gfx950           MI355X only (CDNA4)
  -fno-honor-nans                 NaN inputs are outside the contract; lets
                                  fmax compile to a bare v_max (no canonicalise).
                                  Infinities are still honoured (-inf masks).
  -target-feature -packed-fp32-ops  no packed f32 VALU instructions
"""
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libfa.so")
# (the forward's key widths 80, 96 and 192 have translation units of their own,
# which compile in parallel with the rest)
SOURCES = [os.path.join(HERE, "csrc", f) for f in
           ("fa_fwd.hip", "fa_fwd_d80.hip", "fa_fwd_d96.hip", "fa_fwd_d192.hip", "fa_bwd.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-fno-honor-nans", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include")]


def build(verbose=False, extra_flags=()):
    """Compiles every source to an object (in parallel), then links libfa.so."""
    tmp = tempfile.mkdtemp(prefix="fa_build_")
    try:
        compile_flags = [f for f in FLAGS if f != "-shared"]
        objs, procs = [], []
        for src in SOURCES:
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            cmd = [HIPCC, *compile_flags, *extra_flags, "-c", "-o", obj, src]
            if verbose:
                print(" ".join(cmd), flush=True)
            objs.append(obj)
            procs.append((cmd, subprocess.Popen(cmd)))
        failed = [cmd for cmd, p in procs if p.wait() != 0]
        if failed:
            raise subprocess.CalledProcessError(1, failed[0])
        cmd = [HIPCC, "--offload-arch=gfx950", "-fPIC", "-shared", "-o", LIB + ".tmp", *objs]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(LIB + ".tmp", LIB)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True, extra_flags=sys.argv[1:]))
