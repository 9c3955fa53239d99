"""Build the VALU issue-cost microbenchmark (valu_issue.hip) next to its
source.  bench.py runs it as a child process to report the issue cost of the
instructions the ScaleSweep estimate is built from, beside its HBM roofline.
It is a measurement tool: the library does not use it."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "valu_issue.hip")
EXE = os.path.join(HERE, "valu_issue")
ARCH = os.environ.get("FP4Q_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose=False):
    tmp = EXE + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-Wall",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, EXE)
    return EXE


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
