"""Compile the C oracle into oracle/libfp4q_ref.so (test infrastructure only)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "fp4q_ref.c")
LIB = os.path.join(HERE, "libfp4q_ref.so")

# -ffp-contract=off: no fused multiply-add may merge two of the oracle's
# roundings; no -ffast-math: IEEE binary32/binary64 semantics throughout.
CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
          "-shared", "-pthread", "-Wall", "-Wextra"]


def build(verbose=False):
    cmd = ["gcc", *CFLAGS, "-o", LIB, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
