"""Build tests/capi_example (plain C, gcc) against libfp4q.so, the C oracle
and the HIP runtime.  Run by __graft_entry__.build() after both libraries;
the binary finds them through an $ORIGIN-relative rpath."""
import os
import subprocess
import sys

TESTS = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(TESTS)
EXE = os.path.join(TESTS, "capi_example")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose=False):
    pkg = os.path.join(ROOT, "block_scaled_fp4_fp4q_amd")
    orc = os.path.join(ROOT, "oracle")
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), "-I", orc,
           os.path.join(TESTS, "capi_example.c"), "-o", EXE,
           "-L", pkg, "-l:libfp4q.so", "-L", orc, "-l:libfp4q_ref.so",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../block_scaled_fp4_fp4q_amd:$ORIGIN/../oracle:" + os.path.join(ROCM, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return EXE


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
