"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

Two programs are built with gcc/g++ -fsanitize=address,undefined
-fno-sanitize-recover=all and run; each must exit 0 with no sanitizer report:
  - tests/sanitize/oracle_driver.c with the CPU oracle (oracle/fp4q_ref.c):
    every entry point over every format, rule, objective, rotation, dtype
    and window, on empty, single-block and ragged shapes with 1 and 3
    threads;
  - tests/sanitize/capi_driver.cpp with the C ABI's host code
    (csrc/fp4q_capi.cpp) and stubbed kernel launchers: every entry point
    with valid arguments and with one defect at a time.
The same builds by hand: python tests/test_sanitize_host.py."""
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")


def build_oracle_driver(out):
    cmd = ["gcc", "-std=c11", "-ffp-contract=off", *SAN, "-pthread", "-I",
           os.path.join(ROOT, "oracle"), os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
           os.path.join(ROOT, "oracle", "fp4q_ref.c"), "-o", out, "-lm"]
    subprocess.run(cmd, check=True)


def build_capi_driver(out):
    csrc = os.path.join(ROOT, "block_scaled_fp4_fp4q_amd", "csrc")
    cmd = ["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), "-I", csrc,
           os.path.join(ROOT, "tests", "sanitize", "capi_driver.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "capi_stubs.cpp"),
           os.path.join(csrc, "fp4q_capi.cpp"), "-o", out]
    subprocess.run(cmd, check=True)


def run(exe):
    p = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=ENV)
    assert p.returncode == 0, p.stdout + p.stderr
    assert "runtime error" not in p.stderr and "AddressSanitizer" not in p.stderr, p.stderr
    return p.stdout


needs_gcc = pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None,
                               reason="gcc/g++ not available")


@needs_gcc
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    build_oracle_driver(exe)
    assert "ran clean" in run(exe)


@needs_gcc
@pytest.mark.skipif(not os.path.exists("/opt/rocm/include/hip/hip_runtime.h"),
                    reason="HIP headers not available")
def test_capi_host_code_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "capi_san")
    build_capi_driver(exe)
    assert "ran clean" in run(exe)


if __name__ == "__main__":
    with tempfile.TemporaryDirectory() as d:
        for build, name in ((build_oracle_driver, "oracle_san"), (build_capi_driver, "capi_san")):
            exe = os.path.join(d, name)
            build(exe)
            sys.stdout.write(run(exe))
