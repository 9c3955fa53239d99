"""A plain C program (tests/capi_example.c) drives the C ABI with its own HIP
allocations and compares the results with the C oracle byte for byte."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu
EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "capi_example")


def test_c_consumer_matches_oracle():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(EXE):
        pytest.fail("tests/capi_example is not built: run __graft_entry__.build()")
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "matches the oracle" in r.stdout
    assert "invalid shape" in r.stdout
