"""Host logic of bench.py: the roofline arithmetic and the one-GPU guard
(no GPU needed)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

ISSUE = {"device": "gfx950", "simds": 1024,
         "cycles_per_wave64_instr": {"v_fma_f32": 2.0, "v_mul_f32": 2.0,
                                     "v_cvt_scalef32_pk_fp4_f32": 8.0,
                                     "v_cvt_scalef32_pk_f32_fp4": 6.0,
                                     "v_xor_b32": 1.5, "v_fma_f64": 4.0}}


def test_alu_roofline_arithmetic():
    n, ms = 1 << 20, 0.5
    r = bench.roofline(n, ms, 1000.0, 2.5625, ISSUE)
    assert r["bound"] == "alu"
    # 48 binary32 ops + 8 encodes at 4 FMAs each + 8 decodes at 3 FMAs each
    assert r["algorithmic_lane_ops_per_elem"] == pytest.approx(48 + 8 * 4 + 8 * 3)
    assert r["achieved"] == pytest.approx(n * 104 / (ms * 1e-3) / 1e12)
    assert r["peak"] == pytest.approx(157.3 / 2)
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"])
    assert r["hbm"]["frac"] == pytest.approx(1000.0 / 8000.0)
    assert r["hbm"]["algorithmic_bytes_per_launch"] == pytest.approx(n * 2.5625)


def test_hbm_roofline_without_issue_costs():
    r = bench.roofline(1 << 20, 0.5, 2000.0, 2.5625, None)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert r["frac"] == pytest.approx(0.25)


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one MI355X" in p.stderr
    assert p.stdout.strip() == ""  # no bench line
