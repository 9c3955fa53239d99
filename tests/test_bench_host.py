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


def test_hbm_roofline_arithmetic():
    # the KV workload: 2^30 elements, 2.5625 algorithmic bytes each per launch
    n, ms = 1 << 30, 1.0
    r = bench.roofline(n, ms, ISSUE)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert r["algorithmic_bytes_per_launch"] == pytest.approx(n * 2.5625)
    assert r["achieved"] == pytest.approx(n * 2.5625 / 1e-3 / 1e9)
    assert r["peak"] == 8000.0
    assert r["frac"] == pytest.approx(r["achieved"] / 8000.0)


def test_valu_figures_beside_the_roofline():
    n, ms = 1 << 20, 0.5
    v = bench.roofline(n, ms, ISSUE)["valu"]
    # 35 binary32 ops + 5.5 encodes at 4 FMAs each + 5.5 decodes at 3 FMAs each
    assert v["algorithmic_lane_ops_per_elem"] == pytest.approx(35 + 5.5 * 4 + 5.5 * 3)
    assert v["achieved"] == pytest.approx(n * 73.5 / (ms * 1e-3) / 1e12)
    assert v["peak"] == pytest.approx(157.3 / 2)
    assert v["frac"] == pytest.approx(v["achieved"] / v["peak"])
    # without the microbenchmark the HBM roofline stands alone
    r = bench.roofline(n, ms, None)
    assert r["bound"] == "hbm" and "achieved" not in r["valu"]


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one MI355X" in p.stderr
    assert p.stdout.strip() == ""  # no bench line
