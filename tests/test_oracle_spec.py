"""The C oracle against the independent exact statement of the method
(tests/exactspec.py) on tiny random and adversarial tensors (CPU only)."""
from fractions import Fraction as Fr

import numpy as np
import pytest

import exactspec as X
from block_scaled_fp4_fp4q_amd import synth

f32 = np.float32


def adversarial_nvfp4():
    """Blocks that sit on the edges of the method, under S = 1 (the first
    block holds the tensor maximum 1536)."""
    rows = []
    big = np.zeros(16, np.float32)
    big[3] = 1536.0
    rows.append(big)
    rows.append(np.zeros(16, np.float32))                              # all zero
    z = np.zeros(16, np.float32)
    z[::2] = -0.0
    rows.append(z)                                                     # signed zeros
    s = np.zeros(16, np.float32)
    s[7] = -3.25
    rows.append(s)                                                     # one spike
    g = np.array([0, .5, 1, 1.5, 2, 3, 4, 6] * 2, np.float32) * f32(0.8125)
    g[1::3] *= -1
    rows.append(g)                                                     # on the grid
    rows.append(np.full(16, 4.0, np.float32))                          # sweep finds 1.0
    t = np.linspace(0.01, 1, 16).astype(np.float32)
    t[0] = 6 * 1.0625                                                  # E4M3 tie in s_base
    rows.append(t)
    rows.append((np.arange(16, dtype=np.float32) - 8) * f32(1e-4))     # subnormal E4M3 scale
    rows.append(np.full(16, 1e-6, np.float32))                         # s_base clamps to 0x01
    m = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5, 6] * 2, np.float32)
    rows.append(m)                                                     # E2M1 midpoints
    rows.append(np.array([6, 5.999, -5, 4.5, 0.25, 0.24, 7, -7] * 2, np.float32))
    rows.append(np.array([1, -1] * 8, np.float32) * f32(2.0 ** -120))  # below every code
    return np.stack(rows)


def tiny_tensors():
    rng = np.random.default_rng(11)
    yield "c1", synth.c1(rows=4, cols=64, seed=5)
    yield "c2", synth.bf16_bits_to_f32(synth.c2(rows=3, cols=64, seed=6)[0])
    yield "c4", synth.bf16_bits_to_f32(synth.c4(rows=4, cols=64, seed=7)[0])
    yield "heavy", (rng.standard_t(2, (3, 64)) * 1e-3).astype(np.float32)
    yield "adv", adversarial_nvfp4().reshape(-1, 32)


def blocks_of(x, B):
    return np.ascontiguousarray(x, np.float32).reshape(-1, B)


@pytest.mark.parametrize("rotate", [0, 16])
@pytest.mark.parametrize("mode", ["absmax", "mse", "wmse"])
def test_nvfp4_matches_exact_spec(ref, mode, rotate):
    rng = np.random.default_rng(2)
    for name, x in tiny_tensors():
        rows, cols = x.shape
        imp = rng.lognormal(0, 1, cols).astype(np.float32)
        if mode == "absmax":
            out = ref.quantize(x, rotate=rotate, errors=True)
            sweep, w = None, None
        elif mode == "mse":
            out = ref.quantize(x, rule=ref.SWEEP, objective=ref.MSE, rotate=rotate, errors=True)
            sweep, w = (-3, 7), None
        else:
            out = ref.quantize(x, rule=ref.SWEEP, objective=ref.WMSE, importance=imp,
                               rotate=rotate, errors=True)
            sweep, w = (-8, 7), imp
        xp = ref.prepare(x, rotate=rotate)
        S = X.global_scale(np.abs(xp).max())
        assert out["S"] == S, name
        nib = ref.unpack_nibbles(out["codes"])
        for b, xb in enumerate(blocks_of(xp, 16)):
            wb = None if w is None else w[(b * 16) % cols:(b * 16) % cols + 16]
            sc, nb, e, errs = X.quantize_block_nvfp4(xb, S, sweep, wb)
            assert out["scales"][b] == sc, (name, b)
            assert list(nib[b * 16:(b + 1) * 16]) == nb, (name, b)
            if e == 0:
                assert out["best"][b] == 0
            else:
                assert abs(Fr(out["best"][b]) - e) <= e * Fr(1, 10 ** 12), (name, b)


@pytest.mark.parametrize("rotate", [0, 16])
def test_if4_matches_exact_spec(ref, rotate):
    for name, x in tiny_tensors():
        out = ref.quantize(x, fmt=ref.IF4, rotate=rotate, errors=True)
        xp = ref.prepare(x, rotate=rotate)
        S = X.global_scale(np.abs(xp).max())
        assert out["S"] == S
        nib = ref.unpack_nibbles(out["codes"])
        for b, xb in enumerate(blocks_of(xp, 16)):
            sc, nb, e = X.quantize_block_if4(xb, S)
            assert out["scales"][b] == sc, (name, b)
            assert list(nib[b * 16:(b + 1) * 16]) == nb, (name, b)
            assert abs(Fr(out["best"][b]) - e) <= e * Fr(1, 10 ** 12)


@pytest.mark.parametrize("rotate", [0, 32])
def test_mxfp4_matches_exact_spec(ref, rotate):
    extra = np.array([[0.0] * 32, [1e-40] + [0.0] * 31, [3.0e38] + [1.0] * 31,
                      [7.0, -6.5, 6.0, 5.0] * 8, [2.0 ** -130] * 32], np.float32)
    for name, x in list(tiny_tensors()) + [("edge", extra)]:
        x = x.reshape(-1, 32) if x.shape[1] % 32 else x
        out = ref.quantize(x, fmt=ref.MXFP4, rotate=rotate, errors=True)
        xp = ref.prepare(x, rotate=rotate)
        nib = ref.unpack_nibbles(out["codes"])
        for b, xb in enumerate(blocks_of(xp, 32)):
            sc, nb, e = X.quantize_block_mxfp4(xb)
            assert out["scales"][b] == sc, (name, b)
            assert list(nib[b * 32:(b + 1) * 32]) == nb, (name, b)
            assert abs(Fr(out["best"][b]) - e) <= e * Fr(1, 10 ** 12)


def test_given_global_scale_is_used(ref):
    x = synth.c1(rows=2, cols=64, seed=9)
    out = ref.quantize(x, rule=ref.SWEEP, global_scale=0.37)
    assert out["S"] == f32(0.37)
    for b, xb in enumerate(blocks_of(x, 16)):
        sc, nb, _, _ = X.quantize_block_nvfp4(xb, f32(0.37), (-3, 7))
        assert out["scales"][b] == sc
        assert list(ref.unpack_nibbles(out["codes"])[b * 16:(b + 1) * 16]) == nb


@pytest.mark.parametrize("window", [(3, 9), (-20, -10), (-126, 126), (0, 0)])
def test_windows_past_the_pattern_range(ref, window):
    # a window reaching past 0x01 or 0x7E tries the end pattern; one lying
    # wholly outside the range still yields a candidate
    x = np.array([[1536.0] + [0.3] * 15, [1e-6] * 16, list(np.linspace(-2, 3, 16))], np.float32)
    out = ref.quantize(x, rule=ref.SWEEP, window=window, errors=True)
    S = X.global_scale(np.abs(x).max())
    for b, xb in enumerate(blocks_of(x, 16)):
        sc, nb, e, _ = X.quantize_block_nvfp4(xb, S, window)
        assert out["scales"][b] == sc and 1 <= sc <= 0x7E
        assert list(ref.unpack_nibbles(out["codes"])[b * 16:(b + 1) * 16]) == nb


def test_importance_is_indexed_by_column(ref):
    # [out, in] weights: the importance weight of an element is that of its
    # input column, whatever the row (ScaleSweep page, Method 1: WMSE).
    rng = np.random.default_rng(4)
    x = rng.standard_normal((4, 32)).astype(np.float32)
    imp = np.ones(32, np.float32)
    imp[:16] = 1e-4          # first block of each row barely matters
    imp[5] = 1e4
    out = ref.quantize(x, rule=ref.SWEEP, objective=ref.WMSE, importance=imp, errors=True)
    S = X.global_scale(np.abs(x).max())
    for r in range(4):
        for j in range(2):
            xb = x[r, j * 16:(j + 1) * 16]
            sc, _, e, _ = X.quantize_block_nvfp4(xb, S, (-8, 7), imp[j * 16:(j + 1) * 16])
            assert out["scales"][r * 2 + j] == sc
