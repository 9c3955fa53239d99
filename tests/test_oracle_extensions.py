"""Pins of the oracle's extensions of the search (CPU): Four Over Six, the
MXFP4 exponent window, IF4 over a window, and the FOCUS deploy-side encode --
each against the exact-rational statement, hand-worked blocks and the
invariants they must satisfy."""
import numpy as np
import pytest

import exactspec as X
from block_scaled_fp4_fp4q_amd import synth
from test_oracle_spec import adversarial_nvfp4, tiny_tensors

f32 = np.float32


def blocks(x, B):
    return np.ascontiguousarray(x, np.float32).reshape(-1, B)


@pytest.mark.parametrize("objective", [0, 1])
def test_four_over_six_matches_exact_spec(ref, objective):
    rng = np.random.default_rng(1)
    for name, x in tiny_tensors():
        imp = rng.lognormal(0, 1, x.shape[1]).astype(np.float32)
        out = ref.quantize(x, rule=ref.FOUR_SIX, objective=objective,
                           importance=imp if objective else None, errors=True)
        S = X.global_scale(np.abs(x).max())
        nib = ref.unpack_nibbles(out["codes"])
        for b, xb in enumerate(blocks(x, 16)):
            c0 = (b * 16) % x.shape[1]
            sc, nb, e = X.quantize_block_foursix(xb, S, imp[c0:c0 + 16] if objective else None)
            assert out["scales"][b] == sc, (name, b)
            assert list(nib[b * 16:(b + 1) * 16]) == nb


def test_four_over_six_hand_block_and_invariants(ref):
    # S = 1: max 4 -> 6-scale 0x33 (0.6875, lossy), 4-scale 0x38 (1.0):
    # 4, 3, 2, 1, 0.5 are all on the grid -> error 0, scale 0x38
    x = np.array([[4, 3, 2, 1, 0.5, 0, -4, -3, 2, 1, 0.5, 0, 4, 3, 2, 1]], np.float32)
    out = ref.quantize(x, rule=ref.FOUR_SIX, global_scale=1.0, errors=True)
    assert out["scales"][0] == 0x38 and out["best"][0] == 0.0
    assert ref.quantize(x, global_scale=1.0)["scales"][0] == 0x33
    y = synth.bf16_bits_to_f32(synth.c2(rows=64, cols=256, seed=7)[0])
    f = ref.quantize(y, rule=ref.FOUR_SIX, errors=True)
    a = ref.quantize(y, errors=True)
    s = ref.quantize(y, rule=ref.SWEEP, errors=True)
    assert np.all(f["best"] <= a["best"])         # never worse than AbsMax
    assert np.mean(s["best"]) <= np.mean(f["best"])  # the sweep (which contains
    # s6 but not always s4) still wins on average: ScaleSweep Results


@pytest.mark.parametrize("window", [(0, 1), (-1, 1), (0, 0), (-2, 3)])
def test_mxfp4_window_matches_exact_spec(ref, window):
    x = synth.c3(rows=6, cols=64, seed=2, n_outlier_channels=2)
    xf = synth.bf16_bits_to_f32(x)
    extra = np.array([[0.0] * 32 + [7.0, -6.5, 6.0, 5.0] * 8, [1e-30] * 64], np.float32)
    for xx in (xf, extra, adversarial_nvfp4().reshape(-1, 64)):
        out = ref.quantize(xx, fmt=ref.MXFP4, rule=ref.SWEEP, window=window, errors=True)
        nib = ref.unpack_nibbles(out["codes"])
        for b, xb in enumerate(blocks(xx, 32)):
            sc, nb, e = X.quantize_block_mx_sweep(xb, window)
            assert out["scales"][b] == sc, b
            assert list(nib[b * 32:(b + 1) * 32]) == nb


def test_mxfp4_search_never_worse_and_optimum_location(ref):
    x = synth.c3(rows=128, cols=512, seed=9)
    ocp = ref.quantize(x, fmt=ref.MXFP4, errors=True)
    s = ref.quantize(x, fmt=ref.MXFP4, rule=ref.SWEEP, window=(0, 1), errors=True)
    wide = ref.quantize(x, fmt=ref.MXFP4, rule=ref.SWEEP, window=(-4, 4), errors=True)
    assert np.all(s["best"] <= ocp["best"])
    # the {e, e+1} window (OCP and ceil(log2(max/6))) already holds the
    # brute-force optimum for these blocks
    assert np.array_equal(wide["scales"], s["scales"])
    assert np.mean((s["scales"] != ocp["scales"])) > 0.05


@pytest.mark.parametrize("window", [(-3, 7), (0, 0), (-1, 2)])
def test_if4_window_matches_exact_spec(ref, window):
    for name, x in tiny_tensors():
        out = ref.quantize(x, fmt=ref.IF4, rule=ref.SWEEP, window=window, errors=True)
        S = X.global_scale(np.abs(x).max())
        nib = ref.unpack_nibbles(out["codes"])
        for b, xb in enumerate(blocks(x, 16)):
            sc, nb, e = X.quantize_block_if4_sweep(xb, S, window)
            assert out["scales"][b] == sc, (name, b)
            assert list(nib[b * 16:(b + 1) * 16]) == nb


def test_if4_window_invariants(ref):
    x = synth.c4(rows=32, cols=512, seed=3)[0]
    i1 = ref.quantize(x, fmt=ref.IF4, errors=True)
    i0 = ref.quantize(x, fmt=ref.IF4, rule=ref.SWEEP, window=(0, 0), errors=True)
    iw = ref.quantize(x, fmt=ref.IF4, rule=ref.SWEEP, window=(-3, 7), errors=True)
    sw = ref.quantize(x, rule=ref.SWEEP, window=(-3, 7), errors=True)
    assert np.array_equal(i0["scales"], i1["scales"]) and np.array_equal(i0["codes"], i1["codes"])
    assert np.all(iw["best"] <= i1["best"]) and np.all(iw["best"] <= sw["best"])


@pytest.mark.parametrize("fmt,group", [("nvfp4", 8), ("nvfp4", 16), ("mxfp4", 8), ("mxfp4", 32)])
def test_relaxed_encode_matches_exact_spec(ref, fmt, group):
    rng = np.random.default_rng(group)
    F = ref.NVFP4 if fmt == "nvfp4" else ref.MXFP4
    B = 16 if fmt == "nvfp4" else 32
    x = synth.c1(rows=4, cols=128, seed=3)
    coef = rng.uniform(0.8, 1.25, (4, 128 // group)).astype(np.float32)
    out = ref.quantize_relaxed(x, coef, group, fmt=F)
    S = X.global_scale(np.abs(x).max())
    nib = ref.unpack_nibbles(out["codes"])
    for b, xb in enumerate(blocks(x, B)):
        r, jb = divmod(b, 128 // B)
        cs = [coef[r, (jb * B + i) // group] for i in range(B)]
        sc, nb = X.relaxed_block(xb, S, cs, fmt=fmt)
        assert out["scales"][b] == sc and list(nib[b * B:(b + 1) * B]) == nb
    # caller-given stored scales
    given = rng.integers(0x30, 0x50, x.size // B).astype(np.uint8) if fmt == "nvfp4" else \
        rng.integers(120, 130, x.size // B).astype(np.uint8)
    out = ref.quantize_relaxed(x, coef, group, fmt=F, scales=given, global_scale=0.05)
    assert np.array_equal(out["scales"], given)
    nib = ref.unpack_nibbles(out["codes"])
    for b, xb in enumerate(blocks(x, B)):
        r, jb = divmod(b, 128 // B)
        cs = [coef[r, (jb * B + i) // group] for i in range(B)]
        _, nb = X.relaxed_block(xb, f32(0.05), cs, byte=int(given[b]), fmt=fmt)
        assert list(nib[b * B:(b + 1) * B]) == nb


def test_relaxed_encode_with_infinite_reciprocal(ref):
    # given steps with D c below 2^-128 (E8M0 byte 0, E4M3 byte 1 under the
    # smallest allowed S): r_q = fl(1/D_q) is +inf, zero elements keep code 0
    # (|x| / S_q = 0) and every other element saturates
    rng = np.random.default_rng(7)
    x = rng.standard_normal((2, 64)).astype(np.float32)
    x[0, ::3] = 0.0
    x[1, 1::4] = -0.0
    x[1, 2::4] *= np.float32(2.0 ** -140)
    for F, B, byte, S in ((ref.MXFP4, 32, 0, None), (ref.NVFP4, 16, 1, 2.0 ** -117)):
        fmt = "mxfp4" if F == ref.MXFP4 else "nvfp4"
        for group in (8, B):
            coef = np.full((2, 64 // group), 0.25, np.float32)
            coef[:, ::2] = 1.0
            given = np.full(x.size // B, byte, np.uint8)
            out = ref.quantize_relaxed(x, coef, group, fmt=F, scales=given, global_scale=S)
            nib = ref.unpack_nibbles(out["codes"])
            for b, xb in enumerate(blocks(x, B)):
                r, jb = divmod(b, 64 // B)
                cs = [coef[r, (jb * B + i) // group] for i in range(B)]
                _, nb = X.relaxed_block(xb, f32(S if S else 1.0), cs, byte=byte, fmt=fmt)
                assert list(nib[b * B:(b + 1) * B]) == nb
            zero = x.reshape(-1) == 0
            assert np.all(nib[zero] & 7 == 0)


def test_relaxed_with_unit_coefficients_is_absmax(ref):
    # FOCUS initializes its coefficients to 1: S_q = S_dq, the AbsMax baseline
    x = synth.bf16_bits_to_f32(synth.c2(rows=32, cols=256, seed=4)[0])
    for F, B in ((ref.NVFP4, 16), (ref.MXFP4, 32)):
        for group in (8, B):
            out = ref.quantize_relaxed(x, np.ones((32, 256 // group), np.float32), group, fmt=F)
            a = ref.quantize(x, fmt=F)
            assert np.array_equal(out["scales"], a["scales"]) and np.array_equal(out["codes"], a["codes"])
