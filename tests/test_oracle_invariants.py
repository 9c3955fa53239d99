"""Pins of the oracle against hand-worked examples, brute force over all 126
scales, invariants the method guarantees, and statistical sanity (CPU)."""
import json
import os

import numpy as np
import pytest

import exactspec as X
from block_scaled_fp4_fp4q_amd import synth

f32 = np.float32
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


# --- hand-worked examples ------------------------------------------------------

def test_golden_nvfp4_absmax(ref):
    g = golden()["nvfp4_absmax_given_S"]
    x = np.array([g["x"]], np.float32)
    x[0, 4] = -0.0
    out = ref.quantize(x, global_scale=g["global_scale_given"], errors=True)
    assert list(out["scales"]) == g["scales"]
    assert list(out["codes"]) == g["codes"]
    assert out["best"][0] == g["block_error"]
    mse, _ = ref.error(x, out["codes"], out["scales"], out["S"])
    assert mse == g["mse"]
    _, wmse = ref.error(x, out["codes"], out["scales"], out["S"], importance=np.full(16, 2, np.float32))
    assert wmse == 2 * g["mse"]
    g2 = golden()["nvfp4_absmax_auto_S"]
    out = ref.quantize(x)
    assert out["S"] == g2["S"] and list(out["scales"]) == g2["scales"]
    assert list(out["codes"]) == g2["codes"]


def test_golden_nvfp4_sweep(ref):
    g = golden()["nvfp4_sweep_finds_exact_scale"]
    x = np.array([g["x"]], np.float32)
    a = ref.quantize(x, global_scale=g["global_scale_given"], errors=True)
    assert list(a["scales"]) == g["absmax_scales"] and list(a["codes"]) == g["absmax_codes"]
    assert a["best"][0] == g["absmax_block_error"]
    s = ref.quantize(x, rule=ref.SWEEP, global_scale=g["global_scale_given"], errors=True)
    assert list(s["scales"]) == g["sweep_scales"] and list(s["codes"]) == g["sweep_codes"]
    assert s["best"][0] == g["sweep_block_error"]


def test_golden_if4(ref):
    g = golden()["if4_int4_wins"]
    x = np.array([[f32(q) * (f32(6) / f32(7)) for q in g["q"]]], np.float32)
    assert x.max() == 6.0
    out = ref.quantize(x, fmt=ref.IF4, global_scale=g["global_scale_given"], errors=True)
    assert list(out["scales"]) == g["scales"] and list(out["codes"]) == g["codes"]
    assert out["best"][0] == 0.0 and out["second"][0] > 0
    y = ref.dequantize(out["codes"], out["scales"], out["S"], 1, 16, fmt=ref.IF4)
    assert np.array_equal(y, x)


def test_golden_mxfp4(ref):
    g = golden()["mxfp4_block"]
    x = np.array([g["x"]], np.float32)
    out = ref.quantize(x, fmt=ref.MXFP4)
    assert list(out["scales"]) == g["scales"] and list(out["codes"]) == g["codes"]
    g2 = golden()["mxfp4_small_block"]
    out = ref.quantize(x * f32(g2["x_scale"]), fmt=ref.MXFP4)
    assert list(out["scales"]) == g2["scales"] and list(out["codes"]) == g2["codes"]


# --- brute force over all 126 scales -------------------------------------------

def blocks_for(dist, n, seed):
    rng = np.random.default_rng(seed)
    if dist == "c1":
        x = synth.c1(rows=n * 16 // 1024 + 1, cols=1024, seed=seed).reshape(-1, 16)[:n]
    elif dist == "c2":
        x = synth.bf16_bits_to_f32(synth.c2(rows=n * 16 // 512 + 1, cols=512, seed=seed)[0])
        x = x.reshape(-1, 16)[:n]
    elif dist == "c4":
        x = synth.bf16_bits_to_f32(synth.c4(rows=n * 16 // 512 + 1, cols=512, seed=seed)[0])
        x = x.reshape(-1, 16)[:n]
    elif dist == "c5rot":
        x = rng.standard_normal((n, 16)).astype(np.float32) * rng.lognormal(0, 0.5, (n, 1)).astype(np.float32)
        spikes = rng.random((n, 16)) < 0.01
        x[spikes] *= 30
    else:
        raise ValueError(dist)
    return np.ascontiguousarray(x, np.float32)


@pytest.mark.parametrize("dist", ["c1", "c2", "c4", "c5rot"])
def test_mse_optimum_lies_in_window(ref, dist):
    # Lemmas 4.1 and 4.3 of the ScaleSweep page: the MSE-optimal FP8 scale lies
    # in [4/5, 12/7] x the block's max-based scale; in bit-pattern offsets from
    # the FP8-rounded base that is [-3, +7].  Brute force over all 126 bytes.
    # The bounds hold against the unrounded scale t = max|x|/(6S); the +7
    # pattern (ratio 1.78-1.88 to s_base) wins only when t was rounded down.
    n = 6000
    xb = blocks_for(dist, n, seed=100)
    if dist == "c5rot":
        xb = ref.prepare(xb.reshape(-1, 16), rotate=16)
    S = X.global_scale(np.abs(xb).max())
    E = ref.candidate_errors(xb, S)
    sb = np.array([ref.base_scale(b, S) for b in xb])
    live = sb > 0
    glob = np.nanargmin(E[:, 1:], axis=1) + 1         # ties -> lowest byte
    off = glob - sb
    assert np.all((off[live] >= -3) & (off[live] <= 7)), np.unique(off[live])
    L = ref.lib()
    ev = np.array([L.fp4q_ref_e4m3_value(b) for b in range(127)])
    t = (np.abs(xb).max(axis=1) / (f32(6) * S)).astype(np.float64)
    normal = sb >= 8
    ratio = ev[glob[normal]] / t[normal]
    assert ratio.min() >= 0.8 and ratio.max() <= 12 / 7, (ratio.min(), ratio.max())
    plus7 = live & (off == 7)
    assert np.all(t[plus7] > ev[sb[plus7]])             # base rounded down


@pytest.mark.parametrize("dist", ["c2", "c5rot"])
def test_wmse_optimum_mostly_in_window(ref, dist):
    # The WMSE lower bound 1/2 s_base (offset -8) is empirical on the page;
    # escapes are counted, and must stay rare for lognormal importance.
    n = 4000
    rng = np.random.default_rng(5)
    xb = blocks_for(dist, n, seed=200)
    w = rng.lognormal(0, 1, (n, 16)).astype(np.float32)
    S = X.global_scale(np.abs(xb).max())
    E = ref.candidate_errors(xb, S, w=w)
    sb = np.array([ref.base_scale(b, S) for b in xb])
    off = (np.nanargmin(E[:, 1:], axis=1) + 1) - sb
    escapes = np.mean((off < -8) | (off > 7))
    assert escapes < 0.01, escapes


@pytest.mark.parametrize("objective,window", [("mse", (-3, 7)), ("wmse", (-8, 7))])
def test_sweep_is_window_argmin_and_beats_absmax(ref, objective, window):
    rng = np.random.default_rng(9)
    x = synth.bf16_bits_to_f32(synth.c2(rows=64, cols=256, seed=3)[0])
    imp = rng.lognormal(0, 1, 256).astype(np.float32)
    obj = ref.MSE if objective == "mse" else ref.WMSE
    kw = dict(objective=obj, importance=imp if obj == ref.WMSE else None, errors=True)
    s = ref.quantize(x, rule=ref.SWEEP, window=window, **kw)
    a = ref.quantize(x, rule=ref.ABSMAX, **kw)
    assert np.all(s["best"] <= a["best"])                       # sweep <= AbsMax per block
    assert np.all(s["best"] <= s["second"])
    xb = x.reshape(-1, 16)
    wb = np.tile(imp.reshape(-1, 16), (64, 1)) if obj == ref.WMSE else None
    E = ref.candidate_errors(xb, s["S"], w=wb)
    for b in range(len(xb)):
        sb = int(a["scales"][b])
        cands = [c for c in range(sb + window[0], sb + window[1] + 1) if 1 <= c <= 0x7E]
        want = min(cands, key=lambda c: (E[b, c], c))
        assert s["scales"][b] == want
        assert s["best"][b] == E[b, want]
    mse_s = ref.error(x, s["codes"], s["scales"], s["S"])[0]
    mse_a = ref.error(x, a["codes"], a["scales"], a["S"])[0]
    assert mse_s < mse_a                                        # ScaleSweep beats AbsMax


def test_window_offsets_cover_lemma_bounds(ref):
    # Closed-form check of the page's offset claims over every base byte:
    # E4M3 values in [4/5 s, 12/7 s] are within offsets [-3, +6], values in
    # [1/2 s, 12/7 s] within [-8, +6]; -3 and -8 are attained.
    L = ref.lib()
    vals = [L.fp4q_ref_e4m3_value(b) for b in range(0x7F)]
    lo_mse, lo_w, hi_all = 0, 0, 0
    for b in range(0x10, 0x6F):  # normal bases whose whole window is finite
        s = vals[b]
        for c in range(1, 0x7F):
            if 0.8 * s <= vals[c] <= 12 / 7 * s:
                lo_mse = min(lo_mse, c - b)
                hi_all = max(hi_all, c - b)
            if 0.5 * s <= vals[c] <= 12 / 7 * s:
                lo_w = min(lo_w, c - b)
    assert (lo_mse, lo_w, hi_all) == (-3, -8, 6)


# --- invariants ------------------------------------------------------------------

def test_if4_never_worse_than_fp4(ref):
    x = synth.bf16_bits_to_f32(synth.c4(rows=64, cols=512, seed=8)[0])
    i = ref.quantize(x, fmt=ref.IF4, errors=True)
    f = ref.quantize(x, errors=True)
    assert i["S"] == f["S"]
    assert np.all(i["best"] <= f["best"])
    ind = (i["scales"] & 0x80) != 0
    assert np.all(i["second"][ind] > i["best"][ind])              # INT4 strictly lower
    assert np.array_equal(i["scales"] & 0x7F, f["scales"])        # same base scale
    assert np.array_equal(i["best"][~ind], f["best"][~ind])


def test_int4_code_seven_lands_on_fp4_max(ref):
    # The 6/7 method maps INT4's 7 onto FP4's 6 (IF4 page, Methodology).
    for sb in [0x20, 0x38, 0x45, 0x78]:
        S = f32(0.01)
        x = np.zeros((1, 16), np.float32)
        x[0, 0] = 1.0
        codes = np.array([0x07] + [0] * 7, np.uint8)
        scales = np.array([sb | 0x80], np.uint8)
        y = ref.dequantize(codes, scales, S, 1, 16, fmt=ref.IF4)
        D = f32(ref.lib().fp4q_ref_e4m3_value(sb)) * S
        assert abs(float(y[0, 0]) - 6 * float(D)) <= 4 * np.spacing(f32(6 * D))


def _grid_nvfp4(rng, nblocks, S):
    nib = rng.integers(0, 16, (nblocks, 16)).astype(np.uint8)
    nib[np.arange(nblocks), rng.integers(0, 16, nblocks)] = rng.choice([0x7, 0xF], nblocks)
    sc = rng.integers(0x02, 0x7E, nblocks).astype(np.uint8)
    D = np.array([f32(X.E4M3[c]) * S for c in sc], np.float32)
    val = np.array([float(v) for v in X.E2M1], np.float32)
    x = val[nib & 7] * D[:, None]
    x = np.where(nib & 8, -x, x).astype(np.float32)
    return x, nib, sc


def test_grid_tensors_round_trip_losslessly(ref):
    rng = np.random.default_rng(12)
    S = f32(0.03125)
    x, nib, sc = _grid_nvfp4(rng, 256, S)
    x = x.reshape(16, 256)
    for rule in (ref.ABSMAX, ref.SWEEP):
        out = ref.quantize(x, rule=rule, global_scale=S, errors=True)
        zero_neg = (nib & 7) == 0  # -0 and +0 codes both encode 0; compare values
        got = ref.unpack_nibbles(out["codes"]).reshape(-1, 16)
        assert np.array_equal(out["scales"], sc)
        assert np.array_equal(np.where(zero_neg, got & 7, got), np.where(zero_neg, nib & 7, nib))
        assert np.all(out["best"] == 0)
        y = ref.dequantize(out["codes"], out["scales"], S, 16, 256)
        assert np.array_equal(y, x)
        assert ref.error(x, out["codes"], out["scales"], S)[0] == 0.0
    # MXFP4: v * 2^e with a 6 in every block
    nib = rng.integers(0, 16, (64, 32)).astype(np.uint8)
    nib[:, 5] = 0x7
    e = rng.integers(-20, 20, 64)
    val = np.array([float(v) for v in X.E2M1], np.float32)
    xm = (val[nib & 7] * np.ldexp(1.0, e)[:, None]).astype(np.float32)
    xm = np.where(nib & 8, -xm, xm).astype(np.float32).reshape(16, 128)
    out = ref.quantize(xm, fmt=ref.MXFP4)
    assert np.array_equal(out["scales"], (e + 127).astype(np.uint8))
    assert np.array_equal(ref.dequantize(out["codes"], out["scales"], None, 16, 128, fmt=ref.MXFP4), xm)


def test_dequantize_then_error_in_original_domain(ref):
    x = synth.c3(rows=8, cols=128, seed=3)
    xf = synth.bf16_bits_to_f32(x)
    for rot in (0, 32):
        out = ref.quantize(x, fmt=ref.MXFP4, rotate=rot)
        y = ref.dequantize(out["codes"], out["scales"], None, 8, 128, fmt=ref.MXFP4, unrotate=rot)
        want = np.mean((xf.astype(np.float64) - y.astype(np.float64)) ** 2)
        got = ref.error(x, out["codes"], out["scales"], None, fmt=ref.MXFP4, rotate=rot)[0]
        assert abs(got - want) <= 1e-12 * want


# --- statistical sanity (the pages' qualitative claims) -----------------------------

def test_if4_picks_int4_for_uniform_and_fp4_for_spiky_blocks(ref):
    # IF4 page: evenly spread groups favour INT4, one-large-value groups FP4.
    xb, uni = synth.c4(rows=128, cols=512, seed=21)
    out = ref.quantize(xb, fmt=ref.IF4)
    ind = (out["scales"] & 0x80) != 0
    assert ind[uni].mean() > 0.8 and ind[~uni].mean() < 0.2, (ind[uni].mean(), ind[~uni].mean())


def test_hadamard_helps_mxfp4_with_outlier_channels(ref):
    # MR-GPTQ page: block Hadamard matters most for MXFP4.
    x = synth.c3(rows=256, cols=512, seed=4, n_outlier_channels=8)
    plain = ref.quantize(x, fmt=ref.MXFP4)
    rot = ref.quantize(x, fmt=ref.MXFP4, rotate=32)
    m0 = ref.error(x, plain["codes"], plain["scales"], None, fmt=ref.MXFP4)[0]
    m1 = ref.error(x, rot["codes"], rot["scales"], None, fmt=ref.MXFP4, rotate=32)[0]
    assert m1 < m0, (m0, m1)
