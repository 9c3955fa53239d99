"""Seeded random configurations against the oracle: format, rule, objective,
window, rotation, dtype, given or computed global scale, shape and value
distribution drawn per case, so that combinations the enumerated parity
tests do not name are covered too.  Bar: codes, scale bytes and the global
scale bit-exact; dequantized values (binary32 or bf16) bit-exact on every fourth case."""
import numpy as np
import pytest
import torch

from block_scaled_fp4_fp4q_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
CASES = 1000


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_scaled_fp4_fp4q_amd import binding
    binding.lib()
    return binding


def to_dev(x):
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def values(rng, rows, cols, block):
    """One of six value distributions, times a random power of ten, with
    about 5% of the blocks zeroed."""
    kind = int(rng.integers(0, 6))
    nb = cols // block
    if kind == 0:
        x = rng.standard_normal((rows, cols))
    elif kind == 1:
        x = rng.standard_t(3, (rows, cols))
    elif kind == 2:  # sparse Laplace
        x = rng.laplace(size=(rows, cols)) * (rng.random((rows, cols)) < 0.2)
    elif kind == 3:  # on an E2M1 grid with a power-of-two step per block
        step = 2.0 ** rng.integers(-3, 4, (rows, nb)).repeat(block, axis=1)
        x = rng.integers(-12, 13, (rows, cols)) * 0.5 * step
    elif kind == 4:  # constant blocks
        x = np.repeat(rng.standard_normal((rows, nb)), block, axis=1)
    else:  # wide dynamic range
        x = rng.lognormal(0.0, 3.0, (rows, cols)) * rng.choice([-1.0, 1.0], (rows, cols))
    x = x * 10.0 ** rng.uniform(-15, 15)
    zero = np.repeat(rng.random((rows, nb)) < 0.05, block, axis=1)
    return np.where(zero, 0.0, x).astype(np.float32), kind


def draw(seed, B, fmts=("nvfp4", "mxfp4", "if4")):
    rng = np.random.default_rng(seed)
    fmt = fmts[int(rng.integers(0, len(fmts)))]
    block = 32 if fmt == "mxfp4" else 16
    rules = [B.FP4Q_SCALE_ABSMAX, B.FP4Q_SCALE_SWEEP] + ([B.FP4Q_SCALE_FOUR_OVER_SIX] if fmt == "nvfp4" else [])
    rule = rules[int(rng.integers(0, len(rules)))]
    objective = int(rng.integers(0, 2))
    rotate = block if rng.random() < 0.4 else 0
    window = None
    if rule == B.FP4Q_SCALE_SWEEP:
        if fmt == "mxfp4":
            lo = int(rng.integers(-3, 2))
            window = (lo, lo + int(rng.integers(0, 4)))
        elif rng.random() < 0.5:
            window = [(-3, 7), (-8, 7)][int(rng.integers(0, 2))]
        else:
            lo = int(rng.integers(-12, 3))
            window = (lo, lo + int(rng.integers(0, 16)))
    rows = int(rng.integers(1, 41))
    cols = block * int(rng.integers(1, 41))
    x, kind = values(rng, rows, cols, block)
    bf16 = rng.random() < 0.5
    imp = rng.lognormal(0.0, 2.0, cols).astype(np.float32)
    if rng.random() < 0.2:
        imp[rng.random(cols) < 0.3] = 0.0
    given = None
    if fmt != "mxfp4" and rng.random() < 0.3:
        if rng.random() < 0.5:  # near the computed scale
            g = float(np.abs(x).max()) / 1536.0 * 2.0 ** rng.uniform(-4, 4)
        else:  # anywhere in the allowed range
            g = 2.0 ** rng.uniform(-117, 119)
        given = float(np.float32(min(max(g, 2.0 ** -117), 2.0 ** 119)))
    return dict(fmt=fmt, rule=rule, objective=objective, rotate=rotate, window=window,
                x=synth.f32_to_bf16_bits(x) if bf16 else x, imp=imp, given=given, kind=kind)


def formats(B, ref):
    return ({"nvfp4": B.FP4Q_NVFP4, "mxfp4": B.FP4Q_MXFP4, "if4": B.FP4Q_IF4, "if3": B.FP4Q_IF3,
             "if6": B.FP4Q_IF6},
            {"nvfp4": ref.NVFP4, "mxfp4": ref.MXFP4, "if4": ref.IF4, "if3": ref.IF3, "if6": ref.IF6})


@pytest.mark.parametrize("case", range(CASES))
def test_random_configuration(B, ref, case):
    check_case(B, ref, case, draw(1000 + case, B))


@pytest.mark.parametrize("case", range(300))
def test_random_adaptive(B, ref, case):
    """IF3 and IF6 (AbsMax and pattern windows) drawn the same way."""
    check_case(B, ref, case, draw(7000 + case, B, fmts=("if3", "if6")))


def check_case(B, ref, case, c):
    bfmts, ofmts = formats(B, ref)
    bfmt, ofmt = bfmts[c["fmt"]], ofmts[c["fmt"]]
    x, imp, wmse = c["x"], c["imp"], c["objective"] == 1
    print(f"case {case}: {c['fmt']} rule {c['rule']} objective {c['objective']} rotate {c['rotate']} "
          f"window {c['window']} shape {x.shape} {x.dtype} kind {c['kind']} given {c['given']}", flush=True)
    xd = to_dev(x)
    codes, scales, gs = B.quantize(xd, format=bfmt, scale_rule=c["rule"], objective=c["objective"],
                                   window=c["window"], rotate=c["rotate"],
                                   importance=to_dev(imp) if wmse else None, global_scale=c["given"])
    torch.cuda.synchronize()
    want = ref.quantize(x, fmt=ofmt, rule=c["rule"], objective=c["objective"], window=c["window"],
                        rotate=c["rotate"], importance=imp if wmse else None, global_scale=c["given"])
    if c["fmt"] != "mxfp4":
        assert gs.cpu().numpy()[0] == np.float32(want["S"])
    got_s = scales.cpu().numpy()
    bad = np.nonzero(got_s != want["scales"])[0]
    assert bad.size == 0, f"{bad.size} scale mismatches, first blocks {bad[:5]}"
    assert np.array_equal(codes.cpu().numpy(), want["codes"])
    if case % 4 == 0:  # dequantize, binary32 or (every other time) bf16 output
        rows, cols = x.shape
        bf16_out = case % 8 == 4
        y = B.dequantize(codes, scales, gs, rows, cols, format=bfmt, unrotate=c["rotate"],
                         dtype=torch.bfloat16 if bf16_out else torch.float32)
        yw = ref.dequantize(want["codes"], want["scales"], want.get("S"), rows, cols, fmt=ofmt,
                            unrotate=c["rotate"], out_dtype=ref.BF16 if bf16_out else ref.F32)
        if bf16_out:
            assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), yw)
        else:
            assert np.array_equal(y.cpu().numpy().view(np.uint32), np.asarray(yw, np.float32).view(np.uint32))


@pytest.mark.parametrize("case", range(200))
def test_random_relaxed(B, ref, case):
    """FOCUS deploy encode: format, coefficient group, given or computed
    scale bytes and global scale, dtype, shape and values drawn per case."""
    rng = np.random.default_rng(5000 + case)
    fmt = ["nvfp4", "mxfp4"][int(rng.integers(0, 2))]
    block = 32 if fmt == "mxfp4" else 16
    group = [8, block][int(rng.integers(0, 2))]
    rows, cols = int(rng.integers(1, 41)), block * int(rng.integers(1, 41))
    x, kind = values(rng, rows, cols, block)
    if rng.random() < 0.5:
        x = synth.f32_to_bf16_bits(x)
    coef = rng.lognormal(0.0, [0.1, 1.5][int(rng.integers(0, 2))], (rows, cols // group)).astype(np.float32)
    given_scales = None
    if rng.random() < 0.3:
        top = 0xFE if fmt == "mxfp4" else 0x7E
        given_scales = rng.integers(0, top + 1, rows * cols // block).astype(np.uint8)
    given_S = None
    if fmt == "nvfp4" and rng.random() < 0.3:
        xf = synth.bf16_bits_to_f32(x) if x.dtype == np.uint16 else x
        g = float(np.abs(xf).max()) / 1536.0 * 2.0 ** rng.uniform(-4, 4)
        if rng.random() < 0.5:
            g = 2.0 ** rng.uniform(-117, 119)
        given_S = float(np.float32(min(max(g, 2.0 ** -117), 2.0 ** 119)))
    print(f"case {case}: {fmt} group {group} shape {x.shape} {x.dtype} kind {kind} "
          f"scales given {given_scales is not None} S {given_S}", flush=True)
    bfmt = B.FP4Q_MXFP4 if fmt == "mxfp4" else B.FP4Q_NVFP4
    codes, scales, gs = B.quantize_relaxed(
        to_dev(x), to_dev(coef), group, format=bfmt,
        scales=None if given_scales is None else to_dev(given_scales), global_scale=given_S)
    torch.cuda.synchronize()
    want = ref.quantize_relaxed(x, coef, group, fmt=ref.MXFP4 if fmt == "mxfp4" else ref.NVFP4,
                                global_scale=given_S, scales=given_scales)
    if fmt == "nvfp4":
        assert gs.cpu().numpy()[0] == np.float32(want["S"])
    assert np.array_equal(scales.cpu().numpy(), want["scales"])
    assert np.array_equal(codes.cpu().numpy(), want["codes"])


@pytest.mark.parametrize("case", range(128))
def test_random_error(B, ref, case):
    """MSE and WMSE of a random configuration's quantization against the
    oracle's binary64 sums (1e-10 relative: only the order of the sums differs)."""
    c = draw(9000 + case, B)
    bfmt = {"nvfp4": B.FP4Q_NVFP4, "mxfp4": B.FP4Q_MXFP4, "if4": B.FP4Q_IF4}[c["fmt"]]
    ofmt = {"nvfp4": ref.NVFP4, "mxfp4": ref.MXFP4, "if4": ref.IF4}[c["fmt"]]
    x, imp = c["x"], c["imp"]
    xd = to_dev(x)
    codes, scales, gs = B.quantize(xd, format=bfmt, scale_rule=c["rule"], objective=c["objective"],
                                   window=c["window"], rotate=c["rotate"],
                                   importance=to_dev(imp) if c["objective"] == 1 else None,
                                   global_scale=c["given"])
    got = B.error(xd, codes, scales, gs, format=bfmt, rotate=c["rotate"], importance=to_dev(imp))
    S = float(gs.cpu().numpy()[0]) if c["fmt"] != "mxfp4" else None
    want = ref.error(x, codes.cpu().numpy(), scales.cpu().numpy(), S, fmt=ofmt, rotate=c["rotate"],
                     importance=imp)
    for g, w in zip(got, want):
        assert g == pytest.approx(w, rel=1e-10, abs=1e-300)
