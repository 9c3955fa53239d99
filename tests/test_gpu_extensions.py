"""GPU parity of the extension rules against the CPU oracle, through the C ABI:
Four Over Six (NVFP4), the E8M0 exponent window (MXFP4), the IF4 pattern
window, and the FOCUS deploy-side encode with given coefficients.

Each kernel's choice equals the binary64 comparison of the oracle's binary32
encodes (from certified estimates, or the exact fallback where those do not
separate), so codes, scale bytes, indicators and the global scale must be
bit-exact.
Sizes span several workgroups and end on a ragged tail; edge blocks cover
zeros, signed zeros, subnormal and clamped scales, and saturation."""
import numpy as np
import pytest
import torch

from block_scaled_fp4_fp4q_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


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


def weights(cols, seed):
    return np.random.default_rng(seed).lognormal(0, 1, cols).astype(np.float32)


def student(rows, cols, seed, dtype):
    x = (np.random.default_rng(seed).standard_t(4, (rows, cols)) * 0.02).astype(np.float32)
    return synth.f32_to_bf16_bits(x) if dtype == "bf16" else x


def compare(B, ref, x, fmt, rule, objective=0, window=None, rotate=0, imp=None, given=None):
    ofmt = {B.FP4Q_NVFP4: ref.NVFP4, B.FP4Q_MXFP4: ref.MXFP4, B.FP4Q_IF4: ref.IF4}[fmt]
    orule = {B.FP4Q_SCALE_ABSMAX: ref.ABSMAX, B.FP4Q_SCALE_SWEEP: ref.SWEEP,
             B.FP4Q_SCALE_FOUR_OVER_SIX: ref.FOUR_SIX}[rule]
    if window is None and rule == B.FP4Q_SCALE_SWEEP:
        window = ref.default_window(objective, ofmt)
    codes, scales, gs = B.quantize(to_dev(x), format=fmt, scale_rule=rule, objective=objective,
                                   window=window, rotate=rotate,
                                   importance=to_dev(imp) if objective == 1 else None,
                                   global_scale=given)
    torch.cuda.synchronize()
    want = ref.quantize(x, fmt=ofmt, rule=orule, objective=objective, window=window,
                        rotate=rotate, importance=imp if objective == 1 else None,
                        global_scale=given, errors=True)
    if fmt != B.FP4Q_MXFP4:
        assert gs.item() == np.float32(want["S"])
    s = scales.cpu().numpy()
    bad = np.nonzero(s != want["scales"])[0]
    assert bad.size == 0, f"{bad.size} scale mismatches, first blocks {bad[:5]}"
    assert np.array_equal(codes.cpu().numpy(), want["codes"])
    return s, want


# ---------------------------------------------------------------------------
# Four Over Six
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rotate", [0, 16])
@pytest.mark.parametrize("objective", [0, 1])
def test_four_over_six(B, ref, dtype, rotate, objective):
    x = student(37, 528, seed=40 + rotate + objective, dtype=dtype)   # 1221 blocks
    s, want = compare(B, ref, x, B.FP4Q_NVFP4, B.FP4Q_SCALE_FOUR_OVER_SIX, objective,
                      rotate=rotate, imp=weights(528, 41))
    base = ref.quantize(x, rotate=rotate)["scales"]
    four = np.mean(s != base)
    assert 0.0 < four < 1.0, four          # both choices occur on heavy-tailed data


# ---------------------------------------------------------------------------
# MXFP4 exponent window
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rotate", [0, 32])
@pytest.mark.parametrize("objective", [0, 1])
def test_mxfp4_window(B, ref, dtype, rotate, objective):
    x = synth.c3(rows=53, cols=352, seed=50 + rotate + objective, n_outlier_channels=3)
    if dtype == "f32":
        x = synth.bf16_bits_to_f32(x)
    s, _ = compare(B, ref, x, B.FP4Q_MXFP4, B.FP4Q_SCALE_SWEEP, objective, rotate=rotate,
                   imp=weights(352, 51))
    base = ref.quantize(x, fmt=ref.MXFP4, rotate=rotate)["scales"]
    assert np.all((s == base) | (s == base + 1))


@pytest.mark.parametrize("window", [(-2, 2), (-126, 126), (3, 3), (-5, -1)])
def test_mxfp4_wide_windows(B, ref, window):
    x = synth.c3(rows=11, cols=320, seed=52, n_outlier_channels=2)
    compare(B, ref, x, B.FP4Q_MXFP4, B.FP4Q_SCALE_SWEEP, 0, window=window)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mxfp4_window_extremes(B, ref, dtype):
    # exponents clamped at both ends of E8M0, subnormal inputs, zero blocks,
    # signed zeros and values that saturate, on both input types
    rng = np.random.default_rng(53)
    x = rng.standard_normal((8, 128)).astype(np.float32)
    x[0] *= np.float32(2.0 ** -140)        # subnormal, OCP exponent below -127
    x[1, :32] = 0.0
    x[1, 32:64] = -0.0
    x[2] *= np.float32(2.0 ** 120)         # exponents near the top
    x[3, :32] = np.float32(3.0e38)
    x[3, 5] = -np.float32(3.4e38)
    x[4, :32] = np.float32(7.9)            # above 6 * 2^e: saturation at e, exact at e+1
    x[5, :32] = np.float32(2.0 ** -149)    # smallest subnormal
    if dtype == "bf16":
        x[3, 5] = -np.float32(3.38e38)     # -3.4e38 would round to -inf (inputs must be finite)
        x = synth.f32_to_bf16_bits(x)
    for window in ((0, 1), (-126, 126), (-3, 3)):
        compare(B, ref, x, B.FP4Q_MXFP4, B.FP4Q_SCALE_SWEEP, 0, window=window)


# ---------------------------------------------------------------------------
# IF4 over a pattern window
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rotate", [0, 16])
@pytest.mark.parametrize("objective", [0, 1])
def test_if4_window(B, ref, dtype, rotate, objective):
    x = synth.c4(rows=41, cols=336, seed=60 + rotate + objective)[0]
    if dtype == "f32":
        x = synth.bf16_bits_to_f32(x)
    s, _ = compare(B, ref, x, B.FP4Q_IF4, B.FP4Q_SCALE_SWEEP, objective, rotate=rotate,
                   imp=weights(336, 61))
    ind = (s & 0x80) != 0
    assert 0.0 < ind.mean() < 1.0


@pytest.mark.parametrize("window", [(0, 0), (-126, 126), (-8, 7), (4, 9), (-5, -2), (-9, 6)])
def test_if4_windows_and_given_scale(B, ref, window):
    x = synth.c4(rows=9, cols=256, seed=62)[0]
    compare(B, ref, x, B.FP4Q_IF4, B.FP4Q_SCALE_SWEEP, 0, window=window)
    compare(B, ref, x, B.FP4Q_IF4, B.FP4Q_SCALE_SWEEP, 0, window=window, given=0.004)
    # a given S this small saturates s_base at 0x7E for most blocks
    compare(B, ref, x, B.FP4Q_IF4, B.FP4Q_SCALE_SWEEP, 0, window=window, given=1e-4)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("objective", [0, 1])
def test_if4_window_exact_ties_everywhere(B, ref, objective):
    # three blocks in four are one element 6 S (E4M3 1.0) among zeros under a
    # given S = 1/16: FP4 codes at patterns 1.0 (code 6) and 1.5 (code 4)
    # both reconstruct it exactly, an exact tie that no estimate certifies.
    # With 786432 blocks every wave meets more than 64 of them and drains its
    # queue inside the grid-stride loop as well as at the end.  The remaining
    # blocks mix random values with tiny ones (subnormal s_base).
    rows, cols = 6144, 2048
    rng = np.random.default_rng(66 + objective)
    x = np.zeros((rows * cols // 16, 16), np.float32)
    kind = rng.integers(0, 4, x.shape[0])
    tie = kind < 3
    x[np.nonzero(tie)[0], rng.integers(0, 16, tie.sum())] = 0.375
    n = (~tie).sum()
    vals = rng.standard_normal((n, 16)).astype(np.float32) * np.float32(0.2)
    vals[::7] *= np.float32(2.0 ** -14)          # s_base in E4M3's subnormal range
    x[~tie] = vals
    x = x.reshape(rows, cols)
    imp = weights(cols, 67)
    s, _ = compare(B, ref, x, B.FP4Q_IF4, B.FP4Q_SCALE_SWEEP, objective, window=(-3, 7), imp=imp,
                   given=1.0 / 16)
    # the first zero error in the method's order: FP4 at s_base = E4M3 1.0
    assert np.all(s[tie] == 0x38)


def test_extension_edge_blocks(B, ref):
    rng = np.random.default_rng(63)
    x = rng.standard_normal((6, 192)).astype(np.float32)
    x[0, :16] = 0.0
    x[0, 16:32] = -0.0
    x[1] *= np.float32(1e-30)                # scales clamped to 0x01 under a large S
    x[2, :16] = np.float32(0.25)             # exact E2M1 midpoints
    x[2, 16:32] = np.float32(1.75)
    x[3, 40] = np.float32(1e4)               # the tensor maximum, everything else small
    imp = weights(192, 64)
    for objective in (0, 1):
        compare(B, ref, x, B.FP4Q_NVFP4, B.FP4Q_SCALE_FOUR_OVER_SIX, objective, imp=imp)
        compare(B, ref, x, B.FP4Q_IF4, B.FP4Q_SCALE_SWEEP, objective, imp=imp)
        compare(B, ref, x, B.FP4Q_MXFP4, B.FP4Q_SCALE_SWEEP, objective, imp=imp)


def test_extension_empty(B):
    for fmt, rule in ((B.FP4Q_NVFP4, B.FP4Q_SCALE_FOUR_OVER_SIX),
                      (B.FP4Q_MXFP4, B.FP4Q_SCALE_SWEEP), (B.FP4Q_IF4, B.FP4Q_SCALE_SWEEP)):
        x = torch.empty(0, 64, dtype=torch.bfloat16, device=DEV)
        codes, scales, gs = B.quantize(x, format=fmt, scale_rule=rule)
        torch.cuda.synchronize()
        assert codes.numel() == 0 and scales.numel() == 0
        if fmt != B.FP4Q_MXFP4:
            assert gs.item() == 1.0


# ---------------------------------------------------------------------------
# FOCUS deploy-side encode
# ---------------------------------------------------------------------------

def coefficients(rows, cols, group, seed):
    # relaxation coefficients near 1, as learned scale adjustments are
    return np.random.default_rng(seed).lognormal(0.0, 0.08, (rows, cols // group)).astype(np.float32)


def relaxed_case(B, ref, x, fmt, group, given_scales=None, gs=None, seed=0):
    rows, cols = x.shape
    c = coefficients(rows, cols, group, seed)
    ofmt = ref.MXFP4 if fmt == B.FP4Q_MXFP4 else ref.NVFP4
    sd = to_dev(given_scales) if given_scales is not None else None
    codes, scales, S = B.quantize_relaxed(to_dev(x), to_dev(c), group, format=fmt, scales=sd,
                                          global_scale=gs)
    torch.cuda.synchronize()
    want = ref.quantize_relaxed(x, c, group, fmt=ofmt, global_scale=gs, scales=given_scales)
    if fmt != B.FP4Q_MXFP4:
        assert S.item() == np.float32(want["S"])
    assert np.array_equal(scales.cpu().numpy(), want["scales"])
    assert np.array_equal(codes.cpu().numpy(), want["codes"])
    return codes, scales, S


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("fmt,group", [("nvfp4", 8), ("nvfp4", 16), ("mxfp4", 8), ("mxfp4", 32)])
def test_relaxed(B, ref, dtype, fmt, group):
    f = B.FP4Q_MXFP4 if fmt == "mxfp4" else B.FP4Q_NVFP4
    x = student(29, 544, seed=70 + group, dtype=dtype)
    codes, scales, S = relaxed_case(B, ref, x, f, group, seed=71 + group)
    # the stored scales are the AbsMax ones: only the codes move
    plain = B.quantize(to_dev(x), format=f)
    torch.cuda.synchronize()
    assert torch.equal(plain[1], scales)
    assert not torch.equal(plain[0], codes)


@pytest.mark.parametrize("fmt,group", [("nvfp4", 8), ("nvfp4", 16), ("mxfp4", 8), ("mxfp4", 32)])
def test_relaxed_given_scales(B, ref, fmt, group):
    f = B.FP4Q_MXFP4 if fmt == "mxfp4" else B.FP4Q_NVFP4
    blk = 32 if fmt == "mxfp4" else 16
    x = student(19, 448, seed=80 + group, dtype="bf16")
    rng = np.random.default_rng(81 + group)
    nb = x.size // blk
    if fmt == "mxfp4":
        sc = rng.integers(0x70, 0x80, nb).astype(np.uint8)
        sc[:3] = (0x00, 0xFE, 0x01)                         # E8M0 range ends
    else:
        sc = rng.integers(0x20, 0x48, nb).astype(np.uint8)
        sc[:3] = (0x00, 0x7E, 0x01)                         # zero step, largest, subnormal
    relaxed_case(B, ref, x, f, group, given_scales=sc, seed=82)
    if fmt == "nvfp4":
        relaxed_case(B, ref, x, f, group, given_scales=sc, gs=0.001, seed=83)


def test_relaxed_edges_and_empty(B, ref):
    rng = np.random.default_rng(90)
    x = rng.standard_normal((4, 96)).astype(np.float32)
    x[0, :16] = 0.0
    x[0, 16:32] = -0.0
    x[1] *= np.float32(2.0 ** -135)
    x[2, :8] = np.float32(6.0)
    # binary32 input runs one lane per block, bf16 input B/8 lanes per block
    for xin in (x, synth.f32_to_bf16_bits(x)):
        for f in (B.FP4Q_NVFP4, B.FP4Q_MXFP4):
            for group in (8, 16 if f == B.FP4Q_NVFP4 else 32):
                relaxed_case(B, ref, xin, f, group, seed=91)
    e = torch.empty(0, 64, dtype=torch.float32, device=DEV)
    c = torch.empty(0, 8, dtype=torch.float32, device=DEV)
    codes, scales, S = B.quantize_relaxed(e, c, 8)
    torch.cuda.synchronize()
    assert codes.numel() == 0 and S.item() == 1.0


def test_wide_importance_vector(B, ref):
    # more columns than the kernels keep square roots of in LDS (4096): the
    # per-block square-root path of every weighted kernel
    cols = 4096 + 512
    x = student(7, cols, seed=95, dtype="bf16")
    imp = weights(cols, 96)
    compare(B, ref, x, B.FP4Q_NVFP4, B.FP4Q_SCALE_SWEEP, 1, window=(-8, 7), imp=imp)
    compare(B, ref, x, B.FP4Q_NVFP4, B.FP4Q_SCALE_SWEEP, 1, window=(-3, 7), rotate=16, imp=imp)
    compare(B, ref, x, B.FP4Q_NVFP4, B.FP4Q_SCALE_FOUR_OVER_SIX, 1, imp=imp)
    compare(B, ref, x, B.FP4Q_IF4, B.FP4Q_SCALE_ABSMAX, 1, imp=imp)
    compare(B, ref, x, B.FP4Q_IF4, B.FP4Q_SCALE_SWEEP, 1, window=(-3, 7), imp=imp)
    compare(B, ref, x, B.FP4Q_MXFP4, B.FP4Q_SCALE_SWEEP, 1, window=(0, 1), imp=imp)
    compare(B, ref, x, B.FP4Q_MXFP4, B.FP4Q_SCALE_SWEEP, 1, window=(-1, 2), rotate=32, imp=imp)


def test_relaxed_infinite_reciprocal(B, ref):
    # given steps so small that D c is below 2^-128: r = fl(1/(D c)) is +inf,
    # so a zero element would give 0 * inf; its code must stay sign-only,
    # as for |x| / S_q = 0, and every nonzero element saturates
    rng = np.random.default_rng(95)
    x = rng.standard_normal((3, 128)).astype(np.float32)
    x[0, ::3] = 0.0
    x[1, 1::4] = -0.0
    x[2] *= np.float32(2.0 ** -140)
    for f, fo, blk in ((B.FP4Q_MXFP4, ref.MXFP4, 32), (B.FP4Q_NVFP4, ref.NVFP4, 16)):
        for group in (8, blk):
            coef = np.full((3, 128 // group), 0.25, np.float32)
            coef[:, ::2] = 1.0  # finite reciprocals beside infinite ones
            scales = np.full(3 * 128 // blk, 0 if f == B.FP4Q_MXFP4 else 1, np.uint8)
            S = 2.0 ** -117 if f == B.FP4Q_NVFP4 else None
            for xin in (x, synth.f32_to_bf16_bits(x)):
                codes, sc, _ = B.quantize_relaxed(to_dev(xin), to_dev(coef), group, format=f,
                                                  scales=to_dev(scales), global_scale=S)
                torch.cuda.synchronize()
                want = ref.quantize_relaxed(xin, coef, group, fmt=fo, global_scale=S, scales=scales)
                assert np.array_equal(codes.cpu().numpy(), want["codes"]), (f, group, xin.dtype)
