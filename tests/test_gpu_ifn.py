"""GPU parity of IF3 and IF6 (the adaptive FP-or-INT type at 3 and 6 bits)
against the CPU oracle, through the C ABI.

Source: Adaptive Block-Scaled Data Types, Methodology (the IF4 pick applies
to 3- and 6-bit formats); the grids are the reading stated in include/fp4q.h
(E2M0 / E2M3 against INT3 / INT6 on the step D*fl32(FPmax/INTmax)).

Bar: codes, scale bytes (indicator included), the global scale and
dequantized values bit-exact; the MSE/WMSE report within 1e-10 relative."""
import numpy as np
import pytest
import torch

from block_scaled_fp4_fp4q_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
FMTS = {"if3": (3, 3), "if6": (4, 4)}  # binding code, oracle code


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


def mixed(rows, cols, seed, dtype):
    """half uniform blocks (INT-friendly), half spiky Laplace blocks
    (FP-friendly), as the IF4 workload"""
    x = synth.c4(rows=rows, cols=cols, seed=seed)[0]
    return x if dtype == "bf16" else synth.bf16_bits_to_f32(x) * np.float32(1.0 + 1e-3)


def run(B, ref, fmt, x, rule=0, objective=0, rotate=0, window=None, imp=None, given=None):
    bfmt, ofmt = FMTS[fmt]
    xd = to_dev(x)
    impd = to_dev(imp) if imp is not None else None
    codes, scales, gs = B.quantize(xd, format=bfmt, scale_rule=rule, objective=objective,
                                   window=window, rotate=rotate, importance=impd,
                                   global_scale=given)
    torch.cuda.synchronize()
    want = ref.quantize(x, fmt=ofmt, rule=rule, objective=objective, window=window,
                        rotate=rotate, importance=imp, global_scale=given)
    assert gs.cpu().numpy()[0] == np.float32(want["S"])
    got_s = scales.cpu().numpy()
    bad = np.nonzero(got_s != want["scales"])[0]
    assert bad.size == 0, f"{bad.size} scale mismatches, first blocks {bad[:5]}"
    assert np.array_equal(codes.cpu().numpy(), want["codes"])
    return xd, codes, scales, gs, want


@pytest.mark.parametrize("fmt", ["if3", "if6"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rotate", [0, 16])
@pytest.mark.parametrize("mode", ["absmax_mse", "absmax_wmse", "sweep_mse", "sweep_wmse"])
def test_parity(B, ref, fmt, dtype, rotate, mode):
    rule = 1 if mode.startswith("sweep") else 0
    obj = 1 if mode.endswith("wmse") else 0
    seed = 3 * rotate + len(mode) + (dtype == "bf16") + 7 * (fmt == "if6")
    x = mixed(43, 352, seed, dtype)           # 946 blocks: several workgroups, ragged tail
    imp = np.random.default_rng(seed).lognormal(0, 1, 352).astype(np.float32) if obj else None
    xd, codes, scales, gs, want = run(B, ref, fmt, x, rule, obj, rotate, (-3, 7) if rule else None,
                                      imp)
    ind = (scales.cpu().numpy() & 0x80) != 0
    assert 0 < ind.mean() < 1, "both grids should win some blocks of this mix"


@pytest.mark.parametrize("fmt", ["if3", "if6"])
@pytest.mark.parametrize("rotate", [0, 16])
def test_dequantize_and_error(B, ref, fmt, rotate):
    bfmt, ofmt = FMTS[fmt]
    x = mixed(29, 256, 11 + rotate, "bf16")
    imp = np.random.default_rng(2).lognormal(0, 1, 256).astype(np.float32)
    xd, codes, scales, gs, want = run(B, ref, fmt, x, rotate=rotate)
    rows, cols = x.shape
    S = float(gs.item())
    for dt, odt in ((torch.float32, ref.F32), (torch.bfloat16, ref.BF16)):
        y = B.dequantize(codes, scales, gs, rows, cols, format=bfmt, unrotate=rotate, dtype=dt)
        yw = ref.dequantize(want["codes"], want["scales"], S, rows, cols, fmt=ofmt, unrotate=rotate,
                            out_dtype=odt)
        yg = y.cpu().numpy().view(np.uint32) if dt == torch.float32 else \
            y.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(yg, yw.view(np.uint32) if dt == torch.float32 else yw)
    mse, wmse = B.error(xd, codes, scales, gs, format=bfmt, rotate=rotate, importance=to_dev(imp))
    e = ref.error(x, want["codes"], want["scales"], S, fmt=ofmt, rotate=rotate, importance=imp)
    assert abs(mse - e[0]) <= 1e-10 * e[0] and abs(wmse - e[1]) <= 1e-10 * e[1]


@pytest.mark.parametrize("fmt", ["if3", "if6"])
def test_many_grid_stride_passes(B, ref, fmt):
    # 8192 x 1024: 524288 blocks, more than one round of resident lanes
    x = mixed(8192, 1024, 41, "bf16")
    run(B, ref, fmt, x)


@pytest.mark.parametrize("fmt", ["if3", "if6"])
def test_edge_cases(B, ref, fmt):
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((12, 64)) * 2).astype(np.float32)
    x[0] = 0.0                        # all-zero blocks
    x[1, :16] = -0.0                  # signed zeros only
    x[2, :16] = np.float32(1e-30)     # a tiny constant block (exact ties between grids)
    x[3, :16] = 1e3                   # constant block at the top
    x[4, 16:32] = np.linspace(-7.5, 7.5, 16, dtype=np.float32)
    run(B, ref, fmt, x)
    for S in (2.0 ** -117, 2.0 ** 119, 1.0 / 3.0):   # the ends of the allowed global scale
        run(B, ref, fmt, x, given=S)
    run(B, ref, fmt, x, rule=1, window=(-126, 126))  # window past both ends of E4M3


def test_grid_midpoints(B, ref):
    # elements exactly on the FP and INT midpoints of the base step (S given
    # as 1, block maximum on the FP maximum so the base scale is 1.0)
    L = ref.lib()
    for fmt, n in (("if3", 3), ("if6", 6)):
        vals = [L.fp4q_ref_fpn_value(n, m) for m in range(1 << (n - 1))]
        mids = [(a + b) / 2 for a, b in zip(vals, vals[1:])]
        top = (1 << (n - 1)) - 1
        step = float(np.float32(vals[-1]) / np.float32(top))
        imids = [np.float32((k + 0.5) * step) for k in range(top)]
        pts = np.array(mids + [float(v) for v in imids], np.float32)
        pts = np.concatenate([pts, np.nextafter(pts, np.float32(0)), np.nextafter(pts, np.float32(9))])
        nb = -(-pts.size // 15)
        blocks = np.zeros((nb, 16), np.float32)
        blocks[:, 0] = vals[-1]                          # block maximum: base scale 1.0
        blocks[:, 1:] = np.resize(pts, nb * 15).reshape(nb, 15)
        run(B, ref, fmt, blocks, given=1.0)


def test_empty_tensor(B):
    for fmt in ("if3", "if6"):
        codes, scales, gs = B.quantize(torch.empty(0, 64, device=DEV), format=FMTS[fmt][0])
        torch.cuda.synchronize()
        assert codes.numel() == 0 and scales.numel() == 0 and gs.item() == 1.0


@pytest.mark.timeout(900)
@pytest.mark.parametrize("fmt", ["if3", "if6"])
def test_full_if4_workload(B, ref, fmt):
    # the 8192 x 8192 IF4 workload (half uniform, half spiky-Laplace blocks),
    # every block compared
    x, uniform = synth.c4()
    xd, codes, scales, gs, want = run(B, ref, fmt, x)
    ind = (scales.cpu().numpy() & 0x80) != 0
    print(f"{fmt}: INT share uniform {ind[uniform].mean():.3f}, spiky {ind[~uniform].mean():.3f}")


@pytest.mark.parametrize("fmt", ["if3", "if6"])
def test_int_step_below_2_pow_128(B, ref, fmt):
    # under the smallest global scale, blocks whose maximum is about 2^-123
    # land on pattern 0x01 (D = 2^-126); IF6's INT step is then below 2^-128,
    # its reciprocal +inf, and zero elements must still get q = 0 (the
    # kernels' estimates turn NaN or infinite there and the exact search
    # decides).  Zeros, signed zeros and values across the low patterns.
    rng = np.random.default_rng(77)
    x = (rng.uniform(-1, 1, (8, 64)) * 2.0 ** -123).astype(np.float32)
    x[:, ::5] = 0.0
    x[:, 1::7] = -0.0
    x[3] *= np.float32(64.0)                 # a few patterns higher
    for window in (None, (-3, 7), (-126, 126)):
        run(B, ref, fmt, x, rule=0 if window is None else 1, window=window, given=2.0 ** -117)
