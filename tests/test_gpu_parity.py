"""GPU parity: the HIP library (through the C ABI) against the CPU oracle,
element by element, for every format / rule / objective / dtype / rotation,
at sizes that span many workgroups and end on a ragged tail, plus edge cases.

Bar: codes, scale bytes, IF4 indicators, the global scale and dequantized
values are bit-exact; the MSE/WMSE report agrees to 1e-10 relative (both
sides accumulate binary64, only the summation order differs)."""
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


def host_bf16_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


FMT = {"nvfp4": (0, 0), "mxfp4": (1, 1), "if4": (2, 2)}  # binding code, oracle code


def inputs(kind, rows, cols, seed):
    if kind == "bf16":
        x = synth.f32_to_bf16_bits((np.random.default_rng(seed).standard_t(4, (rows, cols)) * 0.02)
                                   .astype(np.float32))
    else:
        x = synth.c1(rows=rows, cols=cols, seed=seed)
    imp = np.random.default_rng(seed + 1).lognormal(0, 1, cols).astype(np.float32)
    return x, imp


def run_case(B, ref, fmt, rule, objective, rotate, x, imp, window=None, given=None):
    bfmt, ofmt = FMT[fmt]
    rows, cols = x.shape
    xd = to_dev(x)
    impd = to_dev(imp) if imp is not None else None
    codes, scales, gs = B.quantize(xd, format=bfmt, scale_rule=rule, objective=objective,
                                   window=window, rotate=rotate,
                                   importance=impd if objective == 1 else None,
                                   global_scale=given)
    torch.cuda.synchronize()
    want = ref.quantize(x, fmt=ofmt, rule=rule, objective=objective, window=window,
                        rotate=rotate, importance=imp if objective == 1 else None,
                        global_scale=given)
    got_scales = scales.cpu().numpy()
    got_codes = codes.cpu().numpy()
    if fmt != "mxfp4":
        assert gs.cpu().numpy()[0] == np.float32(want["S"])
    bad = np.nonzero(got_scales != want["scales"])[0]
    assert bad.size == 0, f"{bad.size} scale mismatches, first block {bad[:5]}"
    assert np.array_equal(got_codes, want["codes"])
    return xd, codes, scales, gs, want


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rotate", [0, 16])
@pytest.mark.parametrize("mode", ["absmax", "sweep_mse", "sweep_wmse"])
def test_nvfp4_parity(B, ref, dtype, rotate, mode):
    rule, obj = {"absmax": (0, 0), "sweep_mse": (1, 0), "sweep_wmse": (1, 1)}[mode]
    seed = 10 * ["absmax", "sweep_mse", "sweep_wmse"].index(mode) + rotate + (dtype == "bf16")
    x, imp = inputs(dtype, 37, 528, seed=seed)  # 1221 blocks: 5 workgroups, ragged tail
    run_case(B, ref, "nvfp4", rule, obj, rotate, x, imp)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rotate", [0, 16])
@pytest.mark.parametrize("objective", [0, 1])
def test_if4_parity(B, ref, dtype, rotate, objective):
    if dtype == "bf16":
        x = synth.c4(rows=41, cols=336, seed=rotate + objective)[0]
    else:
        x = synth.bf16_bits_to_f32(synth.c4(rows=41, cols=336, seed=5 + rotate)[0])
    imp = np.random.default_rng(3).lognormal(0, 1, 336).astype(np.float32)
    run_case(B, ref, "if4", 0, objective, rotate, x, imp)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rotate", [0, 32])
def test_mxfp4_parity(B, ref, dtype, rotate):
    x = synth.c3(rows=53, cols=352, seed=rotate + 1, n_outlier_channels=3)
    if dtype == "f32":
        x = synth.bf16_bits_to_f32(x)
    run_case(B, ref, "mxfp4", 0, 0, rotate, x, None)


@pytest.mark.parametrize("window", [(0, 0), (-126, 126), (-8, 7), (2, 5)])
def test_sweep_windows(B, ref, window):
    x, imp = inputs("bf16", 9, 256, seed=7)
    run_case(B, ref, "nvfp4", 1, 0, 0, x, imp, window=window)


@pytest.mark.parametrize("scale", [1e-15, 1e-19, 1e-21, 1e-24, 1e-30, 1e-36, 1e12, 1e30])
def test_sweep_extreme_magnitudes(B, ref, scale):
    # global scales whose squared steps fall below (or near the top of) the
    # binary32 range, and importance weights spread over ~17 decades
    rng = np.random.default_rng(int(-np.log10(scale)) + 100)
    x = (rng.standard_t(4, (13, 256)) * scale).astype(np.float32)
    imp = rng.lognormal(0, 4, 256).astype(np.float32)
    for obj, window in ((0, (-3, 7)), (1, (-8, 7)), (1, (-2, 9))):
        run_case(B, ref, "nvfp4", 1, obj, 0, x, imp, window=window)
    run_case(B, ref, "nvfp4", 1, 1, 16, synth.f32_to_bf16_bits(x), imp)


def test_sweep_near_float_max(B, ref):
    # max|x| = 3e38: the top patterns' reconstructions 6 D overflow to inf,
    # which the exact errors see and a binary32 estimate in step units does not
    rng = np.random.default_rng(7)
    x = rng.standard_t(4, (11, 128))
    x = (x / np.abs(x).max() * 3.0e38).astype(np.float32)
    imp = rng.lognormal(0, 1, 128).astype(np.float32)
    for obj, window in ((0, (-3, 7)), (1, (-8, 7))):
        run_case(B, ref, "nvfp4", 1, obj, 0, x, imp, window=window)


def test_given_global_scale(B, ref):
    x, imp = inputs("f32", 12, 256, seed=8)
    run_case(B, ref, "nvfp4", 1, 1, 0, x, imp, given=0.0625)
    run_case(B, ref, "if4", 0, 0, 16, x, imp, given=0.01)


def test_given_scale_extremes(B, ref):
    # the ends of the allowed global scale: at S = 2^-117 large elements give
    # y = |x| r = +inf (saturating codes, overflowing estimates, exact path),
    # at S = 2^119 small elements underflow to zero codes
    rng = np.random.default_rng(9)
    x = rng.standard_t(3, (7, 128)).astype(np.float32)
    x[0] *= np.float32(1e36)  # the 16-point Hadamard of the block stays finite
    x[1] *= np.float32(1e-30)
    x[2, :16] = 0.0
    x[3] = x[3] * np.float32(1e20) + np.float32(1.0)
    imp = rng.lognormal(0, 1, 128).astype(np.float32)
    for S in (2.0 ** -117, 2.0 ** 119):
        for fmt, rule, obj in (("nvfp4", 0, 0), ("nvfp4", 1, 0), ("nvfp4", 1, 1), ("if4", 0, 0),
                               ("if4", 0, 1), ("if4", 1, 0)):
            for rot in (0, 16):
                run_case(B, ref, fmt, rule, obj, rot, x, imp, given=S)
        run_case(B, ref, "nvfp4", 2, 1, 0, x, imp, given=S)


def test_edge_blocks(B, ref):
    # zeros, signed zeros, tiny blocks (subnormal and clamped E4M3 scales),
    # exact midpoints, one spike, and the block holding the maximum
    import exactspec  # noqa: F401  (tests/ is on sys.path)
    from test_oracle_spec import adversarial_nvfp4
    x = adversarial_nvfp4().reshape(-1, 64)
    for fmt, rule in [("nvfp4", 0), ("nvfp4", 1), ("if4", 0), ("mxfp4", 0)]:
        for rot in (0, 32 if fmt == "mxfp4" else 16):
            run_case(B, ref, fmt, rule, 0, rot, x, None)


def test_lane_split_bf16_edge_blocks(B, ref):
    # bf16 MXFP4 runs four lanes per block and bf16 IF4 (MSE) two: the DPP
    # maximum, Hadamard stages and ordered exact sums on the adversarial
    # blocks in bf16, and on a tensor of one block
    from test_oracle_spec import adversarial_nvfp4
    x = synth.f32_to_bf16_bits(adversarial_nvfp4().reshape(-1, 64))
    x1 = synth.f32_to_bf16_bits(np.linspace(-3, 5, 32, dtype=np.float32).reshape(1, 32))
    for rot in (0, 32):
        run_case(B, ref, "mxfp4", 0, 0, rot, x, None)
        run_case(B, ref, "mxfp4", 0, 0, rot, x1, None)
    for rot in (0, 16):
        run_case(B, ref, "if4", 0, 0, rot, x, None)
        run_case(B, ref, "if4", 0, 0, rot, x1[:, :16], None)


def test_empty_and_single_block(B, ref):
    x = np.zeros((0, 64), np.float32)
    codes, scales, gs = B.quantize(to_dev(x))
    torch.cuda.synchronize()
    assert codes.numel() == 0 and gs.cpu().item() == 1.0
    x1 = np.linspace(-3, 5, 16, dtype=np.float32).reshape(1, 16)
    run_case(B, ref, "nvfp4", 1, 0, 16, x1, None)
    x0 = np.zeros((3, 16), np.float32)
    _, _, _, gs, _ = run_case(B, ref, "nvfp4", 1, 0, 0, x0, None)
    assert gs.cpu().item() == 1.0


@pytest.mark.parametrize("fmt,rot", [("nvfp4", 0), ("nvfp4", 16), ("if4", 0), ("if4", 16),
                                     ("mxfp4", 0), ("mxfp4", 32)])
def test_dequantize_and_error_parity(B, ref, fmt, rot):
    bfmt, ofmt = FMT[fmt]
    if fmt == "mxfp4":
        x = synth.c3(rows=19, cols=320, seed=2, n_outlier_channels=2)
    elif fmt == "if4":
        x = synth.c4(rows=19, cols=320, seed=2)[0]
    else:
        x = synth.c2(rows=19, cols=320, seed=2)[0]
    imp = np.random.default_rng(1).lognormal(0, 1, 320).astype(np.float32)
    xd, codes, scales, gs, want = run_case(B, ref, fmt, 0, 0, rot, x, None)
    rows, cols = x.shape
    S = None if fmt == "mxfp4" else want["S"]
    for dt, odt in [(torch.float32, 0), (torch.bfloat16, 1)]:
        y = B.dequantize(codes, scales, gs, rows, cols, format=bfmt, unrotate=rot, dtype=dt)
        torch.cuda.synchronize()
        yw = ref.dequantize(want["codes"], want["scales"], S, rows, cols, fmt=ofmt,
                            unrotate=rot, out_dtype=odt)
        if dt == torch.float32:
            assert np.array_equal(y.cpu().numpy().view(np.uint32), yw.view(np.uint32))
        else:
            assert np.array_equal(host_bf16_bits(y), yw)
    got = B.error(xd, codes, scales, gs, format=bfmt, rotate=rot, importance=to_dev(imp))
    exp = ref.error(x, want["codes"], want["scales"], S, fmt=ofmt, rotate=rot, importance=imp)
    assert abs(got[0] - exp[0]) <= 1e-10 * exp[0]
    assert abs(got[1] - exp[1]) <= 1e-10 * exp[1]
    got = B.error(xd, codes, scales, gs, format=bfmt, rotate=rot)
    assert np.isnan(got[1])


def test_deterministic(B):
    x, imp = inputs("bf16", 64, 1024, seed=3)
    xd, impd = to_dev(x), to_dev(imp)
    a = B.quantize(xd, scale_rule=1, objective=1, importance=impd)
    b = B.quantize(xd, scale_rule=1, objective=1, importance=impd)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_graph_capture_replays(B, ref):
    # quantize (partial maxima + sweep) and dequantize launch kernels only, so
    # they can be captured; each replay, with eager work and synchronizations
    # in between, must reproduce the eager results
    x, imp = inputs("bf16", 64, 512, seed=77)
    xd, impd = to_dev(x), to_dev(imp)
    spec = B.make_spec(B.FP4Q_NVFP4, B.FP4Q_SCALE_SWEEP, B.FP4Q_OBJ_WMSE, (-8, 7))
    dspec = B.make_spec(B.FP4Q_NVFP4)
    ws = B.alloc_workspace(spec, *x.shape, DEV)
    n = x.size

    def outputs():
        return (torch.empty(n // 2, dtype=torch.uint8, device=DEV),
                torch.empty(n // 16, dtype=torch.uint8, device=DEV),
                torch.empty(1, dtype=torch.float32, device=DEV),
                torch.empty(x.shape, dtype=torch.bfloat16, device=DEV))

    ce, se, ge, ye = outputs()
    B.fp4q_quantize(spec, xd, impd, ce, se, ge, ws)
    B.fp4q_dequantize(dspec, ce, se, ge, *x.shape, 0, ye)
    torch.cuda.synchronize()

    c, s, g, y = outputs()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                   # warm-up outside the capture
        B.fp4q_quantize(spec, xd, impd, c, s, g, ws)
        B.fp4q_dequantize(dspec, c, s, g, *x.shape, 0, y)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        B.fp4q_quantize(spec, xd, impd, c, s, g, ws)
        B.fp4q_dequantize(dspec, c, s, g, *x.shape, 0, y)
    for _ in range(3):
        for t in (c, s, g, y):
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(c, ce) and torch.equal(s, se) and torch.equal(g, ge)
        assert torch.equal(y.view(torch.int16), ye.view(torch.int16))


def test_base_scale_rounding_boundaries(B, ref):
    # Block maxima placed so that t = a / fl(6 S) falls on every E4M3 midpoint
    # (ties go to the even pattern) and one binary32 step to either side, in
    # the subnormal range and at the saturation boundary; MXFP4 maxima at and
    # just below every power of two the OCP exponent can see.  S = 2^-10 makes
    # fl(6 S) = 6 2^-10 and t = m exactly for a = 6 2^-10 m.
    vals = [ref.lib().fp4q_ref_e4m3_value(b) for b in range(0x7F)]
    ts = []
    for lo, hi in zip(vals[:-1], vals[1:]):
        mid = np.float32((np.float64(lo) + np.float64(hi)) / 2)
        ts += [mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(1e9))]
    ts += [np.float32(448.0), np.float32(464.0), np.float32(480.0), np.float32(1e6),
           np.float32(2.0 ** -10), np.float32(2.0 ** -11)]
    S = np.float32(2.0 ** -10)
    a = np.array(ts, np.float64) * 6.0 * float(S)
    rng = np.random.default_rng(21)
    x = (rng.uniform(-1, 1, (len(a), 16)) * a[:, None]).astype(np.float32)
    x[np.arange(len(a)), rng.integers(0, 16, len(a))] = a.astype(np.float32)  # the block maximum
    assert np.all(np.abs(x).max(axis=1) == a.astype(np.float32))
    for fmt, rule in (("nvfp4", 0), ("nvfp4", 1), ("if4", 0)):
        run_case(B, ref, fmt, rule, 0, 0, x, None, given=float(S))
    # MXFP4: maxima 2^k and the float just below, k over the whole exponent range
    ks = np.arange(-140, 128)
    m = np.concatenate([np.ldexp(np.float32(1.0), ks).astype(np.float32),
                        np.nextafter(np.ldexp(np.float32(1.0), ks).astype(np.float32), np.float32(0))])
    m = m[np.isfinite(m) & (m > 0)]
    xm = (rng.uniform(-1, 1, (len(m), 32)) * m[:, None].astype(np.float64)).astype(np.float32)
    xm[np.arange(len(m)), rng.integers(0, 32, len(m))] = m
    for rule in (0, 1):
        run_case(B, ref, "mxfp4", rule, 0, 0, xm, None)


def test_concurrent_streams(B, ref):
    # two calls in flight at once on two streams, each with its own workspace
    # (the header's condition for concurrency), repeated; every result must
    # equal the same call run alone
    x1, imp1 = inputs("bf16", 96, 1024, seed=81)
    x2, _ = inputs("bf16", 64, 768, seed=82)
    cases = [(B.make_spec(B.FP4Q_NVFP4, B.FP4Q_SCALE_SWEEP, B.FP4Q_OBJ_WMSE, (-8, 7)), to_dev(x1), to_dev(imp1)),
             (B.make_spec(B.FP4Q_IF4, B.FP4Q_SCALE_SWEEP, B.FP4Q_OBJ_MSE, (-3, 7)), to_dev(x2), None)]

    def outputs(spec, xd):
        n = xd.numel()
        return (torch.empty(n // 2, dtype=torch.uint8, device=DEV),
                torch.empty(n // spec.block, dtype=torch.uint8, device=DEV),
                torch.empty(1, dtype=torch.float32, device=DEV))

    want = []
    for spec, xd, impd in cases:
        ws = B.alloc_workspace(spec, *xd.shape, DEV)
        o = outputs(spec, xd)
        B.fp4q_quantize(spec, xd, impd, *o, ws)
        want.append(o)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    wss = [B.alloc_workspace(spec, *xd.shape, DEV) for spec, xd, _ in cases]
    outs = [[outputs(spec, xd) for _ in range(4)] for spec, xd, _ in cases]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    for rep in range(4):
        for i, (spec, xd, impd) in enumerate(cases):
            B.fp4q_quantize(spec, xd, impd, *outs[i][rep], wss[i], stream=streams[i])
    torch.cuda.synchronize()
    for i in range(2):
        for rep in range(4):
            for got, exp in zip(outs[i][rep], want[i]):
                assert torch.equal(got, exp), (i, rep)
