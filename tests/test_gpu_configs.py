"""Full-size parity on the five workloads, through the C ABI.

Every workload is compared with the oracle on every block: codes, scale
bytes and the global scale byte for byte, dequantized values bit for bit.
The 2 GiB KV tensor is re-quantized by the oracle over row chunks (host
memory stays bounded) under the GPU's global scale, which is itself checked
against the oracle's rule applied to the exact maximum of the rotated
tensor.  The reported MSE/WMSE must agree with the oracle's error of its own
quantization to 1e-9 relative (binary64 sums in different orders)."""
import os

import numpy as np
import pytest
import torch

from block_scaled_fp4_fp4q_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
THREADS = min(16, len(os.sched_getaffinity(0)))


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_scaled_fp4_fp4q_amd import binding
    binding.lib()
    return binding


def to_dev(x):
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(x).to(DEV)


def near_ties(best, second):
    live = best > 0
    gap = np.where(live, (second - best) / np.where(live, best, 1.0), np.inf)
    return int(np.sum(gap < 1e-6))


def compare_rows(ref, x, rows, got_codes, got_scales, S, B_, **kw):
    """Oracle re-quantization of `rows` under global scale S vs the GPU."""
    cols = x.shape[1]
    xs = np.ascontiguousarray(x[rows])
    want = ref.quantize(xs, global_scale=S, nthreads=THREADS, errors=True, **kw)
    nb_row = cols // B_
    gs = got_scales.reshape(-1, nb_row)[rows].reshape(-1)
    gc = got_codes.reshape(-1, cols // 2)[rows].reshape(-1)
    bad = np.nonzero(gs != want["scales"])[0]
    assert bad.size == 0, f"{bad.size} scale mismatches, first {bad[:5]}"
    assert np.array_equal(gc, want["codes"])
    return want


def test_c1_full(B, ref):
    x = synth.c1()
    xd = to_dev(x)
    for rule in (0, 1):
        codes, scales, gs = B.quantize(xd, scale_rule=rule)
        want = ref.quantize(x, rule=rule, nthreads=THREADS, errors=True)
        assert gs.item() == np.float32(want["S"])
        assert np.array_equal(scales.cpu().numpy(), want["scales"])
        assert np.array_equal(codes.cpu().numpy(), want["codes"])
        mse = B.error(xd, codes, scales, gs)[0]
        assert abs(mse - ref.error(x, want["codes"], want["scales"], want["S"])[0]) <= 1e-9 * mse
        print(f"c1 rule={rule}: near-tie blocks {near_ties(want['best'], want['second'])}")


@pytest.fixture(scope="module")
def c2data():
    return synth.c2()


def test_c2_sweep_wmse(B, ref, c2data):
    x, imp = c2data
    xd, impd = to_dev(x), to_dev(imp)
    codes, scales, gs = B.quantize(xd, scale_rule=1, objective=1, window=(-8, 7), importance=impd)
    torch.cuda.synchronize()
    S = gs.item()
    G = np.abs(synth.bf16_bits_to_f32(x)).max()
    assert S == ref.lib().fp4q_ref_global_scale(G)
    rows = synth.rows_sample(x, 1024, seed=2)
    want = compare_rows(ref, x, rows, codes.cpu().numpy(), scales.cpu().numpy(), S, 16,
                        rule=ref.SWEEP, objective=ref.WMSE, importance=imp)
    print(f"c2: sampled {len(rows)} rows, near-tie blocks {near_ties(want['best'], want['second'])}")
    mse, wmse = B.error(xd, codes, scales, gs, importance=impd)
    # oracle on the full tensor: its own quantization must give the same MSE
    full = ref.quantize(x, rule=ref.SWEEP, objective=ref.WMSE, importance=imp, nthreads=THREADS)
    assert np.array_equal(full["scales"], scales.cpu().numpy())
    assert np.array_equal(full["codes"], codes.cpu().numpy())
    e = ref.error(x, full["codes"], full["scales"], full["S"], importance=imp, nthreads=THREADS)
    assert abs(mse - e[0]) <= 1e-9 * e[0] and abs(wmse - e[1]) <= 1e-9 * e[1]


def test_c2_absmax_and_dequant(B, ref, c2data):
    x, imp = c2data
    xd = to_dev(x)
    codes, scales, gs = B.quantize(xd)
    full = ref.quantize(x, nthreads=THREADS)
    assert np.array_equal(full["scales"], scales.cpu().numpy())
    assert np.array_equal(full["codes"], codes.cpu().numpy())
    y = B.dequantize(codes, scales, gs, *x.shape, dtype=torch.bfloat16)
    yw = ref.dequantize(full["codes"], full["scales"], full["S"], *x.shape, out_dtype=ref.BF16,
                        nthreads=THREADS)
    yg = y.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(yg, yw)


@pytest.mark.parametrize("rotate", [0, 32])
def test_c3_mxfp4(B, ref, rotate):
    x = synth.c3()
    xd = to_dev(x)
    codes, scales, _ = B.quantize(xd, format=B.FP4Q_MXFP4, rotate=rotate)
    want = ref.quantize(x, fmt=ref.MXFP4, rotate=rotate, nthreads=THREADS)
    assert np.array_equal(scales.cpu().numpy(), want["scales"])
    assert np.array_equal(codes.cpu().numpy(), want["codes"])
    mse = B.error(xd, codes, scales, None, format=B.FP4Q_MXFP4, rotate=rotate)[0]
    e = ref.error(x, want["codes"], want["scales"], None, fmt=ref.MXFP4, rotate=rotate, nthreads=THREADS)[0]
    assert abs(mse - e) <= 1e-9 * e
    print(f"c3 rotate={rotate}: MSE {mse:.6g}")


def test_c4_if4(B, ref):
    x, uniform = synth.c4()
    xd = to_dev(x)
    codes, scales, gs = B.quantize(xd, format=B.FP4Q_IF4)
    want = ref.quantize(x, fmt=ref.IF4, nthreads=THREADS)
    assert gs.item() == np.float32(want["S"])
    s = scales.cpu().numpy()
    assert np.array_equal(s, want["scales"])
    assert np.array_equal(codes.cpu().numpy(), want["codes"])
    ind = (s & 0x80) != 0
    print(f"c4: INT4 share uniform {ind[uniform].mean():.3f}, spiky {ind[~uniform].mean():.3f}")
    y = B.dequantize(codes, scales, gs, *x.shape, format=B.FP4Q_IF4)
    yw = ref.dequantize(want["codes"], want["scales"], want["S"], *x.shape, fmt=ref.IF4,
                        nthreads=THREADS)
    assert np.array_equal(y.cpu().numpy().view(np.uint32), yw.view(np.uint32))


@pytest.mark.timeout(1200)
def test_c5_kv_sweep_hadamard(B, ref, capsys):
    """Every code and scale byte of the 2 GiB KV tensor (67,108,864 blocks)
    against the oracle, which runs over row chunks so that host memory stays
    bounded; the MSE against the oracle's error of its own quantization."""
    x = synth.c5()
    rows, cols = x.shape
    xd = to_dev(x)
    codes, scales, gs = B.quantize(xd, scale_rule=1, objective=0, window=(-3, 7), rotate=16)
    torch.cuda.synchronize()
    S = gs.item()
    gc, gsc = codes.cpu().numpy(), scales.cpu().numpy()
    mse = B.error(xd, codes, scales, gs, rotate=16)[0]
    del codes, scales
    # dequantize round trip (un-rotated, bf16) of the whole tensor, kept on the host
    y = B.dequantize(*B.quantize(xd, scale_rule=1, objective=0, window=(-3, 7), rotate=16),
                     rows, cols, unrotate=16, dtype=torch.bfloat16)
    yg = y.view(torch.int16).cpu().numpy().view(np.uint16)
    del y, xd
    torch.cuda.empty_cache()
    chunk = 1 << 20
    G = np.float32(0.0)
    sq = 0.0
    ties = 0
    for r0 in range(0, rows, chunk):
        r1 = min(rows, r0 + chunk)
        xs = np.ascontiguousarray(x[r0:r1])
        G = max(G, np.float32(np.abs(ref.prepare(xs, rotate=16, nthreads=THREADS)).max()))
        want = ref.quantize(xs, rule=ref.SWEEP, objective=ref.MSE, window=(-3, 7), rotate=16,
                            global_scale=S, nthreads=THREADS, errors=True)
        b0, b1 = r0 * cols // 16, r1 * cols // 16
        bad = np.nonzero(gsc[b0:b1] != want["scales"])[0]
        assert bad.size == 0, f"rows {r0}..{r1}: {bad.size} scale mismatches, first {bad[:5] + b0}"
        assert np.array_equal(gc[b0 * 8:b1 * 8], want["codes"]), f"rows {r0}..{r1}: codes differ"
        yw = ref.dequantize(want["codes"], want["scales"], S, r1 - r0, cols, unrotate=16,
                            out_dtype=ref.BF16, nthreads=THREADS)
        assert np.array_equal(yg[r0:r1], yw), f"rows {r0}..{r1}: dequantized values differ"
        e = ref.error(xs, want["codes"], want["scales"], S, rotate=16, nthreads=THREADS)[0]
        sq += e * (r1 - r0) * cols
        ties += near_ties(want["best"], want["second"])
        with capsys.disabled():
            print(f"[c5 full parity] rows {r0}..{r1} of {rows}: bit-exact", flush=True)
    assert S == ref.lib().fp4q_ref_global_scale(G)
    e_full = sq / (rows * cols)
    assert abs(mse - e_full) <= 1e-9 * e_full
    print(f"c5: all {rows * cols // 16} blocks bit-exact, oracle near-tie blocks {ties}, "
          f"MSE {mse:.6g}")


# ---------------------------------------------------------------------------
# the extension rules at full size
# ---------------------------------------------------------------------------

def test_c2_four_over_six_wmse(B, ref, c2data):
    x, imp = c2data
    xd, impd = to_dev(x), to_dev(imp)
    codes, scales, gs = B.quantize(xd, scale_rule=B.FP4Q_SCALE_FOUR_OVER_SIX, objective=1,
                                   importance=impd)
    full = ref.quantize(x, rule=ref.FOUR_SIX, objective=ref.WMSE, importance=imp,
                        nthreads=THREADS)
    assert gs.item() == np.float32(full["S"])
    assert np.array_equal(full["scales"], scales.cpu().numpy())
    assert np.array_equal(full["codes"], codes.cpu().numpy())
    wm = B.error(xd, codes, scales, gs, importance=impd)[1]
    base = B.quantize(xd)
    wb = B.error(xd, *base, importance=impd)[1]
    print(f"c2 4/6: WMSE {wm:.6g} vs AbsMax {wb:.6g}")
    assert wm < wb


@pytest.mark.parametrize("rotate", [0, 32])
def test_c3_mxfp4_exponent_window(B, ref, rotate):
    x = synth.c3()
    xd = to_dev(x)
    codes, scales, _ = B.quantize(xd, format=B.FP4Q_MXFP4, scale_rule=B.FP4Q_SCALE_SWEEP,
                                  rotate=rotate)
    want = ref.quantize(x, fmt=ref.MXFP4, rule=ref.SWEEP, window=(0, 1), rotate=rotate,
                        nthreads=THREADS)
    assert np.array_equal(scales.cpu().numpy(), want["scales"])
    assert np.array_equal(codes.cpu().numpy(), want["codes"])
    mse = B.error(xd, codes, scales, None, format=B.FP4Q_MXFP4, rotate=rotate)[0]
    base = B.quantize(xd, format=B.FP4Q_MXFP4, rotate=rotate)
    mb = B.error(xd, *base, format=B.FP4Q_MXFP4, rotate=rotate)[0]
    print(f"c3 rotate={rotate} window [0,1]: MSE {mse:.6g} vs OCP {mb:.6g}")
    assert mse <= mb


def test_c4_if4_sweep(B, ref):
    x, _ = synth.c4()
    xd = to_dev(x)
    codes, scales, gs = B.quantize(xd, format=B.FP4Q_IF4, scale_rule=B.FP4Q_SCALE_SWEEP,
                                   window=(-3, 7))
    want = ref.quantize(x, fmt=ref.IF4, rule=ref.SWEEP, window=(-3, 7), nthreads=THREADS)
    assert gs.item() == np.float32(want["S"])
    assert np.array_equal(scales.cpu().numpy(), want["scales"])
    assert np.array_equal(codes.cpu().numpy(), want["codes"])
    mse = B.error(xd, codes, scales, gs, format=B.FP4Q_IF4)[0]
    base = B.quantize(xd, format=B.FP4Q_IF4)
    mb = B.error(xd, *base, format=B.FP4Q_IF4)[0]
    print(f"c4 IF4 + sweep [-3,7]: MSE {mse:.6g} vs IF4 {mb:.6g}")
    assert mse <= mb


@pytest.mark.parametrize("rotate", [0, 32])
def test_mxfp4_exponent_window_wmse_multi_pass(B, ref, rotate):
    # 8189 rows: 1048192 blocks, several grid-stride passes per lane (the next
    # block is loaded one pass ahead) and a last pass that is only partly full
    x = synth.c3()[:8189]
    imp = np.random.default_rng(13).lognormal(0.0, 1.0, x.shape[1]).astype(np.float32)
    codes, scales, _ = B.quantize(to_dev(x), format=B.FP4Q_MXFP4, scale_rule=B.FP4Q_SCALE_SWEEP,
                                  objective=1, importance=to_dev(imp), rotate=rotate)
    want = ref.quantize(x, fmt=ref.MXFP4, rule=ref.SWEEP, objective=ref.WMSE, importance=imp,
                        window=(0, 1), rotate=rotate, nthreads=THREADS)
    assert np.array_equal(scales.cpu().numpy(), want["scales"])
    assert np.array_equal(codes.cpu().numpy(), want["codes"])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_four_over_six_mse_multi_pass(B, ref, c2data, dtype):
    # 7001 rows of the c2 weight: 1792256 blocks, several passes per lane and
    # a partly full last one
    x = c2data[0][:7001]
    if dtype == "f32":
        x = synth.bf16_bits_to_f32(x)
    codes, scales, gs = B.quantize(to_dev(x), scale_rule=B.FP4Q_SCALE_FOUR_OVER_SIX)
    want = ref.quantize(x, rule=ref.FOUR_SIX, nthreads=THREADS)
    assert gs.item() == np.float32(want["S"])
    assert np.array_equal(scales.cpu().numpy(), want["scales"])
    assert np.array_equal(codes.cpu().numpy(), want["codes"])


@pytest.mark.parametrize("fmt,group", [("nvfp4", 8), ("mxfp4", 8)])
def test_relaxed_full(B, ref, c2data, fmt, group):
    x = c2data[0] if fmt == "nvfp4" else synth.c3()
    f = B.FP4Q_MXFP4 if fmt == "mxfp4" else B.FP4Q_NVFP4
    rows, cols = x.shape
    c = np.random.default_rng(12).lognormal(0.0, 0.08, (rows, cols // group)).astype(np.float32)
    codes, scales, gs = B.quantize_relaxed(to_dev(x), to_dev(c), group, format=f)
    want = ref.quantize_relaxed(x, c, group, fmt=ref.MXFP4 if fmt == "mxfp4" else ref.NVFP4,
                                nthreads=THREADS)
    if fmt == "nvfp4":
        assert gs.item() == np.float32(want["S"])
    assert np.array_equal(scales.cpu().numpy(), want["scales"])
    assert np.array_equal(codes.cpu().numpy(), want["codes"])


def test_sweep_queue_drains(B, ref):
    # a constant tensor: patterns 0x78 and 0x7C both reconstruct 1.0 exactly, so
    # every block is an exact tie that only the binary64 path may decide; at
    # 2^20 blocks every workgroup fills and drains its fallback queue several
    # times in mid-loop, with half the rows random so both paths interleave
    rows, cols = 4096, 4096
    x = np.ones((rows, cols), np.float32)
    rng = np.random.default_rng(21)
    # random rows within [-1, 1], so that S stays 1/1536 and the ties stay ties
    x[1::2] = np.clip(rng.standard_normal((rows // 2, cols)) * 0.25, -1, 1).astype(np.float32)
    imp = rng.lognormal(0, 1, cols).astype(np.float32)
    xd, impd = to_dev(x), to_dev(imp)
    for obj, window in ((1, (-8, 7)), (0, (-3, 7))):
        codes, scales, gs = B.quantize(xd, scale_rule=1, objective=obj, window=window,
                                       importance=impd if obj else None)
        want = ref.quantize(x, rule=ref.SWEEP, objective=obj, window=window,
                            importance=imp if obj else None, nthreads=THREADS)
        assert gs.item() == np.float32(want["S"])
        assert np.array_equal(scales.cpu().numpy(), want["scales"])
        assert np.array_equal(codes.cpu().numpy(), want["codes"])
