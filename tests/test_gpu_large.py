"""More than 2^31 elements: a bf16 tensor of (2^21 + 5) x 1024 values (4 GiB),
generated on the device, quantized whole, and checked on sampled rows on
both sides of element 2^31 and at the tail against the oracle (under the
global scale of the whole tensor, which is itself checked against the
oracle's rule applied to the exact tensor maximum)."""
import numpy as np
import pytest
import torch

from block_scaled_fp4_fp4q_amd import binding as B
from oracle import ref

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
ROWS, COLS = (1 << 21) + 5, 1024  # row 2^21 starts at element 2^31
SAMPLE_ROWS = [0, 1, (1 << 21) - 2, (1 << 21) - 1, 1 << 21, (1 << 21) + 1, ROWS - 1]


@pytest.fixture(scope="module")
def big():
    g = torch.Generator(device=DEV)
    g.manual_seed(31)
    x = torch.randn(ROWS, COLS, generator=g, device=DEV, dtype=torch.float32).to(torch.bfloat16)
    imp = np.random.default_rng(31).lognormal(0.0, 1.0, COLS).astype(np.float32)
    host_rows = x[SAMPLE_ROWS].cpu().view(torch.int16).numpy().view(np.uint16)
    gmax = float(x.abs().max().float().item())  # exact: a maximum of bf16 values
    yield x, imp, host_rows, gmax
    del x
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt,rule,obj", [(B.FP4Q_NVFP4, B.FP4Q_SCALE_SWEEP, B.FP4Q_OBJ_WMSE),
                                          (B.FP4Q_MXFP4, B.FP4Q_SCALE_ABSMAX, B.FP4Q_OBJ_MSE),
                                          (B.FP4Q_IF4, B.FP4Q_SCALE_ABSMAX, B.FP4Q_OBJ_MSE)])
def test_more_than_2_31_elements(big, fmt, rule, obj):
    x, imp, host_rows, gmax = big
    impd = torch.from_numpy(imp).to(DEV) if obj == B.FP4Q_OBJ_WMSE else None
    codes, scales, gs = B.quantize(x, format=fmt, scale_rule=rule, objective=obj, importance=impd)
    torch.cuda.synchronize()
    blk = 32 if fmt == B.FP4Q_MXFP4 else 16
    S = None
    if fmt != B.FP4Q_MXFP4:
        S = float(gs.item())
        assert np.float32(S) == np.float32(ref.lib().fp4q_ref_global_scale(np.float32(gmax)))
    want = ref.quantize(host_rows, fmt=fmt, rule=rule, objective=obj, global_scale=S,
                        importance=imp if obj == B.FP4Q_OBJ_WMSE else None)
    cpr, spr = COLS // 2, COLS // blk
    got_c = np.concatenate([codes[r * cpr:(r + 1) * cpr].cpu().numpy() for r in SAMPLE_ROWS])
    got_s = np.concatenate([scales[r * spr:(r + 1) * spr].cpu().numpy() for r in SAMPLE_ROWS])
    assert np.array_equal(got_s, want["scales"])
    assert np.array_equal(got_c, want["codes"])
    # the dequantized rows, past element 2^31 as well
    y = B.dequantize(codes, scales, gs, ROWS, COLS, format=fmt)
    torch.cuda.synchronize()
    got_y = y[SAMPLE_ROWS].cpu().numpy()
    yw = ref.dequantize(want["codes"], want["scales"], S,
                        len(SAMPLE_ROWS), COLS, fmt=fmt)
    assert np.array_equal(got_y.view(np.uint32), np.asarray(yw, np.float32).view(np.uint32))
    del codes, scales, y
