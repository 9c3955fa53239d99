"""Host-side argument checks of the Python binding (no GPU).

The C ABI receives bare pointers, so the binding is the only place where a
host tensor, a wrong dtype or a short buffer can be refused before a kernel
would read or write out of bounds.  These tests build CPU tensors and call
the binding's check functions: with the device check on, a host tensor is
refused; with it off (as only these tests do), every size, dtype and
contiguity check is exercised on its own.  Nothing here launches a kernel."""
import pytest
import torch

from block_scaled_fp4_fp4q_amd import binding as B

ROWS, COLS = 8, 64


def nv_args(objective=B.FP4Q_OBJ_MSE, rule=B.FP4Q_SCALE_SWEEP, fmt=B.FP4Q_NVFP4):
    spec = B.make_spec(fmt, rule, objective)
    n = ROWS * COLS
    return dict(spec=spec, x=torch.zeros(ROWS, COLS, dtype=torch.bfloat16),
                importance=torch.ones(COLS, dtype=torch.float32),
                codes=torch.empty(n // 2, dtype=torch.uint8),
                scales=torch.empty(n // spec.block, dtype=torch.uint8),
                global_scale=torch.empty(1, dtype=torch.float32),
                workspace=torch.empty(B.fp4q_workspace_bytes(spec, ROWS, COLS), dtype=torch.uint8))


def check(**kw):
    return B.check_quantize_args(require_cuda=False, **kw)


def test_valid_arguments_pass():
    x2 = check(**nv_args())
    assert tuple(x2.shape) == (ROWS, COLS)


def test_host_tensor_refused_before_any_call():
    a = nv_args()
    with pytest.raises(ValueError, match="ROCm device"):
        B.check_quantize_args(**a)
    # the public entry point refuses it as well, before reaching the library
    with pytest.raises(ValueError, match="ROCm device"):
        B.fp4q_quantize(a["spec"], a["x"], a["importance"], a["codes"], a["scales"],
                        a["global_scale"], a["workspace"])


@pytest.mark.parametrize("name,bad,msg", [
    ("codes", torch.empty(ROWS * COLS // 2 - 1, dtype=torch.uint8), "at least"),
    ("codes", torch.empty(ROWS * COLS // 2, dtype=torch.int8), "dtype"),
    ("scales", torch.empty(ROWS * COLS // 16 - 1, dtype=torch.uint8), "at least"),
    ("global_scale", torch.empty(0, dtype=torch.float32), "at least"),
    ("global_scale", torch.empty(1, dtype=torch.float64), "dtype"),
    ("global_scale", None, "required"),
    ("workspace", torch.empty(255, dtype=torch.uint8), "at least"),
    ("importance", torch.ones(COLS - 1, dtype=torch.float32), "at least"),
    ("importance", torch.ones(COLS, dtype=torch.float16), "dtype"),
    ("codes", torch.empty(ROWS * COLS, dtype=torch.uint8)[::2], "contiguous"),
    ("x", torch.zeros(ROWS, COLS, dtype=torch.float16), "dtype"),
    ("x", torch.zeros(COLS, ROWS, dtype=torch.float32).t(), "contiguous"),
])
def test_bad_argument_refused(name, bad, msg):
    a = nv_args()
    a[name] = bad
    with pytest.raises((ValueError, TypeError), match=msg):
        check(**a)


def test_importance_required_only_where_weights_decide():
    a = nv_args(objective=B.FP4Q_OBJ_WMSE)
    a["importance"] = None
    with pytest.raises(ValueError, match="importance is required"):
        check(**a)
    # AbsMax NVFP4 never weighs blocks: no importance needed
    a = nv_args(objective=B.FP4Q_OBJ_WMSE, rule=B.FP4Q_SCALE_ABSMAX)
    a["importance"] = None
    check(**a)
    # IF4 picks FP4 or INT4 by the weighted error even under AbsMax
    a = nv_args(objective=B.FP4Q_OBJ_WMSE, rule=B.FP4Q_SCALE_ABSMAX, fmt=B.FP4Q_IF4)
    a["importance"] = None
    with pytest.raises(ValueError, match="importance is required"):
        check(**a)


def test_mxfp4_needs_no_global_scale():
    a = nv_args(fmt=B.FP4Q_MXFP4, rule=B.FP4Q_SCALE_ABSMAX)
    a["scales"] = torch.empty(ROWS * COLS // 32, dtype=torch.uint8)
    a["global_scale"] = None
    check(**a)


def test_dequantize_checks():
    spec = B.make_spec(B.FP4Q_NVFP4)
    n = ROWS * COLS
    codes = torch.empty(n // 2, dtype=torch.uint8)
    scales = torch.empty(n // 16, dtype=torch.uint8)
    gs = torch.empty(1, dtype=torch.float32)
    y = torch.empty(ROWS, COLS, dtype=torch.bfloat16)
    B.check_dequantize_args(spec, codes, scales, gs, ROWS, COLS, y, require_cuda=False)
    with pytest.raises(ValueError, match="at least"):
        B.check_dequantize_args(spec, codes, scales, gs, ROWS, COLS, y[:-1], require_cuda=False)
    with pytest.raises(ValueError, match="dtype"):
        B.check_dequantize_args(spec, codes, scales, gs, ROWS, COLS,
                                torch.empty(n, dtype=torch.float16), require_cuda=False)
    with pytest.raises(ValueError, match="ROCm device"):
        B.fp4q_dequantize(spec, codes, scales, gs, ROWS, COLS, 0, y)


def test_error_and_relaxed_checks():
    a = nv_args()
    B.check_error_args(a["spec"], a["x"], None, a["codes"], a["scales"], a["global_scale"],
                       a["workspace"], require_cuda=False)
    with pytest.raises(ValueError, match="at least"):
        B.check_error_args(a["spec"], a["x"], torch.ones(3), a["codes"], a["scales"],
                           a["global_scale"], a["workspace"], require_cuda=False)
    coef = torch.ones(ROWS, COLS // 8, dtype=torch.float32)
    B.check_relaxed_args(a["spec"], a["x"], coef, 8, a["codes"], a["scales"], a["global_scale"],
                         a["workspace"], require_cuda=False)
    with pytest.raises(ValueError, match="at least"):
        B.check_relaxed_args(a["spec"], a["x"], coef[:-1], 8, a["codes"], a["scales"],
                             a["global_scale"], a["workspace"], require_cuda=False)
