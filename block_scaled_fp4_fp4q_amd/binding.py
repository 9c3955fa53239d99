"""Thin ctypes binding of libfp4q.so (include/fp4q.h).

Argument marshalling only: tensors are torch tensors on a ROCm device, whose
data pointers and current HIP stream are handed to the C ABI unchanged.  All
arithmetic happens in the library's HIP kernels.  There is no fallback: if the
library is missing, or a call is rejected, this module raises.
"""
import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp4q.so")

FP4Q_NVFP4, FP4Q_MXFP4, FP4Q_IF4, FP4Q_IF3, FP4Q_IF6 = 0, 1, 2, 3, 4
FP4Q_F32, FP4Q_BF16 = 0, 1
FP4Q_SCALE_ABSMAX, FP4Q_SCALE_SWEEP, FP4Q_SCALE_FOUR_OVER_SIX = 0, 1, 2
FP4Q_OBJ_MSE, FP4Q_OBJ_WMSE = 0, 1

STATUS = {0: "FP4Q_OK", -1: "FP4Q_E_NULL", -2: "FP4Q_E_ARG", -3: "FP4Q_E_SHAPE",
          -4: "FP4Q_E_UNSUPPORTED", -5: "FP4Q_E_HIP", -6: "FP4Q_E_ALIGN", -7: "FP4Q_E_SCRATCH"}

# every symbol include/fp4q.h declares
EXPORTS = ("fp4q_workspace_bytes", "fp4q_quantize", "fp4q_quantize_noalloc",
           "fp4q_quantize_relaxed", "fp4q_dequantize", "fp4q_error", "fp4q_status_string",
           "fp4q_abi_version")


class fp4q_spec(C.Structure):
    _fields_ = [("format", C.c_int32), ("block", C.c_int32), ("scale_rule", C.c_int32),
                ("objective", C.c_int32), ("sweep_lo", C.c_int32), ("sweep_hi", C.c_int32),
                ("rotate", C.c_int32), ("global_scale_given", C.c_int32)]


class Fp4qError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        msg = _lib_handle().fp4q_status_string(status).decode() if _LIB is not None else ""
        super().__init__(f"{fn} returned {STATUS.get(status, status)}: {msg}")


_LIB = None


def _lib_handle():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                              "or python block_scaled_fp4_fp4q_amd/build.py")
        L = C.CDLL(LIB_PATH)
        vp, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
        sp = C.POINTER(fp4q_spec)
        L.fp4q_workspace_bytes.restype = sz
        L.fp4q_workspace_bytes.argtypes = [sp, i64, i64]
        L.fp4q_quantize.restype = C.c_int
        L.fp4q_quantize.argtypes = [sp, vp, i32, i64, i64, vp, vp, vp, vp, vp, sz, vp]
        L.fp4q_quantize_noalloc.restype = C.c_int
        L.fp4q_quantize_noalloc.argtypes = [sp, vp, i32, i64, i64, vp, vp, vp, vp, vp]
        L.fp4q_quantize_relaxed.restype = C.c_int
        L.fp4q_quantize_relaxed.argtypes = [sp, vp, i32, i64, i64, vp, i32, i32, vp, vp, vp, vp,
                                            sz, vp]
        L.fp4q_dequantize.restype = C.c_int
        L.fp4q_dequantize.argtypes = [sp, vp, vp, vp, i64, i64, i32, vp, i32, vp]
        L.fp4q_error.restype = C.c_int
        L.fp4q_error.argtypes = [sp, vp, i32, i64, i64, vp, vp, vp, vp, vp, sz,
                                 C.POINTER(C.c_double), vp]
        L.fp4q_status_string.restype = C.c_char_p
        L.fp4q_status_string.argtypes = [C.c_int]
        L.fp4q_abi_version.restype = C.c_int
        L.fp4q_abi_version.argtypes = []
        _LIB = L
    return _LIB


def lib():
    return _lib_handle()


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def _dtype_code(t):
    if t.dtype == torch.float32:
        return FP4Q_F32
    if t.dtype == torch.bfloat16:
        return FP4Q_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _check(fn, st):
    if st != 0:
        raise Fp4qError(fn, st)


def make_spec(format=FP4Q_NVFP4, scale_rule=FP4Q_SCALE_ABSMAX, objective=FP4Q_OBJ_MSE,
              window=None, rotate=0, global_scale_given=False):
    block = 32 if format == FP4Q_MXFP4 else 16
    if window is None:
        # E8M0: the OCP exponent and the next one up; E4M3: the pages' windows
        window = (0, 1) if format == FP4Q_MXFP4 else \
            ((-8, 7) if objective == FP4Q_OBJ_WMSE else (-3, 7))
    lo, hi = window
    return fp4q_spec(format, block, scale_rule, objective, lo, hi, rotate, int(global_scale_given))


def _as_2d(x):
    if not isinstance(x, torch.Tensor):
        raise TypeError("x must be a torch tensor")
    if x.dim() < 2:
        raise ValueError("x must have at least 2 dimensions (rows, cols)")
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    return x.reshape(-1, x.shape[-1])


# The C ABI receives bare device pointers and cannot see a buffer's size,
# device or type: a host tensor or a short buffer would be read or written
# out of bounds by a kernel.  Every tensor argument is therefore checked here,
# before the library is called.  `require_cuda` is only turned off by the
# host-side tests of these checks.

def _check_device(name, t, device, require_cuda):
    if require_cuda and t.device.type != "cuda":
        raise ValueError(f"{name} must be a tensor on a ROCm device, not {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, but x is on {device}")


def _check_tensor(name, t, dtypes, min_numel, device, require_cuda=True, optional=False):
    """A device tensor argument: on x's device, one of `dtypes`, contiguous,
    at least `min_numel` elements.  None passes only when `optional`."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    _check_device(name, t, device, require_cuda)
    if t.dtype not in dtypes:
        want = " or ".join(str(d) for d in dtypes)
        raise ValueError(f"{name} has dtype {t.dtype}; expected {want}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < min_numel:
        raise ValueError(f"{name} has {t.numel()} elements; at least {min_numel} are needed")


_U8 = (torch.uint8,)
_F32 = (torch.float32,)
_X = (torch.float32, torch.bfloat16)


ADAPTIVE = (FP4Q_IF4, FP4Q_IF3, FP4Q_IF6)


def code_bytes(format, n):
    """Bytes of the code stream of n elements: n-bit codes for IF3 (3) and
    IF6 (6), 4-bit codes otherwise."""
    return n * {FP4Q_IF3: 3, FP4Q_IF6: 6}.get(format, 4) // 8


def _needs_importance(spec):
    return spec.objective == FP4Q_OBJ_WMSE and (spec.scale_rule != FP4Q_SCALE_ABSMAX
                                                or spec.format in ADAPTIVE)


def _check_outputs(spec, rows, cols, codes, scales, global_scale, dev, require_cuda):
    n = rows * cols
    _check_tensor("codes", codes, _U8, code_bytes(spec.format, n), dev, require_cuda)
    _check_tensor("scales", scales, _U8, n // spec.block, dev, require_cuda)
    _check_tensor("global_scale", global_scale, _F32, 1, dev, require_cuda,
                  optional=spec.format == FP4Q_MXFP4)


def _check_workspace(spec, rows, cols, workspace, dev, require_cuda):
    need = fp4q_workspace_bytes(spec, rows, cols)
    _check_tensor("workspace", workspace, _U8, need, dev, require_cuda)


def check_quantize_args(spec, x, importance, codes, scales, global_scale, workspace,
                        require_cuda=True):
    """Host-side checks of fp4q_quantize's tensor arguments; raises
    ValueError/TypeError.  Returns x as a [rows, cols] view."""
    x2 = _as_2d(x)
    _check_device("x", x2, None, require_cuda)
    _dtype_code(x2)
    rows, cols = x2.shape
    dev = x2.device
    _check_tensor("importance", importance, _F32, cols, dev, require_cuda,
                  optional=not _needs_importance(spec))
    _check_outputs(spec, rows, cols, codes, scales, global_scale, dev, require_cuda)
    _check_workspace(spec, rows, cols, workspace, dev, require_cuda)
    return x2


def check_quantize_noalloc_args(spec, x, importance, codes, scales, global_scale,
                                require_cuda=True):
    """fp4q_quantize's checks without the workspace (the library's own
    static scratch serves instead)."""
    x2 = _as_2d(x)
    _check_device("x", x2, None, require_cuda)
    _dtype_code(x2)
    rows, cols = x2.shape
    dev = x2.device
    _check_tensor("importance", importance, _F32, cols, dev, require_cuda,
                  optional=not _needs_importance(spec))
    _check_outputs(spec, rows, cols, codes, scales, global_scale, dev, require_cuda)
    return x2


def check_relaxed_args(spec, x, coef, coef_group, codes, scales, global_scale, workspace,
                       require_cuda=True):
    x2 = _as_2d(x)
    _check_device("x", x2, None, require_cuda)
    _dtype_code(x2)
    rows, cols = x2.shape
    dev = x2.device
    if coef_group <= 0:
        raise ValueError("coef_group must be positive")
    _check_tensor("coef", coef, _F32, rows * (cols // coef_group), dev, require_cuda)
    _check_outputs(spec, rows, cols, codes, scales, global_scale, dev, require_cuda)
    _check_workspace(spec, rows, cols, workspace, dev, require_cuda)
    return x2


def check_dequantize_args(spec, codes, scales, global_scale, rows, cols, y, require_cuda=True):
    if not isinstance(y, torch.Tensor):
        raise TypeError("y must be a torch tensor")
    _check_device("y", y, None, require_cuda)
    dev = y.device
    _check_tensor("y", y, _X, rows * cols, dev, require_cuda)
    _check_outputs(spec, rows, cols, codes, scales, global_scale, dev, require_cuda)


def check_error_args(spec, x, importance, codes, scales, global_scale, workspace,
                     require_cuda=True):
    x2 = _as_2d(x)
    _check_device("x", x2, None, require_cuda)
    _dtype_code(x2)
    rows, cols = x2.shape
    dev = x2.device
    _check_tensor("importance", importance, _F32, cols, dev, require_cuda, optional=True)
    _check_outputs(spec, rows, cols, codes, scales, global_scale, dev, require_cuda)
    _check_workspace(spec, rows, cols, workspace, dev, require_cuda)
    return x2


# ---------------------------------------------------------------------------
# the C ABI, one Python function per entry point
# ---------------------------------------------------------------------------

def fp4q_workspace_bytes(spec, rows, cols):
    return int(_lib_handle().fp4q_workspace_bytes(C.byref(spec), rows, cols))


def fp4q_quantize(spec, x, importance, codes, scales, global_scale, workspace, stream=None):
    x2 = check_quantize_args(spec, x, importance, codes, scales, global_scale, workspace)
    rows, cols = x2.shape
    st = _lib_handle().fp4q_quantize(C.byref(spec), _ptr(x2), _dtype_code(x2), rows, cols,
                                     _ptr(importance), _ptr(codes), _ptr(scales),
                                     _ptr(global_scale), _ptr(workspace), workspace.numel(),
                                     _stream(stream))
    _check("fp4q_quantize", st)


def fp4q_quantize_noalloc(spec, x, importance, codes, scales, global_scale, stream=None):
    """fp4q_quantize without a workspace: the library's static per-GPU
    scratch serves instead.  Calls that overlap on one GPU race on it."""
    x2 = check_quantize_noalloc_args(spec, x, importance, codes, scales, global_scale)
    rows, cols = x2.shape
    st = _lib_handle().fp4q_quantize_noalloc(C.byref(spec), _ptr(x2), _dtype_code(x2), rows, cols,
                                             _ptr(importance), _ptr(codes), _ptr(scales),
                                             _ptr(global_scale), _stream(stream))
    _check("fp4q_quantize_noalloc", st)


def fp4q_quantize_relaxed(spec, x, coef, coef_group, scales_given, codes, scales, global_scale,
                          workspace, stream=None):
    x2 = check_relaxed_args(spec, x, coef, coef_group, codes, scales, global_scale, workspace)
    rows, cols = x2.shape
    st = _lib_handle().fp4q_quantize_relaxed(C.byref(spec), _ptr(x2), _dtype_code(x2), rows, cols,
                                             _ptr(coef), coef_group, int(scales_given), _ptr(codes),
                                             _ptr(scales), _ptr(global_scale), _ptr(workspace),
                                             workspace.numel(), _stream(stream))
    _check("fp4q_quantize_relaxed", st)


def fp4q_dequantize(spec, codes, scales, global_scale, rows, cols, unrotate, y, stream=None):
    check_dequantize_args(spec, codes, scales, global_scale, rows, cols, y)
    st = _lib_handle().fp4q_dequantize(C.byref(spec), _ptr(codes), _ptr(scales),
                                       _ptr(global_scale), rows, cols, unrotate, _ptr(y),
                                       _dtype_code(y), _stream(stream))
    _check("fp4q_dequantize", st)


def fp4q_error(spec, x, importance, codes, scales, global_scale, workspace, stream=None):
    x2 = check_error_args(spec, x, importance, codes, scales, global_scale, workspace)
    rows, cols = x2.shape
    out = (C.c_double * 2)()
    st = _lib_handle().fp4q_error(C.byref(spec), _ptr(x2), _dtype_code(x2), rows, cols,
                                  _ptr(importance), _ptr(codes), _ptr(scales),
                                  _ptr(global_scale), _ptr(workspace), workspace.numel(),
                                  out, _stream(stream))
    _check("fp4q_error", st)
    return out[0], out[1]


# ---------------------------------------------------------------------------
# convenience: allocate outputs with torch, then call the entry points
# ---------------------------------------------------------------------------

def alloc_workspace(spec, rows, cols, device):
    n = fp4q_workspace_bytes(spec, rows, cols)
    if n == 0:
        raise ValueError("invalid spec or shape")
    return torch.empty(n, dtype=torch.uint8, device=device)


def quantize(x, format=FP4Q_NVFP4, scale_rule=FP4Q_SCALE_ABSMAX, objective=FP4Q_OBJ_MSE,
             window=None, rotate=0, importance=None, global_scale=None, workspace=None,
             stream=None):
    """Returns (codes uint8 [code_bytes(format, rows*cols)], scales uint8
    [rows*cols/block], global_scale float32 [1])."""
    spec = make_spec(format, scale_rule, objective, window, rotate, global_scale is not None)
    x2 = _as_2d(x)
    rows, cols = x2.shape
    dev = x.device
    codes = torch.empty(code_bytes(format, rows * cols), dtype=torch.uint8, device=dev)
    scales = torch.empty(rows * cols // spec.block, dtype=torch.uint8, device=dev)
    if global_scale is None:
        gs = torch.empty(1, dtype=torch.float32, device=dev)
    else:
        gs = torch.as_tensor(global_scale, dtype=torch.float32, device=dev).reshape(1).clone()
    ws = workspace if workspace is not None else alloc_workspace(spec, rows, cols, dev)
    fp4q_quantize(spec, x2, importance, codes, scales, gs, ws, stream)
    return codes, scales, gs


def quantize_relaxed(x, coef, coef_group, format=FP4Q_NVFP4, scales=None, global_scale=None,
                     workspace=None, stream=None):
    """FOCUS deploy encode.  coef: float32 [rows, cols/coef_group] on the
    device; scales: given S_dq bytes, or None to compute the AbsMax ones.
    Returns (codes, scales, global_scale)."""
    spec = make_spec(format, global_scale_given=global_scale is not None)
    x2 = _as_2d(x)
    rows, cols = x2.shape
    dev = x.device
    codes = torch.empty(rows * cols // 2, dtype=torch.uint8, device=dev)
    given = scales is not None
    sc = scales if given else torch.empty(rows * cols // spec.block, dtype=torch.uint8, device=dev)
    if global_scale is None:
        gs = torch.empty(1, dtype=torch.float32, device=dev)
    else:
        gs = torch.as_tensor(global_scale, dtype=torch.float32, device=dev).reshape(1).clone()
    ws = workspace if workspace is not None else alloc_workspace(spec, rows, cols, dev)
    fp4q_quantize_relaxed(spec, x2, coef, coef_group, given, codes, sc, gs, ws, stream)
    return codes, sc, gs


def dequantize(codes, scales, global_scale, rows, cols, format=FP4Q_NVFP4, unrotate=0,
               dtype=torch.float32, stream=None):
    spec = make_spec(format)
    y = torch.empty(rows, cols, dtype=dtype, device=codes.device)
    fp4q_dequantize(spec, codes, scales, global_scale, rows, cols, unrotate, y, stream)
    return y


def error(x, codes, scales, global_scale, format=FP4Q_NVFP4, rotate=0, importance=None,
          workspace=None, stream=None):
    spec = make_spec(format, rotate=rotate)
    x2 = _as_2d(x)
    rows, cols = x2.shape
    ws = workspace if workspace is not None else alloc_workspace(spec, rows, cols, x.device)
    return fp4q_error(spec, x2, importance, codes, scales, global_scale, ws, stream)
