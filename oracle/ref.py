"""ctypes front end of the C oracle (test infrastructure only).

Arrays are numpy: bf16 tensors travel as uint16 bit patterns, everything
else in its natural dtype.  Nothing here touches a GPU.
"""
import ctypes as C
import os

import numpy as np

from . import build as _build

NVFP4, MXFP4, IF4, IF3, IF6 = 0, 1, 2, 3, 4
F32, BF16 = 0, 1
ABSMAX, SWEEP, FOUR_SIX = 0, 1, 2
MSE, WMSE = 0, 1

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = C.CDLL(_build.LIB)
        f, d, i, i64 = C.c_float, C.c_double, C.c_int, C.c_int64
        vp = C.c_void_p
        sig = {
            "fp4q_ref_e2m1_value": (f, [i]),
            "fp4q_ref_e2m1_round": (i, [f]),
            "fp4q_ref_e4m3_value": (f, [i]),
            "fp4q_ref_e4m3_round": (i, [f]),
            "fp4q_ref_e8m0_value": (f, [i]),
            "fp4q_ref_int4_round": (i, [f]),
            "fp4q_ref_bf16_to_f32": (f, [C.c_uint16]),
            "fp4q_ref_f32_to_bf16": (C.c_uint16, [f]),
            "fp4q_ref_int4_step": (f, []),
            "fp4q_ref_fpn_value": (f, [i, i]),
            "fp4q_ref_fpn_max": (f, [i]),
            "fp4q_ref_fpn_round": (i, [i, f]),
            "fp4q_ref_intn_round": (i, [i, f]),
            "fp4q_ref_ifn_step": (f, [i]),
            "fp4q_ref_ifn_global_scale": (f, [i, f]),
            "fp4q_ref_ifn_base_scale": (i, [i, vp, i, f]),
            "fp4q_ref_fpn_block": (d, [i, vp, i, vp, f, i, vp]),
            "fp4q_ref_intn_block": (d, [i, vp, i, vp, f, i, vp]),
            "fp4q_ref_rotation_scale": (f, [i]),
            "fp4q_ref_fwht": (None, [vp, i]),
            "fp4q_ref_global_scale": (f, [f]),
            "fp4q_ref_prepare": (i, [vp, i, i64, i64, i, vp, i]),
            "fp4q_ref_nvfp4_block": (d, [vp, i, vp, f, i, vp]),
            "fp4q_ref_int4_block": (d, [vp, i, vp, f, i, vp]),
            "fp4q_ref_base_scale": (i, [vp, i, f]),
            "fp4q_ref_candidate_errors": (i, [vp, i64, i, vp, f, vp, i]),
            "fp4q_ref_quantize": (i, [i, i, i, i, i, i, i, i, vp, i, i64, i64,
                                      vp, vp, vp, vp, vp, vp, i]),
            "fp4q_ref_dequantize": (i, [i, i, vp, vp, vp, i64, i64, i, vp, i, i]),
            "fp4q_ref_quantize_relaxed": (i, [i, i, i, vp, i, i64, i64, vp, i, i, vp, vp, vp, i]),
            "fp4q_ref_error": (i, [i, i, i, vp, i, i64, i64, vp, vp, vp, vp, vp, i]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _dtype_code(x):
    if x.dtype == np.float32:
        return F32
    if x.dtype == np.uint16:
        return BF16
    raise TypeError("x must be float32 or uint16 (bf16 bit patterns)")


def block_size(fmt):
    return 32 if fmt == MXFP4 else 16


def code_bits(fmt):
    """Bits per element code: 3 for IF3, 6 for IF6, 4 otherwise."""
    return {IF3: 3, IF6: 6}.get(fmt, 4)


def code_bytes(fmt, n):
    """Bytes of the code stream of n elements."""
    return n * code_bits(fmt) // 8


def default_window(objective, fmt=NVFP4):
    if fmt == MXFP4:
        return (0, 1)
    return (-8, 7) if objective == WMSE else (-3, 7)


def quantize(x, fmt=NVFP4, rule=ABSMAX, objective=MSE, window=None, rotate=0,
             global_scale=None, importance=None, nthreads=0, errors=False):
    """Quantize a 2-D host tensor; returns a dict of numpy outputs."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    B = block_size(fmt)
    lo, hi = window if window is not None else default_window(objective, fmt)
    nb = rows * cols // B
    codes = np.zeros(code_bytes(fmt, rows * cols), np.uint8)
    scales = np.zeros(nb, np.uint8)
    gs = np.array([global_scale if global_scale is not None else 0.0], np.float32)
    imp = None if importance is None else np.ascontiguousarray(importance, np.float32)
    best = np.zeros(nb, np.float64) if errors else None
    second = np.zeros(nb, np.float64) if errors else None
    rc = lib().fp4q_ref_quantize(fmt, B, rule, objective, lo, hi, rotate,
                                 int(global_scale is not None), _p(x), _dtype_code(x),
                                 rows, cols, _p(imp), _p(codes), _p(scales), _p(gs),
                                 _p(best), _p(second), nthreads)
    if rc != 0:
        raise ValueError(f"fp4q_ref_quantize failed: {rc}")
    out = {"codes": codes, "scales": scales, "S": float(gs[0])}
    if errors:
        out["best"] = best
        out["second"] = second
    return out


def quantize_relaxed(x, coef, group, fmt=NVFP4, global_scale=None, scales=None, nthreads=0):
    """FOCUS deploy-side encode with given coefficients (fp32 [rows, cols/group])."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    B = block_size(fmt)
    codes = np.zeros(rows * cols // 2, np.uint8)
    given = scales is not None
    sc = np.array(scales, np.uint8).copy() if given else np.zeros(rows * cols // B, np.uint8)
    gs = np.array([global_scale if global_scale is not None else 0.0], np.float32)
    coef = np.ascontiguousarray(coef, np.float32)
    rc = lib().fp4q_ref_quantize_relaxed(fmt, B, int(global_scale is not None), _p(x),
                                         _dtype_code(x), rows, cols, _p(coef), group, int(given),
                                         _p(codes), _p(sc), _p(gs), nthreads)
    if rc != 0:
        raise ValueError(f"fp4q_ref_quantize_relaxed failed: {rc}")
    return {"codes": codes, "scales": sc, "S": float(gs[0])}


def dequantize(codes, scales, S, rows, cols, fmt=NVFP4, unrotate=0, out_dtype=F32,
               nthreads=0):
    B = block_size(fmt)
    y = np.zeros(rows * cols, np.float32 if out_dtype == F32 else np.uint16)
    gs = np.array([S if S is not None else 1.0], np.float32)
    rc = lib().fp4q_ref_dequantize(fmt, B, _p(np.ascontiguousarray(codes)),
                                   _p(np.ascontiguousarray(scales)), _p(gs), rows, cols,
                                   unrotate, _p(y), out_dtype, nthreads)
    if rc != 0:
        raise ValueError(f"fp4q_ref_dequantize failed: {rc}")
    return y.reshape(rows, cols)


def error(x, codes, scales, S, fmt=NVFP4, rotate=0, importance=None, nthreads=0):
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    B = block_size(fmt)
    out = np.zeros(2, np.float64)
    gs = np.array([S if S is not None else 1.0], np.float32)
    imp = None if importance is None else np.ascontiguousarray(importance, np.float32)
    rc = lib().fp4q_ref_error(fmt, B, rotate, _p(x), _dtype_code(x), rows, cols, _p(imp),
                              _p(np.ascontiguousarray(codes)),
                              _p(np.ascontiguousarray(scales)), _p(gs), _p(out), nthreads)
    if rc != 0:
        raise ValueError(f"fp4q_ref_error failed: {rc}")
    return float(out[0]), float(out[1])


def prepare(x, rotate=0, nthreads=0):
    """Widened (and block-rotated) float32 copy of a host tensor."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    out = np.zeros((rows, cols), np.float32)
    rc = lib().fp4q_ref_prepare(_p(x), _dtype_code(x), rows, cols, rotate, _p(out), nthreads)
    if rc != 0:
        raise ValueError(f"fp4q_ref_prepare failed: {rc}")
    return out


def fwht(v):
    v = np.array(v, np.float32)
    lib().fp4q_ref_fwht(_p(v), len(v))
    return v


def nvfp4_block(xb, S, c, w=None):
    """Error and nibbles of one prepared block encoded with scale byte c."""
    xb = np.ascontiguousarray(xb, np.float32)
    codes = np.zeros(len(xb), np.uint8)
    w = None if w is None else np.ascontiguousarray(w, np.float32)
    e = lib().fp4q_ref_nvfp4_block(_p(xb), len(xb), _p(w), S, c, _p(codes))
    return e, codes


def int4_block(xb, S, c, w=None):
    xb = np.ascontiguousarray(xb, np.float32)
    codes = np.zeros(len(xb), np.uint8)
    w = None if w is None else np.ascontiguousarray(w, np.float32)
    e = lib().fp4q_ref_int4_block(_p(xb), len(xb), _p(w), S, c, _p(codes))
    return e, codes


def base_scale(xb, S):
    xb = np.ascontiguousarray(xb, np.float32)
    return lib().fp4q_ref_base_scale(_p(xb), len(xb), S)


def candidate_errors(blocks, S, w=None, nthreads=0):
    """Errors of every E4M3 scale byte (columns 1..126) for each row of
    `blocks` (prepared float32 values, one block per row)."""
    blocks = np.ascontiguousarray(blocks, np.float32)
    nb, B = blocks.shape
    out = np.zeros((nb, 127), np.float64)
    w = None if w is None else np.ascontiguousarray(w, np.float32)
    rc = lib().fp4q_ref_candidate_errors(_p(blocks), nb, B, _p(w), S, _p(out), nthreads)
    if rc != 0:
        raise ValueError(rc)
    return out


def unpack_codes(codes, fmt):
    """The n-bit element codes of a code stream (element e at bits
    n e .. n e + n - 1, least significant bit first)."""
    n = code_bits(fmt)
    bits = np.unpackbits(np.asarray(codes, np.uint8), bitorder="little")
    bits = bits[: bits.size // n * n].reshape(-1, n).astype(np.uint16)
    return (bits << np.arange(n, dtype=np.uint16)).sum(axis=1).astype(np.uint8)


def fpn_block(n, xb, S, c, w=None):
    """Error and codes of the FP branch of an n-bit adaptive type."""
    xb = np.ascontiguousarray(xb, np.float32)
    codes = np.zeros(len(xb), np.uint8)
    w = None if w is None else np.ascontiguousarray(w, np.float32)
    e = lib().fp4q_ref_fpn_block(n, _p(xb), len(xb), _p(w), S, c, _p(codes))
    return e, codes


def intn_block(n, xb, S, c, w=None):
    xb = np.ascontiguousarray(xb, np.float32)
    codes = np.zeros(len(xb), np.uint8)
    w = None if w is None else np.ascontiguousarray(w, np.float32)
    e = lib().fp4q_ref_intn_block(n, _p(xb), len(xb), _p(w), S, c, _p(codes))
    return e, codes


def unpack_nibbles(codes):
    codes = np.asarray(codes, np.uint8)
    out = np.empty(codes.size * 2, np.uint8)
    out[0::2] = codes & 0xF
    out[1::2] = codes >> 4
    return out
