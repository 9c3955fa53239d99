"""The C ABI on the host: the library loads, exports every symbol the header
declares, and rejects bad arguments before any HIP call (no GPU needed)."""
import ctypes as C
import os
import re

import pytest

from block_scaled_fp4_fp4q_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp4q.h")

# fake, suitably aligned device addresses: validation fails before any is used
X, CODES, SCALES, GS, WS, IMP = (C.c_void_p(0x10000 * k) for k in range(1, 7))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("libfp4q.so not built")
    return B.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp4q_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(B.EXPORTS)


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_abi_version_and_status_strings(L):
    assert L.fp4q_abi_version() == 3
    for st in B.STATUS:
        assert L.fp4q_status_string(st)
    assert L.fp4q_status_string(-99) == b"unknown status"


def spec(**kw):
    s = B.make_spec()
    for k, v in kw.items():
        setattr(s, k, v)
    return s


def q(L, s, x=X, dtype=B.FP4Q_BF16, rows=4, cols=64, imp=None, codes=CODES, scales=SCALES,
      gs=GS, ws=WS, ws_bytes=1 << 20):
    return L.fp4q_quantize(C.byref(s) if s is not None else None, x, dtype, rows, cols, imp,
                           codes, scales, gs, ws, ws_bytes, None)


def test_workspace_bytes(L):
    assert L.fp4q_workspace_bytes(C.byref(spec()), 4, 64) >= 256
    assert L.fp4q_workspace_bytes(C.byref(spec()), 4, 63) == 0
    assert L.fp4q_workspace_bytes(C.byref(spec(block=32)), 4, 64) == 0
    assert L.fp4q_workspace_bytes(None, 4, 64) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(format=7), -2),
    (dict(block=32), -4),
    (dict(format=B.FP4Q_MXFP4), -4),                                  # block stays 16
    (dict(rotate=8), -2),
    (dict(scale_rule=5), -2),
    (dict(objective=3), -2),
    (dict(global_scale_given=2), -2),
    (dict(scale_rule=B.FP4Q_SCALE_SWEEP, sweep_lo=3, sweep_hi=2), -2),
    (dict(scale_rule=B.FP4Q_SCALE_SWEEP, sweep_lo=-127), -2),
    (dict(scale_rule=B.FP4Q_SCALE_SWEEP, sweep_hi=127), -2),
    (dict(scale_rule=B.FP4Q_SCALE_FOUR_OVER_SIX, format=B.FP4Q_IF4), -4),  # 4/6 is NVFP4-only
    (dict(scale_rule=B.FP4Q_SCALE_FOUR_OVER_SIX, format=B.FP4Q_MXFP4, block=32), -4),
    (dict(scale_rule=B.FP4Q_SCALE_SWEEP, format=B.FP4Q_MXFP4, block=32, sweep_lo=2, sweep_hi=1), -2),
    (dict(scale_rule=B.FP4Q_SCALE_SWEEP, format=B.FP4Q_IF4, sweep_hi=127), -2),
])
def test_quantize_rejects_bad_spec(L, kw, status):
    assert q(L, spec(**kw)) == status


def test_quantize_rejects_bad_arguments(L):
    assert q(L, None) == -1
    assert q(L, spec(), x=None) == -1
    assert q(L, spec(), codes=None) == -1
    assert q(L, spec(), scales=None) == -1
    assert q(L, spec(), gs=None) == -1                                   # NVFP4 needs S
    assert q(L, spec(), ws=None) == -1
    w = spec(scale_rule=B.FP4Q_SCALE_SWEEP, objective=B.FP4Q_OBJ_WMSE)
    assert q(L, w, imp=None) == -1                                       # WMSE needs importance
    assert q(L, spec(), dtype=5) == -2
    assert q(L, spec(), cols=63) == -3
    assert q(L, spec(), rows=-1) == -3
    assert q(L, spec(), ws_bytes=100) == -2
    assert q(L, spec(), x=C.c_void_p(0x10008)) == -6                    # x not 16-aligned
    assert q(L, spec(), codes=C.c_void_p(0x10004)) == -6
    assert q(L, spec(), ws=C.c_void_p(0x10080)) == -6
    assert q(L, w, imp=C.c_void_p(0x10004)) == -6
    # every rule whose choice compares block errors needs the weights
    for kw in (dict(scale_rule=B.FP4Q_SCALE_FOUR_OVER_SIX),
               dict(format=B.FP4Q_MXFP4, block=32, scale_rule=B.FP4Q_SCALE_SWEEP),
               dict(format=B.FP4Q_IF4, scale_rule=B.FP4Q_SCALE_SWEEP),
               dict(format=B.FP4Q_IF4)):
        assert q(L, spec(objective=B.FP4Q_OBJ_WMSE, **kw), imp=None) == -1, kw


COEF = C.c_void_p(0x70000)


def rq(L, s, x=X, dtype=B.FP4Q_BF16, rows=4, cols=64, coef=COEF, group=16, given=0,
       codes=CODES, scales=SCALES, gs=GS, ws=WS, ws_bytes=1 << 20):
    return L.fp4q_quantize_relaxed(C.byref(s) if s is not None else None, x, dtype, rows, cols,
                                   coef, group, given, codes, scales, gs, ws, ws_bytes, None)


def test_quantize_relaxed_rejects_bad_arguments(L):
    mx = spec(format=B.FP4Q_MXFP4, block=32)
    assert rq(L, None) == -1
    assert rq(L, spec(), coef=None) == -1
    assert rq(L, spec(), x=None) == -1
    assert rq(L, spec(), scales=None) == -1
    assert rq(L, spec(), gs=None) == -1                                  # NVFP4 needs S
    assert rq(L, spec(), ws=None) == -1
    assert rq(L, spec(format=B.FP4Q_IF4)) == -4                          # relaxed FP4 only
    assert rq(L, spec(rotate=16)) == -4
    assert rq(L, spec(), group=4) == -2
    assert rq(L, spec(), group=32) == -2                                 # 8 or the block
    assert rq(L, mx, group=16) == -2
    assert rq(L, spec(), given=2) == -2
    assert rq(L, spec(), dtype=3) == -2
    assert rq(L, spec(), cols=40) == -3
    assert rq(L, spec(), ws_bytes=64) == -2
    assert rq(L, spec(), coef=C.c_void_p(0x70002)) == -6
    assert rq(L, mx, group=8, codes=C.c_void_p(0x10008)) == -6          # MXFP4 codes 16-aligned


def test_dequantize_and_error_reject_bad_arguments(L):
    s = spec()
    f = L.fp4q_dequantize
    assert f(None, CODES, SCALES, GS, 4, 64, 0, X, 0, None) == -1
    assert f(C.byref(s), None, SCALES, GS, 4, 64, 0, X, 0, None) == -1
    assert f(C.byref(s), CODES, SCALES, None, 4, 64, 0, X, 0, None) == -1
    assert f(C.byref(s), CODES, SCALES, GS, 4, 64, 3, X, 0, None) == -2
    assert f(C.byref(s), CODES, SCALES, GS, 4, 64, 0, X, 9, None) == -2
    assert f(C.byref(s), CODES, SCALES, GS, 4, 60, 0, X, 0, None) == -3
    assert f(C.byref(s), CODES, SCALES, GS, 4, 64, 0, C.c_void_p(0x10004), 0, None) == -6
    out = (C.c_double * 2)()
    e = L.fp4q_error
    assert e(C.byref(s), X, 1, 4, 64, None, CODES, SCALES, GS, WS, 1 << 20, None, None) == -1
    assert e(C.byref(s), X, 1, 4, 64, None, CODES, SCALES, GS, WS, 10, out, None) == -2
    assert e(C.byref(s), X, 1, 4, 60, None, CODES, SCALES, GS, WS, 1 << 20, out, None) == -3
    assert e(C.byref(s), X, 4, 4, 64, None, CODES, SCALES, GS, WS, 1 << 20, out, None) == -2
    # global scale and importance must be aligned for their binary32 loads
    assert f(C.byref(s), CODES, SCALES, C.c_void_p(0x30002), 4, 64, 0, X, 0, None) == -6
    assert e(C.byref(s), X, 1, 4, 64, None, CODES, SCALES, C.c_void_p(0x30002), WS, 1 << 20, out, None) == -6
    assert e(C.byref(s), X, 1, 4, 64, C.c_void_p(0x50002), CODES, SCALES, GS, WS, 1 << 20, out, None) == -6


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(B, "_LIB", None)
    with pytest.raises(ImportError):
        B.lib()


def test_noalloc_rejects_bad_arguments_before_any_hip_call(L):
    def qn(s, x=X, dtype=B.FP4Q_BF16, rows=4, cols=64, imp=None, codes=CODES, scales=SCALES,
           gs=GS):
        return L.fp4q_quantize_noalloc(C.byref(s) if s is not None else None, x, dtype, rows,
                                       cols, imp, codes, scales, gs, None)
    assert qn(None) == -1                                   # FP4Q_E_NULL
    assert qn(spec(format=7)) == -2                         # FP4Q_E_ARG
    assert qn(spec(), cols=60) == -3                        # FP4Q_E_SHAPE
    assert qn(spec(), x=C.c_void_p(0x10008)) == -6          # FP4Q_E_ALIGN
    assert qn(spec(), gs=None) == -1
    assert qn(spec(scale_rule=1, objective=1)) == -1        # WMSE without importance
    assert L.fp4q_status_string(-7) != b"unknown status"


def test_importance_must_be_16_byte_aligned_where_used(L):
    # 4-byte aligned (an offset view of a weight vector): refused before any
    # HIP call (only rejected calls are made here: the pointers are fake)
    s = spec(scale_rule=1, objective=1)
    assert q(L, s, imp=C.c_void_p(IMP.value + 4), dtype=B.FP4Q_F32) == -6
    assert q(L, spec(format=2, objective=1), imp=C.c_void_p(IMP.value + 8)) == -6


def test_if3_if6_argument_checks(L):
    # every call below is rejected before any HIP call (the pointers are fake)
    for fmt, misaligned in ((3, 1), (4, 2)):          # IF3 codes 2-aligned, IF6 4-aligned
        assert q(L, spec(format=fmt), codes=C.c_void_p(CODES.value + misaligned)) == -6
        assert q(L, spec(format=fmt, block=32)) == -4                 # block must be 16
        assert q(L, spec(format=fmt, scale_rule=2)) == -4             # Four Over Six: NVFP4 only
        assert q(L, spec(format=fmt, objective=1)) == -1              # the pick weighs blocks
        s = spec(format=fmt)
        assert L.fp4q_quantize_relaxed(C.byref(s), X, B.FP4Q_BF16, 4, 64, IMP, 8, 0, CODES, SCALES,
                                       GS, WS, 1 << 20, None) == -4   # no relaxed encode
    assert q(L, spec(format=5)) == -2


def test_code_bytes_per_format():
    assert B.code_bytes(B.FP4Q_NVFP4, 64) == 32 and B.code_bytes(B.FP4Q_IF4, 64) == 32
    assert B.code_bytes(B.FP4Q_IF6, 64) == 48 and B.code_bytes(B.FP4Q_IF3, 64) == 24
