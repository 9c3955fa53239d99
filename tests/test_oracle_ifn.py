"""Pins of the oracle's IF3 and IF6 (the adaptive type at 3 and 6 bits).

Source: Adaptive Block-Scaled Data Types, Methodology (the FP-or-INT pick of
IF4 applies to 3-bit IF3 and 6-bit IF6 formats as well).  The page fixes no
grid for them; the reading pinned here is the one under which n = 4 is
exactly IF4: FP element E2M(n-3) (bias 1, exponent field 0 subnormal), INT
element in [-(2^(n-1)-1), 2^(n-1)-1] with step D * fl32(FPmax/INTmax), E4M3
block scale with the indicator in bit 7, base scale E4M3(max/(FPmax S)),
S = max|x|/(256 FPmax), n-bit codes least significant bit first.

Each test ties the oracle to something other than itself: the OCP E2M3 and
E2M0 value sets stated as unions of uniform grids, exact-rational nearest
rounding at every midpoint, the IF4 oracle (pinned elsewhere) for n = 4,
an exact-rational restatement (tests/exactspec.py) on tiny tensors,
hand-worked blocks (tests/golden/hand_examples.json) and invariants."""
import json
import os
from fractions import Fraction as Fr

import numpy as np
import pytest

import exactspec as X

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")
f32 = np.float32


def grid(ref, n):
    return [ref.lib().fp4q_ref_fpn_value(n, m) for m in range(1 << (n - 1))]


# ---- formats -----------------------------------------------------------------

def test_e2m3_value_set(ref):
    # OCP FP6 E2M3: 1/8 steps below 2, 1/4 steps in [2, 4), 1/2 steps in [4, 7.5]
    want = sorted({Fr(k, 8) for k in range(16)} | {Fr(k, 4) for k in range(8, 16)}
                  | {Fr(k, 2) for k in range(8, 16)})
    got = [Fr(float(v)) for v in grid(ref, 6)]
    assert len(want) == 32 and got == want            # ascending with the code
    assert ref.lib().fp4q_ref_fpn_max(6) == 7.5
    assert got == X.fpn_grid(6)


def test_e2m0_and_e2m1_value_sets(ref):
    assert grid(ref, 3) == [0.0, 1.0, 2.0, 4.0]
    assert grid(ref, 4) == [ref.lib().fp4q_ref_e2m1_value(m) for m in range(8)]
    assert grid(ref, 4) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert [ref.lib().fp4q_ref_fpn_max(n) for n in (3, 4, 6)] == [4.0, 6.0, 7.5]


def exact_nearest(y, values):
    """code of the value nearest to y, the even code on an exact tie"""
    return X.nearest(Fr(float(y)), [Fr(float(v)) for v in values])


@pytest.mark.parametrize("n", [3, 4, 6])
def test_fp_rounding_at_every_midpoint(ref, n):
    vals = grid(ref, n)
    L = ref.lib()
    for a, b in zip(vals, vals[1:]):
        mid = f32((a + b) / 2)
        for y in (np.nextafter(mid, f32(0)), mid, np.nextafter(mid, f32(np.inf))):
            assert L.fp4q_ref_fpn_round(n, float(y)) == exact_nearest(y, vals), (n, float(y))
    top = (1 << (n - 1)) - 1
    for y in (vals[-1], vals[-1] * 1.2, 3e38):
        assert L.fp4q_ref_fpn_round(n, y) == top        # saturation
    if n == 4:
        for y in np.linspace(0, 8, 4097, dtype=np.float32):
            assert L.fp4q_ref_fpn_round(4, float(y)) == L.fp4q_ref_e2m1_round(float(y))


@pytest.mark.parametrize("n", [3, 4, 6])
def test_int_rounding_at_every_half_integer(ref, n):
    L = ref.lib()
    top = (1 << (n - 1)) - 1
    ints = list(range(top + 1))
    for k in range(top):
        mid = f32(k + 0.5)
        for y in (np.nextafter(mid, f32(0)), mid, np.nextafter(mid, f32(np.inf))):
            assert L.fp4q_ref_intn_round(n, float(y)) == exact_nearest(y, ints)
    assert L.fp4q_ref_intn_round(n, top + 0.7) == top
    if n == 4:
        for y in np.linspace(0, 9, 2049, dtype=np.float32):
            assert L.fp4q_ref_intn_round(4, float(y)) == L.fp4q_ref_int4_round(float(y))


def test_int_step_maps_the_int_maximum_onto_the_fp_maximum(ref):
    L = ref.lib()
    assert L.fp4q_ref_ifn_step(4) == L.fp4q_ref_int4_step() == f32(6) / f32(7)   # the 6/7 method
    for n, fpmax, top in ((3, 4.0, 3), (4, 6.0, 7), (6, 7.5, 31)):
        s = f32(L.fp4q_ref_ifn_step(n))
        assert s == f32(fpmax) / f32(top)
        assert abs(float(f32(top) * s) - fpmax) <= 2 * np.spacing(f32(fpmax))


def test_global_scale_and_base_scale(ref):
    L = ref.lib()
    assert L.fp4q_ref_ifn_global_scale(4, 6.0) == L.fp4q_ref_global_scale(6.0)
    rng = np.random.default_rng(7)
    for n in (3, 6):
        fpmax = float(L.fp4q_ref_fpn_max(n))
        assert L.fp4q_ref_ifn_global_scale(n, 0.0) == 1.0
        for g in rng.lognormal(0, 3, 50).astype(np.float32):
            S = L.fp4q_ref_ifn_global_scale(n, float(g))
            assert S == f32(g) / (f32(256) * f32(fpmax))
            # the block holding the tensor maximum lands on E4M3 256 (0x78), or
            # its neighbour when fl32 rounding of S tips the quotient
            xb = np.zeros(16, np.float32)
            xb[3] = g
            assert L.fp4q_ref_ifn_base_scale(n, xb.ctypes.data, 16, S) in (0x77, 0x78, 0x79)


# ---- whole blocks against the exact statement --------------------------------

def blocks(seed, nblocks):
    rng = np.random.default_rng(seed)
    out = []
    for b in range(nblocks):
        kind = b % 5
        if kind == 0:
            v = rng.standard_normal(16)
        elif kind == 1:
            v = rng.uniform(-1, 1, 16)
        elif kind == 2:
            v = rng.laplace(0, 0.1, 16)
            v[rng.integers(16)] = rng.choice([-1.0, 1.0])
        elif kind == 3:
            v = rng.standard_normal(16) * 10.0 ** rng.uniform(-6, 6)
        else:
            v = np.round(rng.standard_normal(16) * 4) / 4     # many exact ties
        out.append(v.astype(np.float32))
    return np.stack(out)


@pytest.mark.parametrize("n,fmt_name", [(3, "IF3"), (6, "IF6")])
@pytest.mark.parametrize("window", [None, (-3, 7)])
@pytest.mark.parametrize("weighted", [False, True])
def test_quantize_matches_exact_statement(ref, n, fmt_name, window, weighted):
    fmt = getattr(ref, fmt_name)
    x = blocks(11 + n, 30).reshape(6, 80)
    imp = np.random.default_rng(5).lognormal(0, 1, 80).astype(np.float32) if weighted else None
    rule = ref.SWEEP if window else ref.ABSMAX
    got = ref.quantize(x, fmt=fmt, rule=rule, objective=ref.WMSE if weighted else ref.MSE,
                       window=window or (0, 0), importance=imp)
    S = got["S"]
    assert S == X.ifn_global_scale(n, np.abs(x).max())
    codes = ref.unpack_codes(got["codes"], fmt)
    for b, xb in enumerate(x.reshape(-1, 16)):
        w = None if imp is None else imp[(b % 5) * 16:(b % 5) * 16 + 16]
        byte, cw, _ = X.quantize_block_ifn(n, xb, S, window or (0, 0), w)
        assert got["scales"][b] == byte, (b, got["scales"][b], byte)
        assert list(codes[16 * b:16 * b + 16]) == cw, b
    # the code stream is the n-bit packing of those codes
    all_codes = []
    for b, xb in enumerate(x.reshape(-1, 16)):
        w = None if imp is None else imp[(b % 5) * 16:(b % 5) * 16 + 16]
        all_codes += X.quantize_block_ifn(n, xb, S, window or (0, 0), w)[1]
    assert bytes(got["codes"]) == X.pack_bits(all_codes, n)


def test_n4_statement_reproduces_if4(ref):
    # the generalized statement at n = 4 is the IF4 the oracle already pins
    x = blocks(3, 40).reshape(8, 80)
    got = ref.quantize(x, fmt=ref.IF4)
    S = got["S"]
    nib = ref.unpack_nibbles(got["codes"])
    for b, xb in enumerate(x.reshape(-1, 16)):
        byte, cw, _ = X.quantize_block_ifn(4, xb, S)
        assert got["scales"][b] == byte and list(nib[16 * b:16 * b + 16]) == cw


# ---- invariants ----------------------------------------------------------------

@pytest.mark.parametrize("n", [3, 6])
def test_pick_never_loses_to_either_grid(ref, n):
    x = blocks(21, 200)
    S = float(X.ifn_global_scale(n, np.abs(x).max()))
    L = ref.lib()
    for xb in x:
        xb = np.ascontiguousarray(xb)
        c = L.fp4q_ref_ifn_base_scale(n, xb.ctypes.data, 16, S)
        ef, _ = ref.fpn_block(n, xb, S, c)
        ei, _ = ref.intn_block(n, xb, S, c)
        fmt = ref.IF3 if n == 3 else ref.IF6
        got = ref.quantize(xb.reshape(1, 16), fmt=fmt, global_scale=S, errors=True)
        assert got["best"][0] == min(ef, ei)
        assert bool(got["scales"][0] & 0x80) == (ei < ef)      # INT only when strictly lower


@pytest.mark.parametrize("n", [3, 6])
def test_lossless_round_trip_on_either_grid(ref, n):
    fmt = ref.IF3 if n == 3 else ref.IF6
    L = ref.lib()
    vals = np.array(grid(ref, n), np.float32)
    top = (1 << (n - 1)) - 1
    rng = np.random.default_rng(n)
    S = f32(2.0 ** -5)
    rows = []
    for b in range(64):
        c = int(rng.integers(0x20, 0x60))
        D = f32(L.fp4q_ref_e4m3_value(c)) * S
        if b % 2 == 0:           # on the FP grid, block maximum on the top code
            m = rng.integers(0, top + 1, 16)
            m[0] = top
            sgn = np.where(rng.random(16) < 0.5, -1, 1).astype(np.float32)
            xb = sgn * (vals[m] * D)
        else:                    # on the INT grid
            Di = D * f32(L.fp4q_ref_ifn_step(n))
            q = rng.integers(-top, top + 1, 16)
            q[0] = top
            xb = q.astype(np.float32) * Di
        rows.append(xb.astype(np.float32))
    x = np.stack(rows)
    got = ref.quantize(x, fmt=fmt, global_scale=float(S))
    y = ref.dequantize(got["codes"], got["scales"], float(S), *x.shape, fmt=fmt)
    assert np.array_equal(y, x)
    assert ref.error(x, got["codes"], got["scales"], float(S), fmt=fmt)[0] == 0.0


# ---- hand-worked blocks ---------------------------------------------------------

@pytest.mark.parametrize("key,n", [("if6_fp6_exact", 6), ("if6_int6_wins", 6), ("if3_fp3_exact", 3)])
def test_hand_worked_blocks(ref, key, n):
    g = json.load(open(GOLDEN))[key]
    fmt = ref.IF3 if n == 3 else ref.IF6
    x = np.array(g["x"], np.float32).reshape(1, 16)
    got = ref.quantize(x, fmt=fmt, global_scale=g["global_scale_given"], errors=True)
    assert list(got["scales"]) == g["scales"]
    assert list(ref.unpack_codes(got["codes"], fmt)) == g["element_codes"]
    assert list(got["codes"]) == g["codes"]
    assert got["best"][0] == g["block_error"]


def test_hand_worked_e2m0_ties(ref):
    g = json.load(open(GOLDEN))["fp3_ties_to_even_code"]
    assert [ref.lib().fp4q_ref_fpn_round(3, y) for y in g["y"]] == g["codes"]


def test_if6_int_step_below_2_pow_128(ref):
    # S at its floor 2^-117 and pattern 0x01: D = 2^-126, D_int = D*fl32(7.5/31)
    # is below 2^-128, so 1/D_int is +inf: zero elements stay INT code 0 and
    # every nonzero element saturates, on the oracle as in the exact statement
    S = 2.0 ** -117
    Di = f32(2.0 ** -126) * f32(ref.lib().fp4q_ref_ifn_step(6))
    assert Di < f32(2.0 ** -128) and np.isinf(np.float32(1.0) / Di)
    xb = np.zeros(16, np.float32)
    xb[1], xb[2], xb[5] = 3e-37, -1e-38, -0.0
    e, codes = ref.intn_block(6, xb, S, 0x01)
    assert list(codes[[0, 5]]) == [0, 0] and codes[1] == 31 and codes[2] == (-31) & 63
    we, wcodes = X.encode_intn(6, xb, S, 0x01)
    assert list(codes) == wcodes and e == float(we)
    got = ref.quantize(xb.reshape(1, 16), fmt=ref.IF6, global_scale=S)
    assert list(ref.unpack_codes(got["codes"], ref.IF6)) == X.quantize_block_ifn(6, xb, S)[1]
