"""The kernels' integer-code shortcuts, pinned on the CPU against the plain
statement of the codes.

The quantize kernels do not round and convert element by element when they
form INT codes; they add 1.5 2^23 to the binary32 product (the binary32 ulp
there is 1, so the sum holds the product rounded to the nearest integer, ties
to even, with the sign of x) and read the code from the sum's low mantissa
bits.  Each test rebuilds one such sequence in numpy binary32 and compares it,
element by element, with the method's definition written directly: the codes
of the rounded product min(RNE(fl32(|x| r)), INTmax) with the sign of x.

- IF3 / IF6 INT codes (Adaptive Block-Scaled Data Types, Methodology, at 3
  and 6 bits under the reading stated in include/fp4q.h): the n-bit two's
  complement of the signed integer.
- IF4 INT4 nibbles (same page, Methodology): q + 8 as a byte, whose XOR with
  8 is the two's complement nibble.
- IF3 FP codes (E2M0, magnitudes {0, 1, 2, 4}): the magnitude code from the
  same kind of sum, the sign in bit 2.
"""
import numpy as np
import pytest

f32 = np.float32
M = f32(12582912.0)            # 1.5 2^23


def products(seed, n=200_000):
    """(x, r) pairs over the cases that matter: random magnitudes, exact
    ties k + 1/2 of both signs, zeros of both signs, values far past the
    saturation point, and tiny values."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(n) * np.exp2(rng.integers(-8, 8, n))).astype(f32)
    r = np.exp2(rng.integers(-6, 7, n)).astype(f32) * f32(1.0) / f32(1.125) ** rng.integers(0, 8, n)
    r = r.astype(f32)
    # exact ties: x r = +-(k + 1/2) with r a power of two
    k = rng.integers(0, 40, 4000)
    e = rng.integers(-4, 5, 4000)
    rt = np.exp2(e).astype(f32)
    xt = ((k + 0.5) / rt * np.where(rng.integers(0, 2, 4000) == 1, 1, -1)).astype(f32)
    # one binary32 step either side of those ties
    xs = np.concatenate([xt, np.nextafter(xt, f32(np.inf)), np.nextafter(xt, f32(-np.inf))])
    rs = np.concatenate([rt, rt, rt])
    special = np.array([0.0, -0.0, 1e30, -1e30, 1e-30, -1e-30, 2.0 ** -149, -(2.0 ** -149)], f32)
    x = np.concatenate([x, xs, special])
    r = np.concatenate([r, rs, np.full(special.size, f32(0.75))])
    return x.astype(f32), r.astype(f32)


def plain_signed_int(x, r, top):
    """sign(x) min(RNE(fl32(|x| r)), top) as int64 (the method's INT value)."""
    y = (np.abs(x) * r).astype(f32)
    q = np.minimum(np.rint(y.astype(np.float64)), top).astype(np.int64)
    return np.where(np.signbit(x), -q, q)


def magic_sum(x, r, top):
    """fl32(fl32(x r) + 1.5 2^23) clamped to 1.5 2^23 +- top (one med3)."""
    z = (x * r).astype(f32)
    t = (z + M).astype(f32)
    return np.clip(t, M - f32(top), M + f32(top)).astype(f32)


@pytest.mark.parametrize("n", [3, 6])
def test_ifn_int_codes(n):
    top = (1 << (n - 1)) - 1
    x, r = products(10 + n)
    got = magic_sum(x, r, top).view(np.uint32) & np.uint32((1 << n) - 1)
    want = (plain_signed_int(x, r, top) & ((1 << n) - 1)).astype(np.uint32)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (x[bad[:5]], r[bad[:5]], got[bad[:5]], want[bad[:5]])


def test_if4_int4_nibbles():
    x, r = products(14)
    for clamp in (True, False):
        if clamp:
            t = magic_sum(x, r, 7)
            xx, rr = x, r
        else:
            # the unclamped form is used only where |x| r stays below 7.5
            keep = (np.abs(x) * r).astype(f32) < f32(7.5)
            xx, rr = x[keep], r[keep]
            t = ((xx * rr).astype(f32) + M).astype(f32)
        q8 = (t - (M - f32(8))).astype(f32)          # q + 8, one byte each
        assert np.all((q8 >= 1) & (q8 <= 15) & (q8 == np.floor(q8)))
        nib = (q8.astype(np.uint32) ^ np.uint32(8)) & np.uint32(15)
        want = (plain_signed_int(xx, rr, 7) & 15).astype(np.uint32)
        assert np.array_equal(nib, want)
        # and the term's q: t - 1.5 2^23 is the signed integer itself
        assert np.array_equal((t - M).astype(np.int64), plain_signed_int(xx, rr, 7))


def e2m0_plain(y):
    """Magnitude code of the nearest of {0, 1, 2, 4} to y >= 0, ties to the
    even code, saturating at 4 -- by exhaustive comparison in binary64."""
    grid = np.array([0.0, 1.0, 2.0, 4.0])
    d = np.abs(y.astype(np.float64)[:, None] - grid)
    m = d.min(1, keepdims=True)
    tie = d == m
    even = tie & (np.arange(4) % 2 == 0)
    k = np.where(even.any(1), even.argmax(1), tie.argmax(1))
    # at and beyond 4 the nearest is 4 (and the binary64 distances above
    # would round to ties for huge y)
    return np.where(y >= 4, 3, k).astype(np.uint32)


def test_if3_fp_codes():
    x, r = products(15)
    # midpoints 0.5, 1.5, 3 of the E2M0 grid and their neighbours as products
    mids = np.array([0.5, 1.5, 3.0, 2.5, 3.5, 5.0], f32)
    xm = np.concatenate([mids, np.nextafter(mids, f32(0)), np.nextafter(mids, f32(9))])
    x = np.concatenate([x, xm, -xm])
    r = np.concatenate([r, np.ones(2 * xm.size, f32)])
    y = (np.abs(x) * r).astype(f32)
    t = np.where(y > f32(3), f32(2.0 ** 23 + 3),
                 np.minimum((y + f32(2.0 ** 23)).astype(f32), f32(2.0 ** 23) + f32(2)))
    t = t.astype(f32)
    xb = x.view(np.uint32)
    got = (t.view(np.uint32) & np.uint32(3)) | ((xb >> np.uint32(29)) & ~np.uint32(3))
    want = e2m0_plain(y) | (np.signbit(x).astype(np.uint32) << np.uint32(2))
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (x[bad[:5]], y[bad[:5]], got[bad[:5]], want[bad[:5]])


def fpn_value_kernel(n, y):
    """The kernels' FP rounding of y >= 0 through magic constants: E2M3
    adds 2^20 / 2^21 / 2^22 below 2 / 4 / above (the binary32 ulp there is the
    E2M3 step) and saturates at 7.5; E2M0 takes min(RNE(y), 2) up to 3 and 4
    above."""
    if n == 6:
        m = np.where(y < 2, f32(2.0 ** 20), np.where(y < 4, f32(2.0 ** 21), f32(2.0 ** 22)))
        return np.minimum(((y + m).astype(f32) - m).astype(f32), f32(7.5))
    q = np.minimum(((y + f32(2.0 ** 23)).astype(f32) - f32(2.0 ** 23)).astype(f32), f32(2))
    return np.where(y > 3, f32(4), q).astype(f32)


def fpn_value_plain(n, y):
    """Nearest value of the E2M3 (n = 6) or E2M0 (n = 3) magnitudes, ties to
    the even code, saturating -- by exhaustive comparison in binary64."""
    if n == 6:
        grid = np.array([m / 8 for m in range(8)] + [2.0 ** (e - 1) * (1 + f / 8)
                                                     for e in (1, 2, 3) for f in range(8)])
    else:
        grid = np.array([0.0, 1.0, 2.0, 4.0])
    yy = np.minimum(y.astype(np.float64), grid[-1] + 1.0)     # far past the top: top
    d = np.abs(yy[:, None] - grid)
    m = d.min(1, keepdims=True)
    tie = d == m
    even = tie & (np.arange(grid.size) % 2 == 0)
    k = np.where(even.any(1), even.argmax(1), tie.argmax(1))
    return grid[k].astype(f32)


@pytest.mark.parametrize("n", [3, 6])
def test_fpn_rounding(n):
    rng = np.random.default_rng(20 + n)
    y = np.abs(rng.standard_normal(200_000) * 3).astype(f32)
    top = 7.5 if n == 6 else 4.0
    if n == 6:
        grid = np.array([m / 8 for m in range(8)] + [2.0 ** (e - 1) * (1 + f / 8)
                                                     for e in (1, 2, 3) for f in range(8)], f32)
    else:
        grid = np.array([0.0, 1.0, 2.0, 4.0], f32)
    mids = ((grid[1:].astype(np.float64) + grid[:-1]) / 2).astype(f32)
    y = np.concatenate([y, grid, mids, np.nextafter(mids, f32(0)), np.nextafter(mids, f32(99)),
                        np.array([top + 0.5, 2 * top, 1e30, 2.0 ** -149], f32)])
    got = fpn_value_kernel(n, y)
    want = fpn_value_plain(n, y)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (y[bad[:5]], got[bad[:5]], want[bad[:5]])


def e4m3_round_kernel(t):
    """The kernels' E4M3 rounding of t >= 0 (pattern, ties to even,
    saturating at 448 = 0x7E): scaled RNE below 2^-6, otherwise rounding the
    23-bit mantissa to 3 bits with one integer add."""
    t = t.astype(f32)
    u = t.view(np.uint32).astype(np.uint64)
    u = u + np.uint64(0x7FFFF) + ((u >> np.uint64(20)) & np.uint64(1))
    normal = ((u >> np.uint64(20)) - np.uint64(120 << 3)).astype(np.int64)
    ts = np.minimum(t, f32(2.0 ** -6))                    # the subnormal branch's inputs
    sub = np.rint((ts * f32(512)).astype(f32).astype(np.float64)).astype(np.int64)
    return np.where(t >= 448, 0x7E, np.where(t < 2.0 ** -6, sub, normal))


def e4m3_round_plain(t):
    vals = np.array([(m / 8) * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
                     for e in range(16) for m in range(8)][:0x7F])
    tt = np.minimum(t.astype(np.float64), 448.0)
    d = np.abs(tt[:, None] - vals)
    m = d.min(1, keepdims=True)
    tie = d == m
    even = tie & (np.arange(vals.size) % 2 == 0)
    return np.where(even.any(1), even.argmax(1), tie.argmax(1))


def test_e4m3_rounding():
    rng = np.random.default_rng(30)
    vals = np.array([(m / 8) * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
                     for e in range(16) for m in range(8)][:0x7F], f32)
    mids = ((vals[1:].astype(np.float64) + vals[:-1]) / 2).astype(f32)
    t = np.concatenate([np.exp2(rng.uniform(-12, 10, 100_000)).astype(f32), vals, mids,
                        np.nextafter(mids, f32(0)), np.nextafter(mids, f32(1e9)),
                        np.array([0.0, 2.0 ** -149, 2.0 ** -10, 447.9, 448.0, 464.0, 480.0, 1e30], f32)])
    got = e4m3_round_kernel(t)
    want = e4m3_round_plain(t)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (t[bad[:5]], got[bad[:5]], want[bad[:5]])


def e2m1_kernel(y):
    m = np.where(y < 2, f32(2.0 ** 22), np.where(y < 4, f32(2.0 ** 23), f32(2.0 ** 24)))
    return np.minimum(((y + m).astype(f32) - m).astype(f32), f32(6))


def test_e2m1_rounding():
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], f32)
    mids = ((grid[1:].astype(np.float64) + grid[:-1]) / 2).astype(f32)
    rng = np.random.default_rng(31)
    y = np.concatenate([np.abs(rng.standard_normal(200_000) * 3).astype(f32), grid, mids,
                        np.nextafter(mids, f32(0)), np.nextafter(mids, f32(99)),
                        np.array([6.5, 7.0, 100.0, 1e30, 2.0 ** -149], f32)])
    yy = np.minimum(y.astype(np.float64), 7.0)
    d = np.abs(yy[:, None] - grid)
    m = d.min(1, keepdims=True)
    tie = d == m
    even = tie & (np.arange(8) % 2 == 0)
    want = grid[np.where(even.any(1), even.argmax(1), tie.argmax(1))]
    got = e2m1_kernel(y)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (y[bad[:5]], got[bad[:5]], want[bad[:5]])
