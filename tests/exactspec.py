"""An independent, exact, tiny-input statement of the quantizer.

Used only by the tests to pin the C oracle.  It shares nothing with the
oracle: the formats are built from their bit-field definitions with exact
rationals, the binary32 steps of the scale computation are numpy.float32
operations, every rounding decision is an exhaustive nearest-value search in
exact rational arithmetic, and every error is an exact rational.  It is far
too slow for anything but a handful of blocks.
"""
from fractions import Fraction as Fr

import numpy as np

f32 = np.float32


def e2m1_grid():
    """The 8 non-negative E2M1 values, by code: 2 exponent bits (bias 1),
    1 mantissa bit, exponent field 0 subnormal."""
    vals = []
    for code in range(8):
        e, m = code >> 1, code & 1
        vals.append(Fr(m, 2) if e == 0 else (1 + Fr(m, 2)) * Fr(2) ** (e - 1))
    return vals


def e4m3_values():
    """Values of E4M3FN bytes 0x00..0x7E (0x7F is NaN): 4 exponent bits with
    bias 7, 3 mantissa bits, exponent field 0 subnormal."""
    vals = []
    for b in range(0x7F):
        e, m = b >> 3, b & 7
        vals.append(Fr(m, 8) * Fr(2) ** -6 if e == 0 else (1 + Fr(m, 8)) * Fr(2) ** (e - 7))
    return vals


E2M1 = e2m1_grid()
E4M3 = e4m3_values()


def nearest(y, grid):
    """Index of the value of `grid` (ascending) nearest to the rational y,
    the even index on an exact tie."""
    best, bd = 0, None
    for i, g in enumerate(grid):
        d = abs(y - g)
        if bd is None or d < bd or (d == bd and i % 2 == 0 and best % 2 == 1):
            best, bd = i, d
    return best


def global_scale(g):
    g = f32(g)
    if g == 0:
        return f32(1.0)
    s = g / f32(1536.0)
    return max(s, f32(2.0 ** -117))


def base_byte(a, S):
    t = f32(a) / (f32(6.0) * f32(S))
    b = nearest(Fr(float(t)), E4M3)
    return max(b, 1)


def encode_fp4(xb, S, c, w=None):
    """(exact error, nibbles) of one prepared block with scale byte c."""
    S = f32(S)
    D = f32(float(E4M3[c])) * S
    r = f32(1.0) / D
    err = Fr(0)
    nib = []
    for i, x in enumerate(xb):
        x = f32(x)
        a = abs(x)
        y = a * r
        m = nearest(Fr(float(y)), E2M1)
        xh = f32(float(E2M1[m])) * D
        e = (Fr(float(a)) - Fr(float(xh))) ** 2
        if w is not None:
            e *= Fr(float(f32(w[i])))
        err += e
        nib.append((8 if np.signbit(x) else 0) | m)
    return err, nib


def encode_int4(xb, S, c, w=None):
    S = f32(S)
    D = f32(float(E4M3[c])) * S
    Di = D * (f32(6.0) / f32(7.0))
    ri = f32(1.0) / Di
    err = Fr(0)
    nib = []
    for i, x in enumerate(xb):
        x = f32(x)
        a = abs(x)
        y = a * ri
        q = nearest(Fr(float(y)), [Fr(k) for k in range(8)])
        xh = f32(q) * Di
        e = (Fr(float(a)) - Fr(float(xh))) ** 2
        if w is not None:
            e *= Fr(float(f32(w[i])))
        err += e
        nib.append((-q if np.signbit(x) else q) & 0xF)
    return err, nib


def quantize_block_nvfp4(xb, S, sweep=None, w=None):
    """Returns (scale byte, nibbles, exact error, errors by candidate)."""
    a = max(abs(f32(v)) for v in xb)
    if a == 0:
        return 0, [(8 if np.signbit(f32(v)) else 0) for v in xb], Fr(0), {}
    sb = base_byte(a, S)
    if sweep is None:
        e, nib = encode_fp4(xb, S, sb, w)
        return sb, nib, e, {sb: e}
    lo, hi = sweep
    errs = {}
    for k in range(lo, hi + 1):
        c = min(0x7E, max(0x01, sb + k))
        if c not in errs:
            errs[c] = encode_fp4(xb, S, c, w)[0]
    cbest = min(errs, key=lambda c: (errs[c], c))
    e, nib = encode_fp4(xb, S, cbest, w)
    return cbest, nib, e, errs


def quantize_block_if4(xb, S, w=None):
    a = max(abs(f32(v)) for v in xb)
    if a == 0:
        return 0, [(8 if np.signbit(f32(v)) else 0) for v in xb], Fr(0)
    sb = base_byte(a, S)
    ef, nf = encode_fp4(xb, S, sb, w)
    ei, ni = encode_int4(xb, S, sb, w)
    if ei < ef:
        return sb | 0x80, ni, ei
    return sb, nf, ef


def quantize_block_mxfp4(xb):
    a = max(abs(f32(v)) for v in xb)
    if a == 0:
        e = -127
    else:
        # floor(log2 a) from the exact rational value
        q = Fr(float(a))
        e = 0
        while q >= 2:
            q /= 2
            e += 1
        while q < 1:
            q *= 2
            e -= 1
        e -= 2
    e = min(127, max(-127, e))
    D = Fr(2) ** e
    nib = []
    err = Fr(0)
    for x in xb:
        x = f32(x)
        av = Fr(float(abs(x)))
        m = nearest(av / D, E2M1)
        err += (av - E2M1[m] * D) ** 2
        nib.append((8 if np.signbit(x) else 0) | m)
    return e + 127, nib, err


def hadamard(n):
    """Sylvester Hadamard matrix (natural order), integer entries."""
    H = np.array([[1]], dtype=np.int64)
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H


def pack(nibbles):
    nib = list(nibbles)
    return bytes((nib[i] & 0xF) | ((nib[i + 1] & 0xF) << 4) for i in range(0, len(nib), 2))


def quantize_block_foursix(xb, S, w=None):
    """Four Over Six: the max onto 6 (AbsMax) or onto 4, lower exact error,
    a tie keeps 6."""
    a = max(abs(f32(v)) for v in xb)
    if a == 0:
        return 0, [(8 if np.signbit(f32(v)) else 0) for v in xb], Fr(0)
    s6 = base_byte(a, S)
    t4 = f32(a) / (f32(4.0) * f32(S))
    s4 = max(nearest(Fr(float(t4)), E4M3), 1)
    e6, n6 = encode_fp4(xb, S, s6, w)
    e4, n4 = encode_fp4(xb, S, s4, w)
    if e4 < e6:
        return s4, n4, e4
    return s6, n6, e6


def mx_encode(xb, e, w=None):
    D = Fr(2) ** e
    nib, err = [], Fr(0)
    for i, x in enumerate(xb):
        x = f32(x)
        av = Fr(float(abs(x)))
        m = nearest(av / D, E2M1)
        t = (av - E2M1[m] * D) ** 2
        if w is not None:
            t *= Fr(float(f32(w[i])))
        err += t
        nib.append((8 if np.signbit(x) else 0) | m)
    return err, nib


def quantize_block_mx_sweep(xb, window, w=None):
    e0 = quantize_block_mxfp4(xb)[0] - 127
    errs = {}
    for k in range(window[0], window[1] + 1):
        e = min(127, max(-127, e0 + k))
        if e not in errs:
            errs[e] = mx_encode(xb, e, w)[0]
    eb = min(errs, key=lambda e: (errs[e], e))
    err, nib = mx_encode(xb, eb, w)
    return eb + 127, nib, err


def quantize_block_if4_sweep(xb, S, window, w=None):
    a = max(abs(f32(v)) for v in xb)
    if a == 0:
        return 0, [(8 if np.signbit(f32(v)) else 0) for v in xb], Fr(0)
    sb = base_byte(a, S)
    opts = []
    seen = set()
    for k in range(window[0], window[1] + 1):
        c = min(0x7E, max(0x01, sb + k))
        if c in seen:
            continue
        seen.add(c)
        ef, nf = encode_fp4(xb, S, c, w)
        ei, ni = encode_int4(xb, S, c, w)
        opts.append((ef, c, c, nf))
        opts.append((ei, c + 0.5, c | 0x80, ni))   # INT4 after FP4 of the same pattern
    e, _, byte, nib = min(opts, key=lambda o: (o[0], o[1]))
    return byte, nib, e


def relaxed_block(xb, S, coefs, byte=None, fmt="nvfp4"):
    """FOCUS deploy encode of one block: codes from D*c, S_dq (byte) stored."""
    a = max(abs(f32(v)) for v in xb)
    if byte is None:
        if fmt == "mxfp4":
            byte = quantize_block_mxfp4(xb)[0]
        else:
            byte = 0 if a == 0 else base_byte(a, S)
    if fmt == "mxfp4":
        D = f32(2.0 ** (byte - 127))
    else:
        D = f32(float(E4M3[byte])) * f32(S) if byte else f32(0)
    nib = []
    for x, c in zip(xb, coefs):
        x = f32(x)
        m = 0
        if D != 0 and x != 0:  # |x| / S_q = 0 for a zero element
            Dq = D * f32(c)
            with np.errstate(divide="ignore", over="ignore"):
                rq = f32(1.0) / Dq  # +inf when D_q < 2^-128: every nonzero element saturates
                y = abs(x) * rq
            m = 7 if np.isinf(y) else nearest(Fr(float(y)), E2M1)
        nib.append((8 if np.signbit(x) else 0) | m)
    return byte, nib


# ---- the n-bit adaptive types (IF3, IF6; n = 4 is IF4) ---------------------
# The FP element of an n-bit type is E2M(n-3): sign, two exponent bits with
# bias 1, n-3 mantissa bits, exponent field 0 subnormal; the INT element an
# integer in [-(2^(n-1)-1), 2^(n-1)-1] with step D * fl32(FPmax/INTmax).

def fpn_grid(n):
    """The 2^(n-1) non-negative E2M(n-3) values, by magnitude code, from the
    bit fields (exponent e = code >> (n-3), mantissa f = the low n-3 bits)."""
    k = n - 3
    vals = []
    for code in range(1 << (n - 1)):
        e, f = code >> k, code & ((1 << k) - 1)
        frac = Fr(f, 1 << k)
        vals.append(frac if e == 0 else (1 + frac) * Fr(2) ** (e - 1))
    return vals


def ifn_step(n):
    grid = fpn_grid(n)
    return f32(float(grid[-1])) / f32((1 << (n - 1)) - 1)


def ifn_global_scale(n, g):
    g = f32(g)
    if g == 0:
        return f32(1.0)
    s = g / (f32(256.0) * f32(float(fpn_grid(n)[-1])))
    return max(s, f32(2.0 ** -117))


def ifn_base_byte(n, a, S):
    t = f32(a) / (f32(float(fpn_grid(n)[-1])) * f32(S))
    return max(nearest(Fr(float(t)), E4M3), 1)


def encode_fpn(n, xb, S, c, w=None):
    """(exact error, codes) of the FP branch with scale byte c."""
    grid = fpn_grid(n)
    S = f32(S)
    D = f32(float(E4M3[c])) * S
    r = f32(1.0) / D
    err, codes = Fr(0), []
    for i, x in enumerate(xb):
        x = f32(x)
        a = abs(x)
        y = a * r
        m = nearest(Fr(float(y)), grid)
        xh = f32(float(grid[m])) * D
        e = (Fr(float(a)) - Fr(float(xh))) ** 2
        if w is not None:
            e *= Fr(float(f32(w[i])))
        err += e
        codes.append(((1 << (n - 1)) if np.signbit(x) else 0) | m)
    return err, codes


def encode_intn(n, xb, S, c, w=None):
    top = (1 << (n - 1)) - 1
    S = f32(S)
    D = f32(float(E4M3[c])) * S
    Di = D * ifn_step(n)
    with np.errstate(divide="ignore", over="ignore"):
        ri = f32(1.0) / Di
    err, codes = Fr(0), []
    for i, x in enumerate(xb):
        x = f32(x)
        a = abs(x)
        if a == 0:
            q = 0   # |x| / D_int = 0, also where 1 / D_int overflows to inf
        else:
            with np.errstate(over="ignore"):
                y = a * ri
            q = top if np.isinf(y) else nearest(Fr(float(y)), [Fr(k) for k in range(top + 1)])
        xh = f32(q) * Di
        e = (Fr(float(a)) - Fr(float(xh))) ** 2
        if w is not None:
            e *= Fr(float(f32(w[i])))
        err += e
        codes.append((-q if np.signbit(x) else q) & ((1 << n) - 1))
    return err, codes


def quantize_block_ifn(n, xb, S, window=(0, 0), w=None):
    """(scale byte, codes, exact error): per pattern of the window the FP
    grid, then the INT grid; the first least error wins."""
    a = max(abs(f32(v)) for v in xb)
    if a == 0:
        return 0, [((1 << (n - 1)) if np.signbit(f32(v)) else 0) for v in xb], Fr(0)
    sb = ifn_base_byte(n, a, S)
    opts, seen = [], set()
    for k in range(window[0], window[1] + 1):
        c = min(0x7E, max(0x01, sb + k))
        if c in seen:
            continue
        seen.add(c)
        ef, cf = encode_fpn(n, xb, S, c, w)
        ei, ci = encode_intn(n, xb, S, c, w)
        opts.append((ef, 2 * len(opts), c, cf))
        opts.append((ei, 2 * len(opts) + 1, c | 0x80, ci))
    e, _, byte, codes = min(opts, key=lambda o: (o[0], o[1]))
    return byte, codes, e


def pack_bits(codes, n):
    """Code stream of n-bit codes: code i at bits n i .. n i + n - 1, least
    significant bit first."""
    total = 0
    for i, c in enumerate(codes):
        total |= (int(c) & ((1 << n) - 1)) << (n * i)
    nbytes = (len(codes) * n + 7) // 8
    return bytes((total >> (8 * b)) & 0xFF for b in range(nbytes))
