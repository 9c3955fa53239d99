"""The certification bound of the binary32 candidate estimates, pinned on the CPU.

The quantize kernels pick a scale from binary32 estimates of each candidate's
block error and accept the pick only when the two least estimates are further
apart than a bound T on |binary64 error - estimate|.  The pick is then the
binary64 argmin whenever T really bounds that difference.  This test rebuilds
the estimates with the kernels' operation sequence in numpy binary32 (fused
multiply-adds through extended precision, E2M1 rounding by an exact nearest
search) and checks the bound against the oracle's binary64 errors for every
(block, candidate) on adversarial inputs: heavy tails, tiny and huge global
scales, weights spread over many decades, saturated and on-grid blocks.
"""
import numpy as np
import pytest


f32, f64, fx = np.float32, np.float64, np.longdouble
U = 2.0 ** -24
GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e4m3_values():
    v = []
    for b in range(0x7F):
        e, m = b >> 3, b & 7
        v.append(m / 8 * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    return np.array(v, f32)


E4M3 = e4m3_values()


def e2m1(y):
    """Signed nearest E2M1 value (ties to the even code, saturating at 6) by
    exhaustive comparison in binary64 (exact for binary32 inputs)."""
    a = np.abs(y.astype(f64))
    d = np.abs(a[..., None] - GRID)
    m = d.min(-1, keepdims=True)
    tie = d == m
    even = tie & (np.arange(8) % 2 == 0)
    k = np.where(even.any(-1), even.argmax(-1), tie.argmax(-1))
    return np.copysign(GRID[k], y).astype(f32)


def fma32(x, y, z):
    """fl32(x*y + z) through extended precision (x*y exact in 64 bits)."""
    return (fx(x) * fx(y) + fx(z)).astype(f32)


def estimate(v, w, S, c, mse):
    """The kernels' estimate for pattern c (array over blocks), in units of
    S^2, and the pattern eight steps up from the same products."""
    s = E4M3[c]
    D = (s * f32(S)).astype(f32)
    r = (f32(1) / D).astype(f32)
    y = (v * r[:, None]).astype(f32)
    q = e2m1(y)
    h = (f32(2) * e2m1((y * f32(0.5)).astype(f32))).astype(f32)   # code of y/2, decoded x2
    b = np.sqrt(w).astype(f32)
    F1 = np.zeros(v.shape[0], f32)
    F2 = np.zeros(v.shape[0], f32)
    for i in range(16):
        if mse:
            d1 = (y[:, i] - q[:, i]).astype(f32)
            d2 = (y[:, i] - h[:, i]).astype(f32)
        else:
            by = (b[:, i] * y[:, i]).astype(f32)
            d1 = fma32(-b[:, i], q[:, i], by)
            d2 = fma32(-b[:, i], h[:, i], by)
        F1 = fma32(d1, d1, F1)
        F2 = fma32(d2, d2, F2)
    ss = (s * s).astype(f32)
    return (F1 * ss).astype(f32), (F2 * ss).astype(f32)


def bound(E, A, W, rel):
    E = E.astype(f64)
    return 16 * U * A * np.sqrt(W * E) * 1.0001 + rel * E + 64 * U * U * A * A * W


def window_estimates(ref, v, w, S, lo, hi, mse):
    """Per block: the window's patterns, the kernels' estimates of each (from
    the pair-shared products where a pattern eight steps up is in the window
    too), A and W of the bound, and the oracle's binary64 errors / S^2."""
    nb = v.shape[0]
    a = np.abs(v).max(1)
    t = (a / (f32(6) * f32(S))).astype(f32)
    sb = np.array([max(1, ref.lib().fp4q_ref_e4m3_round(f32(x))) for x in t])
    W = np.full(nb, 16.0)
    if not mse:
        Wf = np.zeros(nb, f32)
        for i in range(16):
            Wf = (Wf + w[:, i]).astype(f32)
        W = Wf.astype(f64)
    invS = f32(1) / f32(S)
    ctop = np.clip(sb + hi, 1, 0x7E)
    A = np.maximum(a.astype(f64) * f64(invS) * (1 + 4 * U), 6 * E4M3[ctop].astype(f64)) * (1 + 4 * U)
    pats, ests = [], []
    for k in range(lo, hi + 1):
        c = sb + k
        if k - 8 >= lo:
            # this pattern is the upper member of the pair (c - 8, c)
            base = np.clip(c - 8, 1, 0x7E)
            e = estimate(v, w, S, base, mse)[1]
        else:
            e = estimate(v, w, S, np.clip(c, 1, 0x7E), mse)[0]
        pats.append(c)
        ests.append(e)
    P = np.stack(pats, 1)
    Est = np.stack(ests, 1).astype(f64)
    E64 = ref.candidate_errors(v, S, None if mse else w, nthreads=8) / (f64(S) * f64(S))
    valid = (P >= 1) & (P <= 0x7E) & ((P - 8 >= 1) | (np.arange(lo, hi + 1) - 8 < lo))
    ex = np.take_along_axis(E64, np.clip(P, 1, 0x7E), 1)
    return P, Est, ex, A, W, valid


def check(ref, v, w, S, lo, hi, mse, rel=32 * U):
    """max over (block, candidate) of |E64/S^2 - estimate| / T; must be <= 1."""
    P, Est, ex, A, W, valid = window_estimates(ref, v, w, S, lo, hi, mse)
    T = bound(Est, A[:, None], W[:, None], rel)
    sel = valid & np.isfinite(Est) & np.isfinite(ex)
    assert sel.mean() > 0.5
    return float((np.abs(ex[sel] - Est[sel]) / T[sel]).max())


def student(rows, seed, scale=0.02, df=4):
    return (np.random.default_rng(seed).standard_t(df, (rows, 16)) * scale).astype(np.float32)


@pytest.mark.parametrize("mse", [True, False])
def test_bound_heavy_tails(ref, mse):
    v = student(4000, 1)
    w = np.random.default_rng(2).lognormal(0, 1, (4000, 16)).astype(np.float32)
    S = ref.lib().fp4q_ref_global_scale(f32(np.abs(v).max()))
    assert check(ref, v, w, S, -8, 7, mse) <= 1.0


@pytest.mark.parametrize("scale", [1e-30, 1e-20, 1e-12, 1e12, 1e30])
def test_bound_extreme_scales_and_weights(ref, scale):
    v = student(1500, 3, scale=scale)
    w = np.random.default_rng(4).lognormal(0, 4, (1500, 16)).astype(np.float32)
    S = ref.lib().fp4q_ref_global_scale(f32(np.abs(v).max()))
    assert check(ref, v, w, S, -8, 7, False) <= 1.0
    assert check(ref, v, w, S, -3, 7, True) <= 1.0


def test_bound_saturation_and_grid_blocks(ref):
    rng = np.random.default_rng(5)
    v = rng.uniform(-1, 1, (2000, 16)).astype(np.float32)
    v[:500] = np.round(v[:500] * 12) / 2          # on a 0.5 grid: many exact errors
    v[500:1000, 0] *= 40                          # one dominant element
    v[1000:1500] = np.float32(1.0)                # constant blocks (exact ties)
    w = rng.lognormal(0, 2, (2000, 16)).astype(np.float32)
    S = ref.lib().fp4q_ref_global_scale(f32(np.abs(v).max()))
    for mse in (True, False):
        assert check(ref, v, w, S, -8, 7, mse) <= 1.0
    # a given global scale far from the data's own
    assert check(ref, v, w, f32(1e-3), -8, 7, False) <= 1.0


def test_bound_is_not_vacuous(ref):
    # tight enough to decide: on c2-like blocks the two least estimates of
    # the [-8, 7] window separate by more than their bounds for > 99% of blocks
    v = student(3000, 6)
    w = np.random.default_rng(7).lognormal(0, 1, (3000, 16)).astype(np.float32)
    S = ref.lib().fp4q_ref_global_scale(f32(np.abs(v).max()))
    P, Est, ex, A, W, valid = window_estimates(ref, v, w, S, -8, 7, False)
    keep = valid.all(1)              # the whole window on finite patterns (the fast path's blocks)
    assert keep.mean() > 0.9
    P, Est, ex, A, W = P[keep], Est[keep], ex[keep], A[keep], W[keep]
    srt = np.sort(Est, 1)
    e1, e2 = srt[:, 0], srt[:, 1]
    t1, t2 = bound(e1, A, W, 64 * U), bound(e2, A, W, 64 * U)
    certified = e2 - t2 > e1 + t1
    assert certified.mean() > 0.99
    # and where certified, the estimated argmin is the binary64 argmin
    pick = P[np.arange(len(P)), Est.argmin(1)]
    exact = P[np.arange(len(P)), ex.argmin(1)]
    assert np.array_equal(pick[certified], exact[certified])


def int4_estimate(v, w, S, c, mse):
    """IF4's INT4 estimate at pattern c in units of S^2 (the single-pattern
    IF4 kernel): q = min(RNE(fl(|x| ri)), 7), the method's integer."""
    s = E4M3[c]
    D = (s * f32(S)).astype(f32)
    Di = (D * f32(6.0 / 7.0)).astype(f32)
    ri = (f32(1) / Di).astype(f32)
    z = (np.abs(v) * ri[:, None]).astype(f32)
    q = np.minimum(np.rint(z), f32(7)).astype(f32)
    b = np.sqrt(w).astype(f32)
    F = np.zeros(v.shape[0], f32)
    for i in range(16):
        if mse:
            d = (z[:, i] - q[:, i]).astype(f32)
        else:
            d = fma32(-b[:, i], q[:, i], (b[:, i] * z[:, i]).astype(f32))
        F = fma32(d, d, F)
    sz = (s * f32(6.0 / 7.0)).astype(f32)
    return (F * (sz * sz).astype(f32)).astype(f32)


def int4_estimate_magic(v, w, S, c, mse, clamp=True):
    """The IF4 window kernel's INT4 estimate at pattern c in units of S^2:
    t = fl(|x| ri + 1.5 2^23) rounds the exact product p = |x| ri to the
    nearest integer (ties to even), q = t - 1.5 2^23 (saturated at 7 when
    clamp), d = fl(p - q) with one rounding.  p is exact in binary64 (two
    24-bit factors), so RNE(p) and p - q are exact there too."""
    s = E4M3[c]
    D = (s * f32(S)).astype(f32)
    Di = (D * f32(6.0 / 7.0)).astype(f32)
    ri = (f32(1) / Di).astype(f32)
    p = np.abs(v).astype(f64) * ri.astype(f64)[:, None]
    q = np.rint(p)
    if clamp:
        q = np.minimum(q, 7.0)
    d = (p - q).astype(f32)
    b = np.sqrt(w).astype(f32)
    F = np.zeros(v.shape[0], f32)
    for i in range(16):
        e = d[:, i] if mse else (b[:, i] * d[:, i]).astype(f32)
        F = fma32(e, e, F)
    sz = (s * f32(6.0 / 7.0)).astype(f32)
    return (F * (sz * sz).astype(f32)).astype(f32)


def int4_window_blocks(ref, seed):
    """Uniform and heavy-tailed blocks, plus blocks whose maximum sits just
    below an E4M3 rounding boundary of max/(6S) (the largest |x| r_int for
    the pattern s_base and the ones above it), with their S and s_base."""
    rng = np.random.default_rng(seed)
    v = np.concatenate([rng.uniform(-1, 1, (300, 16)), student(300, seed + 1, scale=0.1)]).astype(np.float32)
    L = ref.lib()
    S = L.fp4q_ref_global_scale(f32(np.abs(v).max()))
    # push each of 200 blocks' maximum to just below the midpoint above its
    # E4M3 pattern (normal and subnormal patterns alike)
    extra = rng.uniform(-1, 1, (200, 16)).astype(np.float32) * f32(0.01)
    for i in range(200):
        pat = int(rng.integers(1, 0x7D))
        mid = (float(E4M3[pat]) + float(E4M3[pat + 1])) / 2 * 6 * float(S)
        m = np.nextafter(f32(mid), f32(0))
        for _ in range(int(rng.integers(0, 4))):
            m = np.nextafter(m, f32(0))
        extra[i] *= float(m)
        extra[i, int(rng.integers(0, 16))] = m * (1 if rng.random() < 0.5 else -1)
    v = np.concatenate([v, extra]).astype(np.float32)
    a = np.abs(v).max(1)
    sb = np.array([max(1, L.fp4q_ref_e4m3_round(f32(x))) for x in (a / (f32(6) * f32(S))).astype(f32)])
    return v, S, a, sb


def test_int4_saturation_only_below_s_base(ref):
    # the window kernel skips the saturation at 7 for patterns above s_base,
    # and at s_base itself when s_base is normal and not the top pattern: there
    # every |x| r_int stays below 7.5, so min(RNE(|x| r_int), 7) = RNE(|x| r_int)
    v, S, a, sb = int4_window_blocks(ref, 21)
    for k in range(0, 8):
        c = sb + k
        ok = (c <= 0x7E) & ((k > 0) | ((sb >= 8) & (sb < 0x7E)))
        D = (E4M3[np.minimum(c, 0x7E)] * f32(S)).astype(f32)
        ri = (f32(1) / (D * f32(6.0 / 7.0)).astype(f32)).astype(f32)
        p = a.astype(f64) * ri.astype(f64)
        assert p[ok].max() < 7.5
        if k > 0:
            assert p[ok].max() < 7.0
    # and below s_base saturation does occur (the clamp is needed there)
    c = np.maximum(sb - 1, 1)
    ri = (f32(1) / ((E4M3[c] * f32(S)).astype(f32) * f32(6.0 / 7.0)).astype(f32)).astype(f32)
    assert (a.astype(f64) * ri.astype(f64)).max() >= 7.5


@pytest.mark.parametrize("mse", [True, False])
def test_bound_int4_window_estimate(ref, mse):
    # the window kernel's INT4 estimates (rounding through 1.5 2^23), clamped
    # below s_base and not above, against the oracle's binary64 INT4 errors
    v, S, a, sb = int4_window_blocks(ref, 23)
    rng = np.random.default_rng(24)
    w = rng.lognormal(0, 2, v.shape).astype(np.float32)
    W = np.full(len(v), 16.0)
    if not mse:
        Wf = np.zeros(len(v), f32)
        for i in range(16):
            Wf = (Wf + w[:, i]).astype(f32)
        W = Wf.astype(f64)
    worst = 0.0
    for k in range(-3, 8):
        c = np.clip(sb + k, 1, 0x7E)
        real = (sb + k >= 1) & (sb + k <= 0x7E)
        ctop = np.clip(sb + 7, 1, 0x7E)
        A = np.maximum(a.astype(f64) * f64(f32(1) / f32(S)) * (1 + 4 * U),
                       6 * E4M3[ctop].astype(f64)) * (1 + 4 * U)
        E = int4_estimate_magic(v, w, S, c, mse).astype(f64)
        if k > 0:
            # the kernel's unclamped form (above s_base) agrees wherever it is used
            Eu = int4_estimate_magic(v, w, S, c, mse, clamp=False).astype(f64)
            assert np.array_equal(E[real], Eu[real])
        ex = np.array([ref.int4_block(v[i], S, int(c[i]), None if mse else w[i])[0] for i in range(len(v))])
        ex = ex / (f64(S) * f64(S))
        worst = max(worst, float((np.abs(ex - E) / bound(E, A, W, 40 * U)).max()))
    assert worst <= 1.0


@pytest.mark.parametrize("mse", [True, False])
def test_bound_int4_candidates(ref, mse):
    # IF4's INT4 candidates over a window, with the 40u relative term
    rng = np.random.default_rng(8)
    v = np.concatenate([rng.uniform(-1, 1, (300, 16)), student(300, 9, scale=0.1)]).astype(np.float32)
    w = rng.lognormal(0, 2, (600, 16)).astype(np.float32)
    S = ref.lib().fp4q_ref_global_scale(f32(np.abs(v).max()))
    a = np.abs(v).max(1)
    sb = np.array([max(1, ref.lib().fp4q_ref_e4m3_round(f32(x))) for x in (a / (f32(6) * f32(S))).astype(f32)])
    W = np.full(len(v), 16.0)
    if not mse:
        Wf = np.zeros(len(v), f32)
        for i in range(16):
            Wf = (Wf + w[:, i]).astype(f32)
        W = Wf.astype(f64)
    worst = 0.0
    for k in range(-3, 8):
        c = np.clip(sb + k, 1, 0x7E)
        ctop = np.clip(sb + 7, 1, 0x7E)
        A = np.maximum(a.astype(f64) * f64(f32(1) / f32(S)) * (1 + 4 * U),
                       6 * E4M3[ctop].astype(f64)) * (1 + 4 * U)
        E = int4_estimate(v, w, S, c, mse).astype(f64)
        ex = np.array([ref.int4_block(v[i], S, int(c[i]), None if mse else w[i])[0] for i in range(len(v))])
        ex = ex / (f64(S) * f64(S))
        worst = max(worst, float((np.abs(ex - E) / bound(E, A, W, 40 * U)).max()))
    assert worst <= 1.0


def mx_estimate(v, w, el, j, mse):
    """The MXFP4 window's estimate of exponent el + j in units of 2^(2 el)."""
    y = (v * np.ldexp(f32(1), -el)[:, None].astype(f32)).astype(f32)
    P = f32(2.0 ** j)
    q = (P * e2m1((y / P).astype(f32))).astype(f32)
    b = np.sqrt(w).astype(f32)
    F = np.zeros(v.shape[0], f32)
    for i in range(32):
        d = (y[:, i] - q[:, i]).astype(f32) if mse else fma32(-b[:, i], q[:, i], (b[:, i] * y[:, i]).astype(f32))
        F = fma32(d, d, F)
    return F


@pytest.mark.parametrize("mse", [True, False])
def test_bound_mxfp4_window(ref, mse):
    # E8M0 steps are powers of two, so y and every reconstruction are exact;
    # the binary64 error is computed directly from the exact reconstruction
    rng = np.random.default_rng(10)
    v = (rng.standard_normal((800, 32)) * np.where(rng.random((800, 32)) < 0.05, 50, 1)).astype(np.float32)
    w = rng.lognormal(0, 2, (800, 32)).astype(np.float32)
    a = np.abs(v).max(1)
    e0 = np.floor(np.log2(a.astype(f64))).astype(int) - 2
    lo, hi = -1, 2
    el = e0 + lo
    W = np.full(len(v), 32.0)
    if not mse:
        Wf = np.zeros(len(v), f32)
        for i in range(32):
            Wf = (Wf + w[:, i]).astype(f32)
        W = Wf.astype(f64)
    K = hi - lo + 1
    A = np.maximum(a.astype(f64) * np.ldexp(1.0, -el), 6 * 2.0 ** (K - 1)) * (1 + 4 * U)
    worst = 0.0
    for j in range(K):
        E = mx_estimate(v, w, el, j, mse).astype(f64)
        e = el + j
        xh = np.abs(e2m1((v * np.ldexp(f32(1), -e)[:, None].astype(f32)).astype(f32))).astype(f64) \
            * np.ldexp(1.0, e)[:, None]
        t = (np.abs(v).astype(f64) - xh) ** 2
        if not mse:
            t = t * w.astype(f64)
        ex = t.sum(1) / np.ldexp(1.0, 2 * el)
        worst = max(worst, float((np.abs(ex - E) / bound(E, A, W, 32 * U)).max()))
    assert worst <= 1.0


def fpn_grid_round(n, y):
    """The method's FP rounding of binary32 y >= 0 for the n-bit type (the
    oracle's own scalar routine, applied element-wise)."""
    L = __import__("oracle.ref", fromlist=["lib"]).lib()
    codes = np.vectorize(lambda t: L.fp4q_ref_fpn_round(n, f32(t)))(y)
    return np.vectorize(lambda m: L.fp4q_ref_fpn_value(n, int(m)))(codes).astype(f32)


def ifn_estimates(ref, n, v, w, S, c, mse):
    """The IF3/IF6 kernel's binary32 estimates at pattern c, in units of S^2:
    FP d = fl(y - q) from y = fl(|x| r); INT through 1.5 2^23 (RNE of the
    exact product, saturated at INTmax), d = fl(|x| r_int - q)."""
    L = ref.lib()
    step = f32(L.fp4q_ref_ifn_step(n))
    top = float((1 << (n - 1)) - 1)
    s = E4M3[c]
    D = (s * f32(S)).astype(f32)
    r = (f32(1) / D).astype(f32)
    Di = (D * step).astype(f32)
    ri = (f32(1) / Di).astype(f32)
    b = np.sqrt(w).astype(f32)
    y = (np.abs(v) * r[:, None]).astype(f32)
    dfp = (y - fpn_grid_round(n, y)).astype(f32)
    p = np.abs(v).astype(f64) * ri.astype(f64)[:, None]
    dint = (p - np.minimum(np.rint(p), top)).astype(f32)
    out = []
    for d, unit in ((dfp, (s * s).astype(f32)), (dint, ((s * step).astype(f32) ** 2).astype(f32))):
        F = np.zeros(v.shape[0], f32)
        for i in range(16):
            e = d[:, i] if mse else (b[:, i] * d[:, i]).astype(f32)
            F = fma32(e, e, F)
        out.append((F * unit).astype(f32).astype(f64))
    return out


@pytest.mark.parametrize("n", [3, 6])
@pytest.mark.parametrize("mse", [True, False])
def test_bound_ifn_estimates(ref, n, mse):
    # IF3 / IF6: the kernel's FP and INT estimates over a window against the
    # oracle's binary64 errors of the same codes, with the 40u relative term
    L = ref.lib()
    rng = np.random.default_rng(30 + n)
    v = np.concatenate([rng.uniform(-1, 1, (200, 16)), student(200, 31, scale=0.1)]).astype(np.float32)
    v[::17] *= np.float32(1e-3)                       # blocks far below the tensor maximum
    w = rng.lognormal(0, 2, v.shape).astype(np.float32)
    fpmax = float(L.fp4q_ref_fpn_max(n))
    S = L.fp4q_ref_ifn_global_scale(n, f32(np.abs(v).max()))
    a = np.abs(v).max(1)
    sb = np.array([max(1, L.fp4q_ref_ifn_base_scale(n, v[i].ctypes.data, 16, f32(S))) for i in range(len(v))])
    W = np.full(len(v), 16.0)
    if not mse:
        Wf = np.zeros(len(v), f32)
        for i in range(16):
            Wf = (Wf + w[:, i]).astype(f32)
        W = Wf.astype(f64)
    worst = 0.0
    for k in range(-3, 8):
        c = np.clip(sb + k, 1, 0x7E)
        ctop = np.clip(sb + 7, 1, 0x7E)
        A = np.maximum(a.astype(f64) * f64(f32(1) / f32(S)) * (1 + 4 * U),
                       fpmax * E4M3[ctop].astype(f64)) * (1 + 4 * U)
        Ef, Ei = ifn_estimates(ref, n, v, w, S, c, mse)
        exf = np.array([ref.fpn_block(n, v[i], S, int(c[i]), None if mse else w[i])[0] for i in range(len(v))])
        exi = np.array([ref.intn_block(n, v[i], S, int(c[i]), None if mse else w[i])[0] for i in range(len(v))])
        for E, ex in ((Ef, exf), (Ei, exi)):
            ex = ex / (f64(S) * f64(S))
            worst = max(worst, float((np.abs(ex - E) / bound(E, A, W, 40 * U)).max()))
    assert worst <= 1.0
