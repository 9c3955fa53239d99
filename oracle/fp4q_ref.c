/*
 * fp4q_ref.c -- CPU oracle for block-scaled 4-bit quantization.
 *
 * TEST INFRASTRUCTURE ONLY (see fp4q_ref.h).  Plain scalar C, one block at a
 * time, in the order the method states.  Built with -O2 -ffp-contract=off
 * and without fast-math, so every float operation below is one IEEE
 * binary32 operation and every double operation one binary64 operation.
 *
 * The method, step by step, with the page each step follows:
 *   1. widen bf16 to f32 (exact);
 *   2. optional block Hadamard along the contiguous axis, block length n
 *      equal to the quantization block   [MR, Method 1: block-wise Hadamard];
 *   3. NVFP4 / IF4: global scale S = max|x| / (256*6)
 *                                         [SS, Method 2: global scale];
 *   4. per block: AbsMax base scale s_base = E4M3(max|x| / (6 S))
 *      ("block max rounded to FP8")       [SS, Method 2: upper bound];
 *   5. candidates: AbsMax -> {s_base}; ScaleSweep -> the E4M3 bit patterns
 *      s_base + k, k in [lo, hi] ([-3,7] for MSE, [-8,7] for WMSE)
 *                                         [SS, Method 2 and 3];
 *   6. encode each element to the nearest E2M1 value of |x| / (s S);
 *   7. keep the candidate of least block error, MSE or importance-weighted
 *      MSE                                [SS, Method 1: objectives];
 *   8. IF4: compare the FP4 encoding with a scaled INT4 encoding whose step
 *      carries the 6/7 factor, keep the lower MSE and record the choice in
 *      the scale's sign bit               [IF4, Methodology];
 *   9. MXFP4: one E8M0 power-of-two scale per 32 elements, no global scale
 *                                         [MR, Problem];
 *  10. extensions of the same search: Four Over Six (the block maximum onto
 *      6 or onto 4, lower error kept) [IF4, Problem; SS, Problem definition];
 *      a window of E8M0 exponents for MXFP4 [MR, Method 2: format-specific
 *      scale search]; IF4 over a window of patterns, both grids per pattern;
 *      and the FOCUS deploy-side encode, codes from S_q = S_dq * c with given
 *      coefficients c per block or per 8 elements, S_dq stored [FOCUS,
 *      Method 2 and 3].
 *
 * Readings taken where the pages are silent (each is listed in the design
 * notes): E2M1 and INT4 rounding is round-to-nearest with ties to the even
 * code and saturation at the largest magnitude; the sign of a zero code is
 * the sign of the input; every scale computation is the binary32 sequence
 * written below (D = s*S, r = 1/D, y = |x|*r); block errors are evaluated in
 * binary64, and exact ties keep the smaller scale byte (the FP4 branch for
 * IF4); the sweep offset is added to the 7-bit E4M3 magnitude pattern and
 * a pattern outside [0x01, 0x7E] stands for the nearer end pattern (so a
 * window reaching past an end adds nothing new, and a window lying wholly
 * outside still has a candidate); S = 1 for an all-zero tensor
 * and S is never below 2^-117 so that every candidate reciprocal is finite;
 * the MXFP4 exponent is floor(log2 max|x|) - 2 clamped to [-127, 127]; the
 * Hadamard is the Sylvester (natural-order) matrix evaluated by butterflies
 * with stage widths 1, 2, 4, ..., n/2 and then scaled by fl32(1/sqrt(n)).
 */
#include "fp4q_ref.h"

#include <limits.h>
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* ------------------------------------------------------------------------ */
/* formats                                                                  */
/* ------------------------------------------------------------------------ */

/* E2M1: one sign bit (carried separately), two exponent bits with bias 1,
 * one mantissa bit; exponent field 0 is subnormal.  Largest magnitude 6
 * [IF4, Problem: FP4's maximum is 6]. */
float fp4q_ref_e2m1_value(int m)
{
    int e = (m >> 1) & 3;
    int f = m & 1;
    if (e == 0)
        return (float)(0.5 * f);
    return (float)ldexp(1.0 + 0.5 * f, e - 1);
}

/* nearest E2M1 magnitude to y >= 0; on an exact tie the even code wins.
 * Above 6 the nearest value is 6, which is the saturating behaviour. */
int fp4q_ref_e2m1_round(float y)
{
    if (y >= 6.0f) /* also catches +inf, whose distance to every value is inf */
        return 7;
    int best = 0;
    double bestd = INFINITY;
    for (int m = 0; m < 8; ++m) {
        double d = fabs((double)y - (double)fp4q_ref_e2m1_value(m));
        if (d < bestd || (d == bestd && (m & 1) == 0 && (best & 1) == 1)) {
            best = m;
            bestd = d;
        }
    }
    return best;
}

/* E4M3FN (OCP FP8): sign, 4 exponent bits with bias 7, 3 mantissa bits,
 * exponent field 0 subnormal, 0x7F / 0xFF are NaN, no infinities.  Bytes
 * 0x01..0x7E are the 126 positive finite values [SS, Method 2]. */
float fp4q_ref_e4m3_value(int byte)
{
    int b = byte & 0x7F;
    double sgn = (byte & 0x80) ? -1.0 : 1.0;
    if (b == 0x7F)
        return NAN;
    int e = b >> 3;
    int f = b & 7;
    if (e == 0)
        return (float)(sgn * ldexp((double)f, -9));
    return (float)(sgn * ldexp((double)(8 + f), e - 10));
}

/* nearest non-negative E4M3 value to t >= 0, ties to the even byte, with
 * saturation at 448 (0x7E): the nearest finite value to anything above 448
 * is 448 itself. */
int fp4q_ref_e4m3_round(float t)
{
    if (t >= 448.0f)
        return 0x7E;
    int best = 0;
    double bestd = INFINITY;
    for (int b = 0; b <= 0x7E; ++b) {
        double d = fabs((double)t - (double)fp4q_ref_e4m3_value(b));
        if (d < bestd || (d == bestd && (b & 1) == 0 && (best & 1) == 1)) {
            best = b;
            bestd = d;
        }
    }
    return best;
}

/* E8M0: an unsigned biased power of two, 2^(byte-127); 0xFF is NaN. */
float fp4q_ref_e8m0_value(int byte)
{
    if ((byte & 0xFF) == 0xFF)
        return NAN;
    return (float)ldexp(1.0, (byte & 0xFF) - 127);
}

/* nearest integer in 0..7 to y >= 0, ties to even, saturating at 7 */
int fp4q_ref_int4_round(float y)
{
    if (y >= 7.0f)
        return 7;
    int best = 0;
    double bestd = INFINITY;
    for (int q = 0; q <= 7; ++q) {
        double d = fabs((double)y - (double)q);
        if (d < bestd || (d == bestd && (q & 1) == 0 && (best & 1) == 1)) {
            best = q;
            bestd = d;
        }
    }
    return best;
}

float fp4q_ref_bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* bf16 keeps the top 16 bits of a binary32: choose the nearer of the two
 * truncations that bracket f, the one with an even last bit on a tie. */
uint16_t fp4q_ref_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if (isnan(f))
        return (uint16_t)((u >> 16) | 0x0040);
    uint32_t lo = u & 0xFFFF0000u;   /* truncation toward zero */
    uint32_t hi = lo + 0x00010000u;  /* next bf16 away from zero */
    float flo;
    memcpy(&flo, &lo, 4);
    double vlo = (double)flo;
    double vhi;
    if ((hi & 0x7F800000u) == 0x7F800000u) {
        /* the step past the largest finite bf16 lands on 2^128 */
        vhi = copysign(ldexp(1.0, 128), (double)f);
    } else {
        float fhi;
        memcpy(&fhi, &hi, 4);
        vhi = (double)fhi;
    }
    double dlo = fabs((double)f - vlo);
    double dhi = fabs(vhi - (double)f);
    if (dlo < dhi)
        return (uint16_t)(lo >> 16);
    if (dhi < dlo)
        return (uint16_t)(hi >> 16);
    return (uint16_t)((((lo >> 16) & 1) == 0 ? lo : hi) >> 16);
}

/* the INT4 step factor of the 6/7 method [IF4, Methodology]: INT4 codes
 * 0..7 are stretched so that 7 lands where FP4's 6 does. */
float fp4q_ref_int4_step(void)
{
    return 6.0f / 7.0f;
}

/* ---- IF3 and IF6: the adaptive type at 3 and 6 bits ------------------ */
/* [IF4, Methodology: the same idea applies to 3-bit (IF3) and 6-bit (IF6)
 * formats].  The page names the types but fixes no grid, so the reading is
 * the one under which n = 4 is exactly IF4: the FP element of an n-bit type
 * is E2M(n-3) -- a sign bit, two exponent bits with bias 1 and n-3 mantissa
 * bits, exponent field 0 subnormal, no infinities or NaN (E2M0, E2M1 and
 * the OCP FP6 E2M3); the INT element is an integer in
 * [-(2^(n-1) - 1), 2^(n-1) - 1]; an INT block uses the step
 * D * fl32(FPmax / INTmax), which maps the INT maximum onto the FP maximum
 * as 6/7 does for IF4; everything else is IF4's (E4M3 block scale with the
 * indicator in bit 7, base scale E4M3(max|x| / (FPmax S)), and the global
 * scale S = max|x| / (256 FPmax), 256*6 for FP4 [SS, Method 2]). */

/* value of magnitude code m (0 .. 2^(n-1) - 1) of E2M(n-3) */
float fp4q_ref_fpn_value(int n, int m)
{
    int k = n - 3;                 /* mantissa bits */
    int e = (m >> k) & 3;
    int f = m & ((1 << k) - 1);
    double frac = ldexp((double)f, -k);
    if (e == 0)
        return (float)frac;        /* subnormal: f / 2^k */
    return (float)ldexp(1.0 + frac, e - 1);
}

/* largest magnitude of E2M(n-3): 4, 6 and 7.5 for n = 3, 4, 6 */
float fp4q_ref_fpn_max(int n)
{
    return fp4q_ref_fpn_value(n, (1 << (n - 1)) - 1);
}

/* nearest E2M(n-3) magnitude code to y >= 0, the even code on an exact tie,
 * saturating at the largest magnitude */
int fp4q_ref_fpn_round(int n, float y)
{
    int top = (1 << (n - 1)) - 1;
    if (y >= fp4q_ref_fpn_max(n))
        return top;
    int best = 0;
    double bestd = INFINITY;
    for (int m = 0; m <= top; ++m) {
        double d = fabs((double)y - (double)fp4q_ref_fpn_value(n, m));
        if (d < bestd || (d == bestd && (m & 1) == 0 && (best & 1) == 1)) {
            best = m;
            bestd = d;
        }
    }
    return best;
}

/* nearest integer in 0 .. 2^(n-1) - 1 to y >= 0, ties to even, saturating */
int fp4q_ref_intn_round(int n, float y)
{
    int top = (1 << (n - 1)) - 1;
    if (y >= (float)top)
        return top;
    int best = 0;
    double bestd = INFINITY;
    for (int q = 0; q <= top; ++q) {
        double d = fabs((double)y - (double)q);
        if (d < bestd || (d == bestd && (q & 1) == 0 && (best & 1) == 1)) {
            best = q;
            bestd = d;
        }
    }
    return best;
}

/* the INT step factor fl32(FPmax / INTmax): 4/3, 6/7 and 7.5/31 */
float fp4q_ref_ifn_step(int n)
{
    return fp4q_ref_fpn_max(n) / (float)((1 << (n - 1)) - 1);
}

/* bits per element of a format: 3 for IF3, 6 for IF6, 4 otherwise */
static int format_bits(int format)
{
    return format == REF_IF3 ? 3 : (format == REF_IF6 ? 6 : 4);
}

/* ------------------------------------------------------------------------ */
/* Hadamard and global scale                                                */
/* ------------------------------------------------------------------------ */

float fp4q_ref_rotation_scale(int n)
{
    return (float)(1.0 / sqrt((double)n));
}

/* y = H_n x / sqrt(n) for the Sylvester matrix H_n[i][j] = (-1)^popcount(i&j),
 * evaluated as log2(n) butterfly stages of widths 1, 2, ..., n/2 followed by
 * one multiplication [MR, Method 1: block-wise Hadamard before quantizing]. */
void fp4q_ref_fwht(float* v, int n)
{
    for (int h = 1; h < n; h *= 2) {
        for (int i = 0; i < n; i += 2 * h) {
            for (int j = i; j < i + h; ++j) {
                float a = v[j];
                float b = v[j + h];
                v[j] = a + b;
                v[j + h] = a - b;
            }
        }
    }
    float c = fp4q_ref_rotation_scale(n);
    for (int k = 0; k < n; ++k)
        v[k] = v[k] * c;
}

/* S = max|x| / (256*6) [SS, Method 2: global scale]; 1 for an all-zero
 * tensor, and at least 2^-117 so that D = s*S >= 2^-126 for every E4M3
 * byte and 1/D stays finite. */
float fp4q_ref_global_scale(float g)
{
    if (g == 0.0f)
        return 1.0f;
    float s = g / 1536.0f;
    float floor_s = (float)ldexp(1.0, -117);
    return s < floor_s ? floor_s : s;
}

/* the same rule for the n-bit adaptive types: S = max|x| / (256 FPmax) */
float fp4q_ref_ifn_global_scale(int n, float g)
{
    if (g == 0.0f)
        return 1.0f;
    float s = g / (256.0f * fp4q_ref_fpn_max(n));
    float floor_s = (float)ldexp(1.0, -117);
    return s < floor_s ? floor_s : s;
}

/* ------------------------------------------------------------------------ */
/* a tiny row-range thread pool                                             */
/* ------------------------------------------------------------------------ */

typedef void (*row_fn)(void* ctx, int64_t r0, int64_t r1);

typedef struct {
    row_fn fn;
    void* ctx;
    int64_t r0, r1;
} row_job;

static void* row_job_run(void* p)
{
    row_job* j = (row_job*)p;
    j->fn(j->ctx, j->r0, j->r1);
    return NULL;
}

static int resolve_threads(int nthreads)
{
    if (nthreads > 0)
        return nthreads;
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    return n > 0 ? (int)n : 1;
}

static void parallel_rows(int64_t rows, int nthreads, row_fn fn, void* ctx)
{
    int nt = resolve_threads(nthreads);
    if (nt > rows)
        nt = rows > 0 ? (int)rows : 1;
    if (nt <= 1) {
        fn(ctx, 0, rows);
        return;
    }
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nt);
    row_job* jobs = (row_job*)malloc(sizeof(row_job) * (size_t)nt);
    for (int t = 0; t < nt; ++t) {
        jobs[t].fn = fn;
        jobs[t].ctx = ctx;
        jobs[t].r0 = rows * t / nt;
        jobs[t].r1 = rows * (t + 1) / nt;
        pthread_create(&th[t], NULL, row_job_run, &jobs[t]);
    }
    for (int t = 0; t < nt; ++t)
        pthread_join(th[t], NULL);
    free(th);
    free(jobs);
}

/* ------------------------------------------------------------------------ */
/* widening and rotation                                                    */
/* ------------------------------------------------------------------------ */

typedef struct {
    const void* x;
    int dtype;
    int64_t cols;
    int rotate;
    float* out;
} prep_ctx;

static void prep_rows(void* p, int64_t r0, int64_t r1)
{
    prep_ctx* c = (prep_ctx*)p;
    for (int64_t r = r0; r < r1; ++r) {
        float* o = c->out + r * c->cols;
        for (int64_t j = 0; j < c->cols; ++j) {
            int64_t k = r * c->cols + j;
            if (c->dtype == REF_BF16)
                o[j] = fp4q_ref_bf16_to_f32(((const uint16_t*)c->x)[k]);
            else
                o[j] = ((const float*)c->x)[k];
        }
        if (c->rotate > 0)
            for (int64_t j = 0; j < c->cols; j += c->rotate)
                fp4q_ref_fwht(o + j, c->rotate);
    }
}

int fp4q_ref_prepare(const void* x, int x_dtype, int64_t rows, int64_t cols,
                     int rotate, float* out, int nthreads)
{
    if (!x || !out || rows < 0 || cols < 0)
        return -1;
    if (x_dtype != REF_F32 && x_dtype != REF_BF16)
        return -2;
    if (rotate != 0 && (rotate < 2 || (rotate & (rotate - 1)) || cols % rotate))
        return -2;
    prep_ctx c = {x, x_dtype, cols, rotate, out};
    parallel_rows(rows, nthreads, prep_rows, &c);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* per-block encoders                                                       */
/* ------------------------------------------------------------------------ */

static float block_absmax(const float* xb, int B)
{
    float a = 0.0f;
    for (int i = 0; i < B; ++i) {
        float v = fabsf(xb[i]);
        if (v > a)
            a = v;
    }
    return a;
}

int fp4q_ref_base_scale(const float* xb, int B, float S)
{
    float a = block_absmax(xb, B);
    if (a == 0.0f)
        return 0;
    float s6 = 6.0f * S;
    int sb = fp4q_ref_e4m3_round(a / s6);
    return sb == 0 ? 1 : sb;
}

/* squared error of one element, weighted when w != NULL, in binary64 */
static double elem_err(float a, float xh, const float* w, int i)
{
    double d = (double)a - (double)xh;
    double t = d * d;
    if (w)
        t = (double)w[i] * t;
    return t;
}

double fp4q_ref_nvfp4_block(const float* xb, int B, const float* w, float S,
                            int c, uint8_t* codes)
{
    float s = fp4q_ref_e4m3_value(c);
    float D = s * S;
    float r = 1.0f / D;
    double E = 0.0;
    for (int i = 0; i < B; ++i) {
        float a = fabsf(xb[i]);
        float y = a * r;
        int m = fp4q_ref_e2m1_round(y);
        float xh = fp4q_ref_e2m1_value(m) * D;
        E = E + elem_err(a, xh, w, i);
        if (codes)
            codes[i] = (uint8_t)((signbit(xb[i]) ? 8 : 0) | m);
    }
    return E;
}

double fp4q_ref_int4_block(const float* xb, int B, const float* w, float S,
                           int c, uint8_t* codes)
{
    float s = fp4q_ref_e4m3_value(c);
    float D = s * S;
    float Di = D * fp4q_ref_int4_step();
    float ri = 1.0f / Di;
    double E = 0.0;
    for (int i = 0; i < B; ++i) {
        float a = fabsf(xb[i]);
        float y = a * ri;
        int q = fp4q_ref_int4_round(y);
        float xh = (float)q * Di;
        E = E + elem_err(a, xh, w, i);
        if (codes) {
            int sq = signbit(xb[i]) ? -q : q;
            codes[i] = (uint8_t)(sq & 0xF);
        }
    }
    return E;
}

/* base scale of an n-bit adaptive type: E4M3(max|x| / (FPmax S)), >= 1 */
int fp4q_ref_ifn_base_scale(int n, const float* xb, int B, float S)
{
    float a = block_absmax(xb, B);
    if (a == 0.0f)
        return 0;
    float sm = fp4q_ref_fpn_max(n) * S;
    int sb = fp4q_ref_e4m3_round(a / sm);
    return sb == 0 ? 1 : sb;
}

/* FP branch of an n-bit adaptive type with scale byte c: codes are
 * sign << (n-1) | magnitude code */
double fp4q_ref_fpn_block(int n, const float* xb, int B, const float* w, float S,
                          int c, uint8_t* codes)
{
    float s = fp4q_ref_e4m3_value(c);
    float D = s * S;
    float r = 1.0f / D;
    double E = 0.0;
    for (int i = 0; i < B; ++i) {
        float a = fabsf(xb[i]);
        float y = a * r;
        int m = fp4q_ref_fpn_round(n, y);
        float xh = fp4q_ref_fpn_value(n, m) * D;
        E = E + elem_err(a, xh, w, i);
        if (codes)
            codes[i] = (uint8_t)((signbit(xb[i]) ? (1 << (n - 1)) : 0) | m);
    }
    return E;
}

/* INT branch: step D * fl32(FPmax / INTmax); codes are the n-bit two's
 * complement of the signed integer.  A zero element is the integer 0
 * (|x| / D_int = 0), also where D_int < 2^-128 makes ri infinite and
 * |x| * ri would be NaN: IF6's step 7.5/31 is below 1/4, so the smallest
 * patterns under the smallest global scales get there. */
double fp4q_ref_intn_block(int n, const float* xb, int B, const float* w, float S,
                           int c, uint8_t* codes)
{
    float s = fp4q_ref_e4m3_value(c);
    float D = s * S;
    float Di = D * fp4q_ref_ifn_step(n);
    float ri = 1.0f / Di;
    double E = 0.0;
    for (int i = 0; i < B; ++i) {
        float a = fabsf(xb[i]);
        int q = 0;
        if (a != 0.0f)
            q = fp4q_ref_intn_round(n, a * ri);
        float xh = (float)q * Di;
        E = E + elem_err(a, xh, w, i);
        if (codes) {
            int sq = signbit(xb[i]) ? -q : q;
            codes[i] = (uint8_t)(sq & ((1 << n) - 1));
        }
    }
    return E;
}

typedef struct {
    const float* xb;
    int B;
    const float* w;
    float S;
    double* out;
} cand_ctx;

static void cand_rows(void* p, int64_t b0, int64_t b1)
{
    cand_ctx* c = (cand_ctx*)p;
    for (int64_t b = b0; b < b1; ++b) {
        const float* xb = c->xb + b * c->B;
        const float* w = c->w ? c->w + b * c->B : NULL;
        double* o = c->out + b * 127;
        o[0] = NAN;
        for (int s = 1; s <= 0x7E; ++s)
            o[s] = fp4q_ref_nvfp4_block(xb, c->B, w, c->S, s, NULL);
    }
}

int fp4q_ref_candidate_errors(const float* xb, int64_t nblocks, int B,
                              const float* w, float S, double* out, int nthreads)
{
    if (!xb || !out || nblocks < 0 || B <= 0)
        return -1;
    cand_ctx c = {xb, B, w, S, out};
    parallel_rows(nblocks, nthreads, cand_rows, &c);
    return 0;
}

/* floor(log2(a)) for a > 0, subnormals included */
static int floor_log2(float a)
{
    int e;
    double m = frexp((double)a, &e); /* a = m 2^e, m in [0.5, 1) */
    (void)m;
    return e - 1;
}

/* ------------------------------------------------------------------------ */
/* quantize                                                                 */
/* ------------------------------------------------------------------------ */

typedef struct {
    int format, block, rule, objective, lo, hi;
    const float* xr; /* widened, rotated */
    int64_t cols;
    const float* imp;
    float S;
    uint8_t* codes;
    uint8_t* scales;
    double* best;
    double* second;
} quant_ctx;

static void put_nibbles(uint8_t* codes, int64_t elem0, const uint8_t* nib, int B)
{
    for (int i = 0; i < B; i += 2)
        codes[(elem0 + i) / 2] = (uint8_t)((nib[i] & 0xF) | ((nib[i + 1] & 0xF) << 4));
}

/* n-bit codes: element e of the tensor occupies bits n e .. n e + n - 1 of
 * the code stream, least significant bit first (for n = 4: element 2k in the
 * low nibble of byte k, as put_nibbles writes) */
static void put_codes(uint8_t* codes, int64_t elem0, const uint8_t* c, int B, int n)
{
    for (int i = 0; i < B; ++i) {
        for (int b = 0; b < n; ++b) {
            int64_t bit = (elem0 + i) * n + b;
            uint8_t mask = (uint8_t)(1u << (bit & 7));
            if ((c[i] >> b) & 1)
                codes[bit >> 3] |= mask;
            else
                codes[bit >> 3] &= (uint8_t)~mask;
        }
    }
}

static int get_code(const uint8_t* codes, int64_t e, int n)
{
    int v = 0;
    for (int b = 0; b < n; ++b) {
        int64_t bit = e * n + b;
        v |= ((codes[bit >> 3] >> (bit & 7)) & 1) << b;
    }
    return v;
}

/* keep the first least error among candidates tried in order; also the
 * second least.  *cbest == NONE until the first candidate. */
#define NONE INT_MIN
static void consider(double E, int cand, double* best, double* second, int* cbest)
{
    if (*cbest == NONE || E < *best) {
        if (*cbest != NONE)
            *second = *best;
        *best = E;
        *cbest = cand;
    } else if (E < *second) {
        *second = E;
    }
}

static int clamp_pattern(int c) { return c < 0x01 ? 0x01 : (c > 0x7E ? 0x7E : c); }

/* MXFP4: E8M0 exponent of the OCP rule, floor(log2 max) - 2 in [-127, 127]
 * ["Bridging the Gap ... Microscaling FP4", Problem: power-of-two scales] */
static int mx_exponent(float a)
{
    int e = (a == 0.0f) ? -127 : floor_log2(a) - 2;
    return e < -127 ? -127 : (e > 127 ? 127 : e);
}

/* MXFP4 encode of one block with exponent e; returns the block error */
static double mx_block(const float* xb, int B, const float* w, int e, uint8_t* nib)
{
    float D = (float)ldexp(1.0, e);
    float rr = (float)ldexp(1.0, -e);
    double E = 0.0;
    for (int i = 0; i < B; ++i) {
        float av = fabsf(xb[i]);
        int m = fp4q_ref_e2m1_round(av * rr);
        float xh = fp4q_ref_e2m1_value(m) * D;
        E = E + elem_err(av, xh, w, i);
        if (nib)
            nib[i] = (uint8_t)((signbit(xb[i]) ? 8 : 0) | m);
    }
    return E;
}

/* Four Over Six: the pattern that maps the block maximum onto 4 instead of 6
 * [Adaptive Block-Scaled Data Types, Problem; ScaleSweep, Problem definition] */
static int four_scale(const float* xb, int B, float S)
{
    float a = block_absmax(xb, B);
    float s4 = 4.0f * S;
    int sb = fp4q_ref_e4m3_round(a / s4);
    return sb == 0 ? 1 : sb;
}

static void quant_rows(void* p, int64_t r0, int64_t r1)
{
    quant_ctx* q = (quant_ctx*)p;
    const int B = q->block;
    const int64_t nbr = q->cols / B;
    uint8_t nib[64];
    for (int64_t r = r0; r < r1; ++r) {
        for (int64_t jb = 0; jb < nbr; ++jb) {
            int64_t e0 = r * q->cols + jb * B;
            int64_t bi = r * nbr + jb;
            const float* xb = q->xr + e0;
            const float* w = (q->objective == REF_WMSE) ? q->imp + jb * B : NULL;
            double best = 0.0, second = INFINITY;
            int cbest = NONE;
            uint8_t sbyte = 0;
            float a = block_absmax(xb, B);

            if (q->format == REF_MXFP4) {
                int e0x = mx_exponent(a);
                if (q->rule == REF_SWEEP) {
                    /* a window of E8M0 exponents around the OCP one, MSE or
                     * WMSE argmin ["Bridging the Gap", Method 2: format-
                     * specific scale search / scale fitting] */
                    int eprev = 1000;
                    for (int k = q->lo; k <= q->hi; ++k) {
                        int e = e0x + k;
                        e = e < -127 ? -127 : (e > 127 ? 127 : e);
                        if (e == eprev)
                            continue;
                        eprev = e;
                        consider(mx_block(xb, B, w, e, NULL), e, &best, &second, &cbest);
                    }
                } else {
                    cbest = e0x;
                    best = mx_block(xb, B, w, e0x, NULL);
                }
                best = mx_block(xb, B, w, cbest, nib);
                sbyte = (uint8_t)(cbest + 127);
            } else if (a == 0.0f) {
                /* all-zero block: scale byte 0, codes keep only the sign */
                sbyte = 0;
                for (int i = 0; i < B; ++i)
                    nib[i] = (uint8_t)(signbit(xb[i]) ? 1 << (format_bits(q->format) - 1) : 0);
                best = 0.0;
                second = (q->format != REF_NVFP4 || q->rule != REF_ABSMAX) ? 0.0 : INFINITY;
            } else if (q->format == REF_IF3 || q->format == REF_IF6) {
                /* the n-bit adaptive type: per pattern the FP grid first, then
                 * the INT grid (indicator bit 7), as IF4 */
                int n = format_bits(q->format);
                int sb = fp4q_ref_ifn_base_scale(n, xb, B, q->S);
                int lo = q->rule == REF_SWEEP ? q->lo : 0;
                int hi = q->rule == REF_SWEEP ? q->hi : 0;
                int cprev = -1;
                for (int k = lo; k <= hi; ++k) {
                    int c = clamp_pattern(sb + k);
                    if (c == cprev)
                        continue;
                    cprev = c;
                    consider(fp4q_ref_fpn_block(n, xb, B, w, q->S, c, NULL), c, &best, &second, &cbest);
                    consider(fp4q_ref_intn_block(n, xb, B, w, q->S, c, NULL), c | 0x80, &best, &second, &cbest);
                }
                if (cbest & 0x80)
                    fp4q_ref_intn_block(n, xb, B, w, q->S, cbest & 0x7F, nib);
                else
                    fp4q_ref_fpn_block(n, xb, B, w, q->S, cbest, nib);
                sbyte = (uint8_t)cbest;
            } else {
                int sb = fp4q_ref_base_scale(xb, B, q->S);
                if (q->format == REF_IF4) {
                    /* per pattern: FP4 first, then INT4 (indicator bit 7) */
                    int lo = q->rule == REF_SWEEP ? q->lo : 0;
                    int hi = q->rule == REF_SWEEP ? q->hi : 0;
                    int cprev = -1;
                    for (int k = lo; k <= hi; ++k) {
                        int c = clamp_pattern(sb + k);
                        if (c == cprev)
                            continue;
                        cprev = c;
                        consider(fp4q_ref_nvfp4_block(xb, B, w, q->S, c, NULL), c, &best, &second, &cbest);
                        consider(fp4q_ref_int4_block(xb, B, w, q->S, c, NULL), c | 0x80, &best, &second, &cbest);
                    }
                    if (cbest & 0x80)
                        fp4q_ref_int4_block(xb, B, w, q->S, cbest & 0x7F, nib);
                    else
                        fp4q_ref_nvfp4_block(xb, B, w, q->S, cbest, nib);
                    sbyte = (uint8_t)cbest;
                } else if (q->rule == REF_ABSMAX) {
                    sbyte = (uint8_t)sb;
                    best = fp4q_ref_nvfp4_block(xb, B, w, q->S, sb, nib);
                } else if (q->rule == REF_FOUR_SIX) {
                    int s4 = four_scale(xb, B, q->S);
                    consider(fp4q_ref_nvfp4_block(xb, B, w, q->S, sb, NULL), sb, &best, &second, &cbest);
                    if (s4 != sb)
                        consider(fp4q_ref_nvfp4_block(xb, B, w, q->S, s4, NULL), s4, &best, &second, &cbest);
                    sbyte = (uint8_t)cbest;
                    fp4q_ref_nvfp4_block(xb, B, w, q->S, cbest, nib);
                } else {
                    int cprev = -1;
                    for (int k = q->lo; k <= q->hi; ++k) {
                        /* patterns past either end of [0x01, 0x7E] stand for the
                         * end pattern itself; each pattern is tried once */
                        int c = clamp_pattern(sb + k);
                        if (c == cprev)
                            continue;
                        cprev = c;
                        consider(fp4q_ref_nvfp4_block(xb, B, w, q->S, c, NULL), c, &best, &second, &cbest);
                    }
                    sbyte = (uint8_t)cbest;
                    fp4q_ref_nvfp4_block(xb, B, w, q->S, cbest, nib);
                }
            }
            if (format_bits(q->format) == 4)
                put_nibbles(q->codes, e0, nib, B);
            else
                put_codes(q->codes, e0, nib, B, format_bits(q->format));
            q->scales[bi] = sbyte;
            if (q->best)
                q->best[bi] = best;
            if (q->second)
                q->second[bi] = second;
        }
    }
}

typedef struct {
    const float* xr;
    int64_t cols;
    float* rowmax;
} max_ctx;

static void max_rows(void* p, int64_t r0, int64_t r1)
{
    max_ctx* m = (max_ctx*)p;
    for (int64_t r = r0; r < r1; ++r) {
        float g = 0.0f;
        const float* row = m->xr + r * m->cols;
        for (int64_t j = 0; j < m->cols; ++j) {
            float v = fabsf(row[j]);
            if (v > g)
                g = v;
        }
        m->rowmax[r] = g;
    }
}

static int check_common(int format, int block, int rotate, int64_t rows, int64_t cols)
{
    if (rows < 0 || cols < 0)
        return -3;
    if (format == REF_MXFP4) {
        if (block != 32)
            return -4;
    } else if (format == REF_NVFP4 || format == REF_IF4 || format == REF_IF3 || format == REF_IF6) {
        if (block != 16)
            return -4;
    } else {
        return -2;
    }
    if (cols % block)
        return -3;
    if (rotate != 0 && rotate != block)
        return -2;
    return 0;
}

int fp4q_ref_quantize(int format, int block, int scale_rule, int objective,
                      int sweep_lo, int sweep_hi, int rotate,
                      int global_scale_given,
                      const void* x, int x_dtype, int64_t rows, int64_t cols,
                      const float* importance,
                      uint8_t* codes, uint8_t* scales, float* global_scale,
                      double* best_err, double* second_err, int nthreads)
{
    int rc = check_common(format, block, rotate, rows, cols);
    if (rc)
        return rc;
    if (!x || !codes || !scales)
        return -1;
    if (format != REF_MXFP4 && !global_scale)
        return -1;
    if (objective == REF_WMSE && !importance)
        return -1;
    if (scale_rule == REF_SWEEP && sweep_lo > sweep_hi)
        return -2;
    if (scale_rule == REF_FOUR_SIX && format != REF_NVFP4)
        return -4;
    if (scale_rule < REF_ABSMAX || scale_rule > REF_FOUR_SIX)
        return -2;

    int64_t n = rows * cols;
    float* xr = (float*)malloc(sizeof(float) * (size_t)(n > 0 ? n : 1));
    if (!xr)
        return -6;
    fp4q_ref_prepare(x, x_dtype, rows, cols, rotate, xr, nthreads);

    float S = 1.0f;
    if (format != REF_MXFP4) {
        if (global_scale_given) {
            S = *global_scale;
        } else {
            float* rowmax = (float*)calloc((size_t)(rows > 0 ? rows : 1), sizeof(float));
            max_ctx mc = {xr, cols, rowmax};
            parallel_rows(rows, nthreads, max_rows, &mc);
            float g = 0.0f;
            for (int64_t r = 0; r < rows; ++r)
                if (rowmax[r] > g)
                    g = rowmax[r];
            free(rowmax);
            S = (format == REF_IF3 || format == REF_IF6)
                    ? fp4q_ref_ifn_global_scale(format_bits(format), g)
                    : fp4q_ref_global_scale(g);
            *global_scale = S;
        }
    }

    quant_ctx q = {format, block, scale_rule, objective, sweep_lo, sweep_hi,
                   xr, cols, importance, S, codes, scales, best_err, second_err};
    parallel_rows(rows, nthreads, quant_rows, &q);
    free(xr);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* FOCUS deploy-side encode                                                 */
/* ------------------------------------------------------------------------ */

/* Codes from the relaxed quantization scale S_q = S_dq * c while the stored
 * (dequantization) scale stays S_dq [FOCUS, Method 2 "coupled-relaxation
 * scaling": S_q = S_dq c_i; Method 3 "dual-granularity scaling": one c_k per
 * sub-block of 8 with S_dq shared by the block].  S_dq is the AbsMax scale
 * (NVFP4: E4M3 of max/(6S); MXFP4: the OCP exponent) or, when scales_given,
 * the caller's bytes.  Per element: D_q = fl(D c), r_q = fl(1/D_q),
 * code = E2M1(fl(|x| r_q)); a block whose step D is 0 keeps only signs. */
typedef struct {
    int format, block, group, scales_given;
    const float* xr;
    int64_t cols;
    const float* coef;
    float S;
    uint8_t* codes;
    uint8_t* scales;
} relax_ctx;

static void relax_rows(void* p, int64_t r0, int64_t r1)
{
    relax_ctx* q = (relax_ctx*)p;
    const int B = q->block;
    const int64_t nbr = q->cols / B, ngr = q->cols / q->group;
    uint8_t nib[64];
    for (int64_t r = r0; r < r1; ++r) {
        for (int64_t jb = 0; jb < nbr; ++jb) {
            int64_t e0 = r * q->cols + jb * B;
            int64_t bi = r * nbr + jb;
            const float* xb = q->xr + e0;
            int byte;
            float D;
            if (q->scales_given) {
                byte = q->scales[bi];
                D = (q->format == REF_MXFP4) ? fp4q_ref_e8m0_value(byte)
                                             : fp4q_ref_e4m3_value(byte) * q->S;
            } else if (q->format == REF_MXFP4) {
                int e = mx_exponent(block_absmax(xb, B));
                byte = e + 127;
                D = (float)ldexp(1.0, e);
            } else {
                byte = fp4q_ref_base_scale(xb, B, q->S);
                D = byte ? fp4q_ref_e4m3_value(byte) * q->S : 0.0f;
            }
            for (int i = 0; i < B; ++i) {
                int m = 0;
                if (D != 0.0f && xb[i] != 0.0f) {
                    /* a zero element keeps code 0: |x| / S_q = 0, also where
                     * D_q < 2^-128 makes rq = +inf and |x| * rq would be NaN */
                    float c = q->coef[r * ngr + (jb * B + i) / q->group];
                    float Dq = D * c;
                    float rq = 1.0f / Dq;
                    m = fp4q_ref_e2m1_round(fabsf(xb[i]) * rq);
                }
                nib[i] = (uint8_t)((signbit(xb[i]) ? 8 : 0) | m);
            }
            put_nibbles(q->codes, e0, nib, B);
            if (!q->scales_given)
                q->scales[bi] = (uint8_t)byte;
        }
    }
}

int fp4q_ref_quantize_relaxed(int format, int block, int global_scale_given,
                              const void* x, int x_dtype, int64_t rows, int64_t cols,
                              const float* coef, int group, int scales_given,
                              uint8_t* codes, uint8_t* scales, float* global_scale,
                              int nthreads)
{
    int rc = check_common(format, block, 0, rows, cols);
    if (rc)
        return rc;
    if (format == REF_IF4 || format == REF_IF3 || format == REF_IF6)
        return -4;
    if (group != 8 && group != block)
        return -2;
    if (!x || !coef || !codes || !scales || (format != REF_MXFP4 && !global_scale))
        return -1;
    int64_t n = rows * cols;
    float* xr = (float*)malloc(sizeof(float) * (size_t)(n > 0 ? n : 1));
    if (!xr)
        return -6;
    fp4q_ref_prepare(x, x_dtype, rows, cols, 0, xr, nthreads);
    float S = 1.0f;
    if (format != REF_MXFP4) {
        if (global_scale_given) {
            S = *global_scale;
        } else {
            float g = 0.0f;
            for (int64_t k = 0; k < n; ++k)
                if (fabsf(xr[k]) > g)
                    g = fabsf(xr[k]);
            S = fp4q_ref_global_scale(g);
            *global_scale = S;
        }
    }
    relax_ctx q = {format, block, group, scales_given, xr, cols, coef, S, codes, scales};
    parallel_rows(rows, nthreads, relax_rows, &q);
    free(xr);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* dequantize                                                               */
/* ------------------------------------------------------------------------ */

typedef struct {
    int format, block, unrotate;
    const uint8_t* codes;
    const uint8_t* scales;
    float S;
    int64_t cols;
    float* out; /* f32 [rows, cols] */
} deq_ctx;

/* value of one stored element of block with scale byte sb */
static float deq_elem(int format, int sb, int nibble, float S)
{
    if (format == REF_IF3 || format == REF_IF6) {
        int n = format_bits(format);
        float D = fp4q_ref_e4m3_value(sb & 0x7F) * S;
        if (sb & 0x80) {
            float Di = D * fp4q_ref_ifn_step(n);
            int q = (nibble & (1 << (n - 1))) ? nibble - (1 << n) : nibble;
            return (float)q * Di;
        }
        float v = fp4q_ref_fpn_value(n, nibble & ((1 << (n - 1)) - 1)) * D;
        return (nibble >> (n - 1)) ? -v : v;
    }
    if (format == REF_MXFP4) {
        float D = fp4q_ref_e8m0_value(sb);
        float v = fp4q_ref_e2m1_value(nibble & 7) * D;
        return (nibble & 8) ? -v : v;
    }
    if (format == REF_IF4 && (sb & 0x80)) {
        float D = fp4q_ref_e4m3_value(sb & 0x7F) * S;
        float Di = D * fp4q_ref_int4_step();
        int q = (nibble & 8) ? nibble - 16 : nibble;
        return (float)q * Di;
    }
    int byte = (format == REF_IF4) ? (sb & 0x7F) : sb;
    float D = fp4q_ref_e4m3_value(byte) * S;
    float v = fp4q_ref_e2m1_value(nibble & 7) * D;
    return (nibble & 8) ? -v : v;
}

static void deq_rows(void* p, int64_t r0, int64_t r1)
{
    deq_ctx* d = (deq_ctx*)p;
    const int B = d->block;
    const int64_t nbr = d->cols / B;
    for (int64_t r = r0; r < r1; ++r) {
        for (int64_t jb = 0; jb < nbr; ++jb) {
            int64_t e0 = r * d->cols + jb * B;
            int sb = d->scales[r * nbr + jb];
            float* o = d->out + e0;
            for (int i = 0; i < B; ++i) {
                int64_t e = e0 + i;
                int nib = format_bits(d->format) != 4 ? get_code(d->codes, e, format_bits(d->format))
                        : (e & 1) ? (d->codes[e / 2] >> 4) : (d->codes[e / 2] & 0xF);
                o[i] = deq_elem(d->format, sb, nib, d->S);
            }
            if (d->unrotate)
                fp4q_ref_fwht(o, B);
        }
    }
}

static float* dequant_f32(int format, int block, const uint8_t* codes,
                          const uint8_t* scales, float S, int64_t rows,
                          int64_t cols, int unrotate, int nthreads)
{
    int64_t n = rows * cols;
    float* out = (float*)malloc(sizeof(float) * (size_t)(n > 0 ? n : 1));
    if (!out)
        return NULL;
    deq_ctx d = {format, block, unrotate, codes, scales, S, cols, out};
    parallel_rows(rows, nthreads, deq_rows, &d);
    return out;
}

int fp4q_ref_dequantize(int format, int block, const uint8_t* codes,
                        const uint8_t* scales, const float* global_scale,
                        int64_t rows, int64_t cols, int unrotate,
                        void* y, int y_dtype, int nthreads)
{
    int rc = check_common(format, block, unrotate, rows, cols);
    if (rc)
        return rc;
    if (!codes || !scales || !y)
        return -1;
    if (format != REF_MXFP4 && !global_scale)
        return -1;
    float S = (format == REF_MXFP4) ? 1.0f : *global_scale;
    float* f = dequant_f32(format, block, codes, scales, S, rows, cols, unrotate, nthreads);
    if (!f)
        return -6;
    int64_t n = rows * cols;
    for (int64_t k = 0; k < n; ++k) {
        if (y_dtype == REF_BF16)
            ((uint16_t*)y)[k] = fp4q_ref_f32_to_bf16(f[k]);
        else
            ((float*)y)[k] = f[k];
    }
    free(f);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* error                                                                    */
/* ------------------------------------------------------------------------ */

typedef struct {
    const float* x;  /* widened, un-rotated */
    const float* xh; /* dequantized, un-rotated */
    const float* imp;
    int64_t cols;
    double* rs;  /* per-row sum of squared errors */
    double* rws; /* per-row importance-weighted sum */
} err_ctx;

static void err_rows(void* p, int64_t r0, int64_t r1)
{
    err_ctx* e = (err_ctx*)p;
    for (int64_t r = r0; r < r1; ++r) {
        double s = 0.0, ws = 0.0;
        for (int64_t j = 0; j < e->cols; ++j) {
            int64_t k = r * e->cols + j;
            double d = (double)e->x[k] - (double)e->xh[k];
            double t = d * d;
            s = s + t;
            if (e->imp)
                ws = ws + (double)e->imp[j] * t;
        }
        e->rs[r] = s;
        e->rws[r] = ws;
    }
}

/* MSE = sum (x - xhat)^2 / N and WMSE = sum w_col (x - xhat)^2 / N in the
 * caller's (un-rotated) domain [SS, Method 1: objectives]. */
int fp4q_ref_error(int format, int block, int rotate,
                   const void* x, int x_dtype, int64_t rows, int64_t cols,
                   const float* importance, const uint8_t* codes,
                   const uint8_t* scales, const float* global_scale,
                   double out[2], int nthreads)
{
    int rc = check_common(format, block, rotate, rows, cols);
    if (rc)
        return rc;
    if (!x || !codes || !scales || !out)
        return -1;
    if (format != REF_MXFP4 && !global_scale)
        return -1;
    int64_t n = rows * cols;
    if (n == 0) {
        out[0] = 0.0;
        out[1] = importance ? 0.0 : NAN;
        return 0;
    }
    float S = (format == REF_MXFP4) ? 1.0f : *global_scale;
    float* xw = (float*)malloc(sizeof(float) * (size_t)n);
    fp4q_ref_prepare(x, x_dtype, rows, cols, 0, xw, nthreads);
    float* xh = dequant_f32(format, block, codes, scales, S, rows, cols, rotate, nthreads);
    double* rs = (double*)calloc((size_t)rows, sizeof(double));
    double* rws = (double*)calloc((size_t)rows, sizeof(double));
    err_ctx e = {xw, xh, importance, cols, rs, rws};
    parallel_rows(rows, nthreads, err_rows, &e);
    double s = 0.0, ws = 0.0;
    for (int64_t r = 0; r < rows; ++r) {
        s = s + rs[r];
        ws = ws + rws[r];
    }
    out[0] = s / (double)n;
    out[1] = importance ? ws / (double)n : NAN;
    free(xw);
    free(xh);
    free(rs);
    free(rws);
    return 0;
}
