/* oracle_driver.c -- runs every entry point of the CPU oracle on small
 * seeded tensors, edge shapes and threads, so that a build with
 * -fsanitize=address,undefined checks its memory accesses and arithmetic.
 * Exits 0 when every call returned what it should; the sanitizers abort on
 * the first error they find. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fp4q_ref.h"

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;

static uint64_t next_u64(void) /* splitmix64 */
{
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static float uniform(void) { return (float)((next_u64() >> 40) * 0x1p-24) * 2.0f - 1.0f; }

static int failures = 0;
#define CHECK(cond)                                                               \
    do {                                                                          \
        if (!(cond)) {                                                            \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond);    \
            ++failures;                                                           \
        }                                                                         \
    } while (0)

static void fill(float* x, uint16_t* xb, int64_t n, float scale)
{
    for (int64_t i = 0; i < n; ++i) {
        float v = uniform() * scale;
        if (i % 97 == 3)
            v *= 40.0f; /* outliers */
        if (i % 211 == 5)
            v = 0.0f;
        x[i] = v;
        xb[i] = fp4q_ref_f32_to_bf16(v);
    }
}

static void run_shape(int64_t rows, int64_t cols, int nthreads)
{
    const int64_t n = rows * cols;
    const size_t nn = (size_t)(n > 0 ? n : 1);
    float* x = malloc(nn * sizeof(float));
    uint16_t* xb = malloc(nn * sizeof(uint16_t));
    float* imp = malloc((size_t)(cols > 0 ? cols : 1) * sizeof(float));
    uint8_t* codes = malloc(nn * 3 / 4 + 1); /* IF6 needs 6 bits per element */
    uint8_t* scales = malloc(nn / 16 + 1);
    double* best = malloc((nn / 16 + 1) * sizeof(double));
    double* second = malloc((nn / 16 + 1) * sizeof(double));
    float* y = malloc(nn * sizeof(float));
    uint16_t* yb = malloc(nn * sizeof(uint16_t));
    float* coef = malloc(nn / 8 * sizeof(float) + sizeof(float));
    fill(x, xb, n, 1.5f);
    for (int64_t j = 0; j < cols; ++j)
        imp[j] = 0.1f + fabsf(uniform()) * 3.0f;
    for (int64_t j = 0; j < n / 8; ++j)
        coef[j] = 0.8f + 0.4f * fabsf(uniform());

    const int windows[3][2] = {{-3, 7}, {-8, 7}, {-126, 126}};
    for (int fmt = 0; fmt <= REF_IF6; ++fmt) {
        const int B = fmt == REF_MXFP4 ? 32 : 16;
        if (cols % B)
            continue;
        for (int rule = 0; rule < 3; ++rule) {
            if (rule == REF_FOUR_SIX && fmt != REF_NVFP4)
                continue;
            for (int obj = 0; obj < 2; ++obj)
                for (int rot = 0; rot <= B; rot += B)
                    for (int dt = 0; dt < 2; ++dt)
                        for (int w = 0; w < 3; ++w) {
                            if (rule != REF_SWEEP && w > 0)
                                continue;
                            int lo = windows[w][0], hi = windows[w][1];
                            if (fmt == REF_MXFP4 && w == 0) {
                                lo = 0;
                                hi = 1;
                            }
                            for (int given = 0; given < 2; ++given) {
                                float S = given ? 0.0123f : 0.0f;
                                const void* xp = dt ? (const void*)xb : (const void*)x;
                                int rc = fp4q_ref_quantize(fmt, B, rule, obj, lo, hi, rot, given, xp, dt,
                                                           rows, cols, obj ? imp : NULL, codes, scales,
                                                           &S, best, second, nthreads);
                                CHECK(rc == 0);
                                rc = fp4q_ref_dequantize(fmt, B, codes, scales, &S, rows, cols, rot, y,
                                                         REF_F32, nthreads);
                                CHECK(rc == 0);
                                rc = fp4q_ref_dequantize(fmt, B, codes, scales, &S, rows, cols, 0, yb,
                                                         REF_BF16, nthreads);
                                CHECK(rc == 0);
                                double e[2];
                                rc = fp4q_ref_error(fmt, B, rot, xp, dt, rows, cols, obj ? imp : NULL,
                                                    codes, scales, &S, e, nthreads);
                                CHECK(rc == 0);
                                CHECK(n == 0 || e[0] >= 0.0);
                            }
                        }
        }
        if (fmt == REF_NVFP4 || fmt == REF_MXFP4) {
            for (int group = 8; group <= B; group += B - 8) {
                for (int sg = 0; sg < 2; ++sg) {
                    float S = 0.0f;
                    int rc = fp4q_ref_quantize_relaxed(fmt, B, 0, xb, REF_BF16, rows, cols, coef, group,
                                                       sg, codes, scales, &S, nthreads);
                    CHECK(rc == 0);
                }
            }
        }
    }
    if (n > 0) {
        float* xr = malloc(nn * sizeof(float));
        CHECK(fp4q_ref_prepare(xb, REF_BF16, rows, cols, cols % 32 == 0 ? 32 : 16, xr, nthreads) == 0);
        const int64_t nb = n / 16 < 40 ? n / 16 : 40;
        double* ce = malloc((size_t)nb * 127 * sizeof(double));
        CHECK(fp4q_ref_candidate_errors(xr, nb, 16, NULL, 0.01f, ce, nthreads) == 0);
        free(ce);
        free(xr);
    }
    free(x); free(xb); free(imp); free(codes); free(scales); free(best); free(second);
    free(y); free(yb); free(coef);
}

int main(void)
{
    /* scalar helpers over their whole domains */
    for (int m = 0; m < 8; ++m)
        CHECK(fp4q_ref_e2m1_round(fp4q_ref_e2m1_value(m)) == m);
    for (int b = 0; b < 127; ++b)
        CHECK(fp4q_ref_e4m3_round(fp4q_ref_e4m3_value(b)) == b);
    for (int b = 0; b < 255; ++b)
        CHECK(fp4q_ref_e8m0_value(b) > 0.0f);
    CHECK(isnan(fp4q_ref_e8m0_value(255)));
    for (int q = 0; q < 8; ++q)
        CHECK(fp4q_ref_int4_round((float)q) == q);
    CHECK(fp4q_ref_global_scale(0.0f) == 1.0f);
    CHECK(fp4q_ref_global_scale(3e38f) > 0.0f);
    float v[32];
    for (int i = 0; i < 32; ++i)
        v[i] = uniform();
    fp4q_ref_fwht(v, 16);
    fp4q_ref_fwht(v, 32);
    uint8_t nib[16];
    CHECK(fp4q_ref_nvfp4_block(v, 16, NULL, 0.01f, 0x30, nib) >= 0.0);
    CHECK(fp4q_ref_int4_block(v, 16, NULL, 0.01f, 0x30, nib) >= 0.0);
    CHECK(fp4q_ref_base_scale(v, 16, 0.01f) >= 0);
    for (int n = 3; n <= 6; n += 3) {
        for (int m = 0; m < (1 << (n - 1)); ++m)
            CHECK(fp4q_ref_fpn_round(n, fp4q_ref_fpn_value(n, m)) == m);
        CHECK(fp4q_ref_intn_round(n, 1e9f) == (1 << (n - 1)) - 1);
        CHECK(fp4q_ref_fpn_block(n, v, 16, NULL, 0.01f, 0x30, nib) >= 0.0);
        CHECK(fp4q_ref_intn_block(n, v, 16, NULL, 0.01f, 0x30, nib) >= 0.0);
        CHECK(fp4q_ref_ifn_base_scale(n, v, 16, 0.01f) >= 0);
        CHECK(fp4q_ref_ifn_global_scale(n, 3.0f) > 0.0f);
    }

    /* shapes: empty, one block, ragged row counts, several threads */
    const int64_t shapes[][2] = {{0, 64}, {5, 0}, {1, 32}, {3, 96}, {7, 64}, {33, 160}};
    for (size_t s = 0; s < sizeof shapes / sizeof shapes[0]; ++s)
        for (int nt = 1; nt <= 3; nt += 2)
            run_shape(shapes[s][0], shapes[s][1], nt);
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle driver: all entry points ran clean\n");
    return 0;
}
