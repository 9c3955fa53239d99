/*
 * capi_example.c -- a plain C consumer of libfp4q.so, checked against the C
 * oracle (test infrastructure: the oracle is linked only here).
 *
 * It allocates device memory with the HIP runtime, quantizes a seeded fp32
 * tensor with NVFP4 ScaleSweep WMSE [-8, 7] through include/fp4q.h,
 * dequantizes it, and compares codes, scale bytes, the global scale and the
 * dequantized values with fp4q_ref_quantize / fp4q_ref_dequantize, byte for
 * byte.  It also shows a rejected call (cols not a multiple of the block).
 * Exit status 0 when everything matches.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fp4q.h"
#include "fp4q_ref.h"

#define CHECK_HIP(call)                                                              \
    do {                                                                             \
        hipError_t e_ = (call);                                                      \
        if (e_ != hipSuccess) {                                                      \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));        \
            return 2;                                                                \
        }                                                                            \
    } while (0)

/* 64-bit linear congruential generator (Knuth's MMIX constants) */
static uint64_t lcg_state = 0x9E3779B97F4A7C15ull;
static double uniform01(void)
{
    lcg_state = lcg_state * 6364136223846793005ull + 1442695040888963407ull;
    return ((lcg_state >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

int main(void)
{
    const int64_t rows = 96, cols = 512, n = rows * cols;
    float* x = malloc(sizeof(float) * n);
    float* imp = malloc(sizeof(float) * cols);
    for (int64_t i = 0; i < n; ++i) { /* heavy-tailed values: normal / sqrt(uniform) */
        double g = sqrt(-2.0 * log(uniform01())) * cos(6.283185307179586 * uniform01());
        x[i] = (float)(0.02 * g / sqrt(uniform01() + 0.05));
    }
    for (int64_t j = 0; j < cols; ++j)
        imp[j] = (float)exp(2.0 * uniform01() - 1.0);

    fp4q_spec spec = {FP4Q_NVFP4, 16, FP4Q_SCALE_SWEEP, FP4Q_OBJ_WMSE, -8, 7, 0, 0};
    const size_t ws_bytes = fp4q_workspace_bytes(&spec, rows, cols);
    void *dx, *dimp, *dcodes, *dscales, *dgs, *dws, *dy;
    CHECK_HIP(hipMalloc(&dx, sizeof(float) * n));
    CHECK_HIP(hipMalloc(&dimp, sizeof(float) * cols));
    CHECK_HIP(hipMalloc(&dcodes, n / 2));
    CHECK_HIP(hipMalloc(&dscales, n / 16));
    CHECK_HIP(hipMalloc(&dgs, sizeof(float)));
    CHECK_HIP(hipMalloc(&dws, ws_bytes));
    CHECK_HIP(hipMalloc(&dy, sizeof(float) * n));
    CHECK_HIP(hipMemcpy(dx, x, sizeof(float) * n, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dimp, imp, sizeof(float) * cols, hipMemcpyHostToDevice));

    /* a rejected call leaves everything untouched and says why */
    fp4q_status st = fp4q_quantize(&spec, dx, FP4Q_F32, rows, cols - 12, dimp, dcodes, dscales,
                                   dgs, dws, ws_bytes, NULL);
    printf("cols %lld: %s\n", (long long)(cols - 12), fp4q_status_string(st));
    if (st != FP4Q_E_SHAPE)
        return 1;

    st = fp4q_quantize(&spec, dx, FP4Q_F32, rows, cols, dimp, dcodes, dscales, dgs, dws, ws_bytes,
                       NULL);
    if (st != FP4Q_OK) {
        fprintf(stderr, "fp4q_quantize: %s\n", fp4q_status_string(st));
        return 1;
    }
    st = fp4q_dequantize(&spec, dcodes, dscales, dgs, rows, cols, 0, dy, FP4Q_F32, NULL);
    if (st != FP4Q_OK) {
        fprintf(stderr, "fp4q_dequantize: %s\n", fp4q_status_string(st));
        return 1;
    }
    CHECK_HIP(hipDeviceSynchronize());

    uint8_t* codes = malloc(n / 2);
    uint8_t* scales = malloc(n / 16);
    float* y = malloc(sizeof(float) * n);
    float gs;
    CHECK_HIP(hipMemcpy(codes, dcodes, n / 2, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(scales, dscales, n / 16, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(&gs, dgs, sizeof(float), hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(y, dy, sizeof(float) * n, hipMemcpyDeviceToHost));

    uint8_t* rcodes = malloc(n / 2);
    uint8_t* rscales = malloc(n / 16);
    float* ry = malloc(sizeof(float) * n);
    float rgs = 0.0f;
    if (fp4q_ref_quantize(0, 16, 1, 1, -8, 7, 0, 0, x, 0, rows, cols, imp, rcodes, rscales, &rgs,
                          NULL, NULL, 0) != 0 ||
        fp4q_ref_dequantize(0, 16, rcodes, rscales, &rgs, rows, cols, 0, ry, 0, 0) != 0) {
        fprintf(stderr, "oracle call failed\n");
        return 1;
    }
    const int ok = memcmp(&gs, &rgs, sizeof(float)) == 0 && memcmp(codes, rcodes, n / 2) == 0 &&
                   memcmp(scales, rscales, n / 16) == 0 && memcmp(y, ry, sizeof(float) * n) == 0;
    printf("NVFP4 ScaleSweep WMSE %lldx%lld through the C ABI: S %.9g, %s the oracle\n",
           (long long)rows, (long long)cols, gs, ok ? "matches" : "DIFFERS FROM");
    hipFree(dx); hipFree(dimp); hipFree(dcodes); hipFree(dscales); hipFree(dgs); hipFree(dws); hipFree(dy);
    free(x); free(imp); free(codes); free(scales); free(y); free(rcodes); free(rscales); free(ry);
    return ok ? 0 : 1;
}
