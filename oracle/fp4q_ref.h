/*
 * fp4q_ref.h -- CPU oracle for block-scaled 4-bit quantization.
 *
 * TEST INFRASTRUCTURE ONLY.  This is a deliberately plain, slow, scalar
 * implementation of what the quantizer computes.  Only the test suite, the
 * smoke check and the CPU-baseline leg of the benchmark may load it.  It
 * shares no code, header, table or constant with the HIP library, and the
 * HIP library never calls it.
 *
 * All tensor pointers are HOST pointers.  Every function returns 0 on
 * success and a negative value for an argument it cannot handle.
 *
 * Sources (page titles as published on gist.science):
 *   [SS]  "ScaleSweep" technical summary: Problem definition; Method
 *         (1 objectives MSE/WMSE, 2 theoretical bounds: global scale
 *         S = max|x|/(256*6), upper bound 12/7 s_base (+7), lower bounds
 *         4/5 s_base (-3, MSE) and 1/2 s_base (-8, WMSE); 3 implementation:
 *         sweep a window of FP8 bit patterns).
 *   [IF4] "Adaptive Block-Scaled Data Types": Methodology (IF4 structure,
 *         indicator in the scale sign bit, the 6/7 method).
 *   [MR]  "Bridging the Gap Between Promise and Performance for
 *         Microscaling FP4 Quantization": Method 1 (block-wise Hadamard);
 *         Problem (MXFP4 power-of-two E8M0 scales, 32-element blocks).
 */
#ifndef FP4Q_REF_H
#define FP4Q_REF_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* numeric codes used by the oracle's own entry points */
enum { REF_NVFP4 = 0, REF_MXFP4 = 1, REF_IF4 = 2, REF_IF3 = 3, REF_IF6 = 4 };
enum { REF_F32 = 0, REF_BF16 = 1 };
enum { REF_ABSMAX = 0, REF_SWEEP = 1, REF_FOUR_SIX = 2 };
enum { REF_MSE = 0, REF_WMSE = 1 };

/* ---- element / scale formats ------------------------------------------ */
float fp4q_ref_e2m1_value(int m);          /* magnitude code 0..7 -> value   */
int   fp4q_ref_e2m1_round(float y);        /* y >= 0 -> nearest code 0..7     */
float fp4q_ref_e4m3_value(int byte);       /* E4M3FN byte (sign honoured)     */
int   fp4q_ref_e4m3_round(float t);        /* t >= 0 -> byte 0x00..0x7E (sat) */
float fp4q_ref_e8m0_value(int byte);       /* 2^(byte-127); 0xFF -> NaN       */
int   fp4q_ref_int4_round(float y);        /* y >= 0 -> nearest integer 0..7  */
float fp4q_ref_bf16_to_f32(uint16_t h);
uint16_t fp4q_ref_f32_to_bf16(float f);    /* round to nearest even            */
float fp4q_ref_int4_step(void);            /* fl32(6/7)                        */

/* ---- IF3 / IF6: the adaptive type at n = 3 and 6 bits ------------------
 * [IF4, Methodology: the idea applies to 3-bit (IF3) and 6-bit (IF6)
 * formats].  Reading: FP element E2M(n-3) (bias 1, exponent field 0
 * subnormal), INT element in [-(2^(n-1)-1), 2^(n-1)-1] with step
 * D * fl32(FPmax/INTmax), E4M3 scale with the indicator in bit 7, base scale
 * E4M3(max/(FPmax S)), S = max|x|/(256 FPmax); n = 4 is exactly IF4.  Codes
 * are n-bit fields, element e at bits n*e .. n*e+n-1 of the code stream. */
float fp4q_ref_fpn_value(int n, int m);    /* magnitude code -> value         */
float fp4q_ref_fpn_max(int n);             /* 4, 6, 7.5 for n = 3, 4, 6       */
int   fp4q_ref_fpn_round(int n, float y);  /* nearest code, even on tie, sat. */
int   fp4q_ref_intn_round(int n, float y); /* nearest 0..2^(n-1)-1, even, sat.*/
float fp4q_ref_ifn_step(int n);            /* fl32(FPmax / INTmax)            */
float fp4q_ref_ifn_global_scale(int n, float g);
int   fp4q_ref_ifn_base_scale(int n, const float* xb, int B, float S);
double fp4q_ref_fpn_block(int n, const float* xb, int B, const float* w, float S,
                          int c, uint8_t* codes);
double fp4q_ref_intn_block(int n, const float* xb, int B, const float* w, float S,
                           int c, uint8_t* codes);

/* ---- transform and global scale --------------------------------------- */
float fp4q_ref_rotation_scale(int n);      /* fl32(1/sqrt(n))                  */
void  fp4q_ref_fwht(float* v, int n);      /* in place, scaled by 1/sqrt(n)   */
float fp4q_ref_global_scale(float g);      /* S from the tensor max G          */

/* widen (bf16 -> f32) and optionally rotate every n-block of a row-major
 * [rows, cols] tensor into out (f32, same shape). */
int fp4q_ref_prepare(const void* x, int x_dtype, int64_t rows, int64_t cols,
                     int rotate, float* out, int nthreads);

/* ---- per-block primitives (used by the brute-force tests) ------------- */
/* NVFP4 encode of one block of widened (and rotated) values with scale
 * byte c (1..126) under global scale S; returns the block error in fp64
 * (importance w may be NULL) and writes B sign|magnitude nibbles to codes
 * (one per byte) when codes != NULL. */
double fp4q_ref_nvfp4_block(const float* xb, int B, const float* w, float S,
                            int c, uint8_t* codes);
/* the AbsMax base scale byte of one block (0 for an all-zero block) */
int fp4q_ref_base_scale(const float* xb, int B, float S);
/* IF4 INT4 branch of one block with FP4 scale byte c; returns the error */
double fp4q_ref_int4_block(const float* xb, int B, const float* w, float S,
                           int c, uint8_t* codes);

/* block errors of every scale byte 1..126 for nblocks prepared blocks laid
 * out back to back; out[b*127 + c] (out[b*127] is NaN).  w, when not NULL,
 * holds B weights per block. */
int fp4q_ref_candidate_errors(const float* xb, int64_t nblocks, int B,
                              const float* w, float S, double* out, int nthreads);

/* ---- whole-tensor entry points ---------------------------------------- */
int fp4q_ref_quantize(int format, int block, int scale_rule, int objective,
                      int sweep_lo, int sweep_hi, int rotate,
                      int global_scale_given,
                      const void* x, int x_dtype, int64_t rows, int64_t cols,
                      const float* importance,
                      uint8_t* codes, uint8_t* scales, float* global_scale,
                      double* best_err, double* second_err, int nthreads);

/* FOCUS deploy-side encode: codes from S_q = S_dq * c (c per `group`
 * elements, group 8 or the block), S_dq stored (AbsMax rule, or read from
 * `scales` when scales_given).  coef: fp32 [rows, cols/group]. */
int fp4q_ref_quantize_relaxed(int format, int block, int global_scale_given,
                              const void* x, int x_dtype, int64_t rows, int64_t cols,
                              const float* coef, int group, int scales_given,
                              uint8_t* codes, uint8_t* scales, float* global_scale,
                              int nthreads);

int fp4q_ref_dequantize(int format, int block, const uint8_t* codes,
                        const uint8_t* scales, const float* global_scale,
                        int64_t rows, int64_t cols, int unrotate,
                        void* y, int y_dtype, int nthreads);

int fp4q_ref_error(int format, int block, int rotate,
                   const void* x, int x_dtype, int64_t rows, int64_t cols,
                   const float* importance, const uint8_t* codes,
                   const uint8_t* scales, const float* global_scale,
                   double out[2], int nthreads);

#ifdef __cplusplus
}
#endif
#endif
