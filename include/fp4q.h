/*
 * fp4q.h -- C ABI of libfp4q.so: block-scaled 4-bit (FP4) quantization of a
 * tensor with error-minimizing scale selection, for AMD Instinct MI355X
 * (gfx950).
 *
 * Formats (see the pages cited at each entry point):
 *   NVFP4  E2M1 element codes, 16-element blocks, one E4M3 scale byte per
 *          block under one fp32 global scale S.
 *   MXFP4  E2M1 element codes, 32-element blocks, one E8M0 (power-of-two)
 *          scale byte per block, no global scale.
 *   IF4    NVFP4 layout; each block holds either FP4 (E2M1) codes or scaled
 *          INT4 codes, and bit 7 (the sign bit) of its E4M3 scale byte says
 *          which: 0 = FP4, 1 = INT4.
 *   IF3, IF6  the same adaptive pick at 3 and 6 bits (Adaptive Block-Scaled
 *          Data Types page, Methodology, which says the idea applies to
 *          3-bit and 6-bit formats but fixes no grid).  Reading, under which
 *          n = 4 is exactly IF4: the FP element is E2M(n-3) -- sign, two
 *          exponent bits with bias 1, n-3 mantissa bits, no inf/NaN (IF3:
 *          E2M0, magnitudes {0,1,2,4}; IF6: OCP FP6 E2M3, up to 7.5); the
 *          INT element is an integer in [-(2^(n-1)-1), 2^(n-1)-1] (IF3 +-3,
 *          IF6 +-31) on the step D*fl32(FPmax/INTmax), which maps the INT
 *          maximum onto the FP maximum as 6/7 does for IF4; the base scale is
 *          E4M3(max|x| / (FPmax S)) and a computed global scale is
 *          S = max|x| / (256 FPmax) (1024 for IF3, 1920 for IF6).
 *
 * Tensor layout.  x is a row-major [rows, cols] tensor; blocks are `block`
 * consecutive elements of one row (cols % block == 0), numbered in memory
 * order.  A KV cache [B, H, T, D] is passed as [B*H*T, D].
 *   codes   [rows*cols/2] bytes: element 2k in the low nibble of byte k,
 *           element 2k+1 in the high nibble.  An FP4 nibble is
 *           (sign << 3) | magnitude code, magnitudes 0..7 =
 *           {0, 0.5, 1, 1.5, 2, 3, 4, 6}; an INT4 nibble is the 4-bit two's
 *           complement of the integer in [-7, 7].
 *           IF3 / IF6: [rows*cols*n/8] bytes of n-bit codes, element e at
 *           bits n*e .. n*e+n-1 of the stream, least significant bit first
 *           (the nibble layout above is the n = 4 case): 6 bytes per IF3
 *           block, 12 per IF6 block.  An FP code is (sign << (n-1)) |
 *           magnitude code (E2M3: (exponent << 3) | mantissa); an INT code
 *           is the n-bit two's complement.
 *   scales  [rows*cols/block] bytes, one per block in memory order.
 *   S       one fp32 (NVFP4 and IF4 only).
 *
 * Ownership and threading.  Every tensor pointer is a DEVICE pointer owned by
 * the caller, as is the workspace; the library allocates nothing, frees
 * nothing and keeps no state between calls, apart from the static scratch of
 * fp4q_quantize_noalloc.  Calls are asynchronous on the given stream (a
 * hipStream_t passed as void*; NULL is the null stream) except fp4q_error,
 * which waits for its own result.  Two calls may run concurrently only with
 * separate workspaces (fp4q_quantize_noalloc calls: never on one GPU).
 *
 * Errors.  Every entry point returns an fp4q_status.  Argument, shape and
 * alignment errors are detected on the host before anything is launched and
 * leave every output untouched.  A failed launch returns FP4Q_E_HIP.  Faults
 * inside a kernel surface at the caller's next synchronization.
 *
 * An empty tensor (rows == 0 or cols == 0) is valid; its tensor pointers may
 * then be NULL, and a computed global scale is 1.
 *
 * Preconditions (not checked, results unspecified otherwise): inputs are
 * finite; importance weights are finite and non-negative (zero allowed); a
 * caller-supplied global scale is a normal fp32 in [2^-117, 2^119]; output
 * buffers do not overlap inputs.
 */
#ifndef FP4Q_H
#define FP4Q_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP4Q_ABI_VERSION 3

typedef enum {
    FP4Q_OK = 0,
    FP4Q_E_NULL = -1,        /* a required pointer is NULL                   */
    FP4Q_E_ARG = -2,         /* bad enum, window, rotation or workspace size */
    FP4Q_E_SHAPE = -3,       /* negative sizes or cols % block != 0          */
    FP4Q_E_UNSUPPORTED = -4, /* a combination outside the methods' scope     */
    FP4Q_E_HIP = -5,         /* the HIP runtime refused a launch or copy     */
    FP4Q_E_ALIGN = -6,       /* a tensor pointer is not aligned as required  */
    FP4Q_E_SCRATCH = -7      /* more scratch than fp4q_quantize_noalloc has  */
} fp4q_status;

typedef enum { FP4Q_NVFP4 = 0, FP4Q_MXFP4 = 1, FP4Q_IF4 = 2, FP4Q_IF3 = 3, FP4Q_IF6 = 4 } fp4q_format;
typedef enum { FP4Q_F32 = 0, FP4Q_BF16 = 1 } fp4q_dtype;
typedef enum {
    FP4Q_SCALE_ABSMAX = 0,
    FP4Q_SCALE_SWEEP = 1,
    FP4Q_SCALE_FOUR_OVER_SIX = 2
} fp4q_scale_rule;
typedef enum { FP4Q_OBJ_MSE = 0, FP4Q_OBJ_WMSE = 1 } fp4q_objective;

/* The problem statement of one quantization.
 *   format      fp4q_format.
 *   block       16 for NVFP4, IF4, IF3 and IF6, 32 for MXFP4.
 *   scale_rule  ABSMAX: the block scale is the block maximum mapped onto the
 *               FP4 maximum 6 and rounded to FP8 ("AbsMax", ScaleSweep page,
 *               Problem definition).
 *               SWEEP: a window of scales around the AbsMax one is tried and
 *               the one of least block error kept.
 *                 NVFP4: ScaleSweep -- every E4M3 bit pattern s_base + k,
 *                 k in [sweep_lo, sweep_hi] (ScaleSweep page, Method 2 and 3).
 *                 MXFP4: every E8M0 exponent e_base + k ("Bridging the Gap
 *                 ... Microscaling FP4" page, Method 2, format-specific
 *                 scale search).
 *                 IF4, IF3, IF6: every pattern s_base + k, each with the FP
 *                 grid then with the INT grid (the pick of the Adaptive
 *                 Block-Scaled Data Types page, Methodology, run at every
 *                 pattern of the window).
 *               FOUR_OVER_SIX (NVFP4 only): the block maximum is mapped onto
 *               6 or onto 4, E4M3(a / (6 S)) vs E4M3(a / (4 S)), and the one
 *               of lower block error kept, 6 on a tie (Adaptive Block-Scaled
 *               Data Types page, Problem; ScaleSweep page, Problem definition).
 *               Every choice compares binary64 block errors of the binary32
 *               encodes; an exact tie keeps the candidate tried first.
 *   objective   MSE, or WMSE weighted by a per-column importance vector
 *               (ScaleSweep page, Method 1).  Used wherever block errors
 *               decide: SWEEP, FOUR_OVER_SIX and the FP-vs-INT pick of IF4,
 *               IF3 and IF6.
 *   sweep_lo, sweep_hi
 *               the window of offsets, -126 <= lo <= hi <= 126; the pages use
 *               [-3, 7] for MSE and [-8, 7] for WMSE (NVFP4).  An offset that
 *               leads past the ends of the scale range (E4M3 patterns 0x01 and
 *               0x7E, E8M0 exponents -127 and 127) stands for that end, and
 *               each scale is tried once.
 *   rotate      0, or equal to block: apply the orthonormal Sylvester block
 *               Hadamard transform to every block before quantizing
 *               ("Bridging the Gap ... Microscaling FP4" page, Method 1).
 *   global_scale_given
 *               0: S = max|x| / (256*6) is computed on the device (ScaleSweep
 *               page, Method 2) and written to *global_scale; 1: *global_scale
 *               is read as S.  Ignored for MXFP4. */
typedef struct {
    int32_t format;
    int32_t block;
    int32_t scale_rule;
    int32_t objective;
    int32_t sweep_lo;
    int32_t sweep_hi;
    int32_t rotate;
    int32_t global_scale_given;
} fp4q_spec;

/* Bytes of device workspace that fp4q_quantize and fp4q_error need for this
 * problem (at least 256; the workspace must be 256-byte aligned).  Returns 0
 * for an invalid spec. */
size_t fp4q_workspace_bytes(const fp4q_spec* spec, int64_t rows, int64_t cols);

/* Quantize x [rows, cols] (dtype FP4Q_F32 or FP4Q_BF16; 16-byte aligned).
 *   importance  fp32 [cols] per-input-column weights, required for WMSE,
 *               ignored otherwise (may be NULL); 16-byte aligned wherever it
 *               is used (it is read four weights at a time), else
 *               FP4Q_E_ALIGN.
 *   codes       [rows*cols/2] bytes, 8-byte aligned (16 for MXFP4); IF3
 *               [rows*cols*3/8] bytes, 2-byte aligned; IF6 [rows*cols*3/4]
 *               bytes, 4-byte aligned.
 *   scales      [rows*cols/block] bytes.
 *   global_scale  one fp32: output (or input when global_scale_given); may be
 *               NULL for MXFP4.
 *   workspace   device scratch of fp4q_workspace_bytes() bytes.
 * Per block (ScaleSweep page, Method; Adaptive Block-Scaled Data Types page,
 * Methodology): the block maximum a gives the base scale
 * s_base = E4M3(a / (6 S)) (at least 0x01; an all-zero block gets scale 0 and
 * sign-only codes); each element is encoded as the nearest E2M1 value of
 * |x| * fl32(1 / fl32(s S)) (ties to the even code, saturating at 6).  IF4
 * also encodes the block as integers q = round(|x| / (D 6/7)) clamped to 7
 * and keeps INT4 only when its error is strictly lower; IF3 and IF6 do the
 * same with their own grids, maxima and steps (see the formats above), the
 * errors compared in binary64.  MXFP4 uses the
 * power of two 2^(floor(log2 a) - 2).  SWEEP and FOUR_OVER_SIX then choose
 * among the scales listed at fp4q_spec. */
fp4q_status fp4q_quantize(const fp4q_spec* spec, const void* x, int32_t x_dtype,
                          int64_t rows, int64_t cols, const float* importance,
                          uint8_t* codes, uint8_t* scales, float* global_scale,
                          void* workspace, size_t ws_bytes, void* stream);

/* fp4q_quantize for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The arguments are fp4q_quantize's without the workspace, and the results
 * are the same.  The scratch fp4q_quantize takes from the workspace (the
 * partial maxima of the global-scale pass) is instead a static device array
 * of FP4Q_NOALLOC_SCRATCH_BYTES inside the library: each GPU it runs on
 * holds its own copy until the process ends.  The first call on a GPU looks
 * up that array's address there; no call allocates or frees anything.
 *   Limit: problems whose fp4q_workspace_bytes() exceeds
 *   FP4Q_NOALLOC_SCRATCH_BYTES are refused with FP4Q_E_SCRATCH (in this
 *   version every valid problem needs exactly that much, so none is).
 *   Sharing: every call on one GPU uses the same array and leaves its
 *   contents behind (nothing in it needs to start at zero).  Calls that
 *   overlap on one GPU -- on two streams, or from two host threads -- race
 *   on it and must be serialized by the caller. */
#define FP4Q_NOALLOC_SCRATCH_BYTES 32768
fp4q_status fp4q_quantize_noalloc(const fp4q_spec* spec, const void* x, int32_t x_dtype,
                                  int64_t rows, int64_t cols, const float* importance,
                                  uint8_t* codes, uint8_t* scales, float* global_scale,
                                  void* stream);

/* Deploy-side encode of FOCUS (FOCUS page, Method 2, coupled-relaxation
 * scaling: the quantization scale S_q = S_dq c while the stored
 * dequantization scale stays S_dq; Method 3, dual-granularity scaling: one
 * coefficient c per sub-block of 8 under a shared S_dq).  spec->format is
 * NVFP4 or MXFP4 (the adaptive formats give FP4Q_E_UNSUPPORTED),
 * spec->rotate 0; scale_rule, objective and the window are ignored;
 * global_scale_given as for fp4q_quantize.
 *   coef        fp32 [rows, cols / coef_group], positive and finite, the
 *               learned relaxation coefficients; row-major, so block b of a
 *               row owns coef[row][b*block/coef_group ...].
 *   coef_group  8 (dual granularity) or spec->block (one per block).
 *   scales_given 0: S_dq is the AbsMax scale (as fp4q_quantize with
 *               FP4Q_SCALE_ABSMAX) and is written to scales; 1: scales is an
 *               input of finite non-negative bytes (E4M3 0x00..0x7E, E8M0
 *               0x00..0xFE) and is not written.
 * Per element, with D the step of S_dq (fl32(s S), or 2^(byte-127)):
 * D_q = fl32(D c), code = E2M1 nearest to fl32(|x| fl32(1 / D_q)), ties to
 * the even code, saturating at 6; a block with D = 0 gets sign-only codes, and
 * so does every zero element (also where D_q < 2^-128 makes fl32(1 / D_q)
 * infinite, since |x| / D_q = 0).
 * fp4q_dequantize of the result applies S_dq, as the method intends.
 * Alignment: x 16, codes 8 (16 for MXFP4), coef 4, workspace 256 bytes. */
fp4q_status fp4q_quantize_relaxed(const fp4q_spec* spec, const void* x, int32_t x_dtype,
                                  int64_t rows, int64_t cols, const float* coef,
                                  int32_t coef_group, int32_t scales_given,
                                  uint8_t* codes, uint8_t* scales, float* global_scale,
                                  void* workspace, size_t ws_bytes, void* stream);

/* Dequantize codes/scales/S into y [rows, cols] (y_dtype FP4Q_F32 or
 * FP4Q_BF16, 16-byte aligned): x_hat = +-value(code) * D, D = fl32(s S) for
 * NVFP4/IF4 (fl32(D * fl32(6/7)) for IF4 INT4 blocks, the 6/7 method) or
 * 2^(byte-127) for MXFP4; IF3 / IF6 INT blocks use D*fl32(4/3) and
 * D*fl32(7.5/31); unrotate (0 or block) applies the block Hadamard,
 * which is its own inverse.  bf16 output is rounded to nearest even.
 * Alignment: y 16, codes 8 (16 for MXFP4, 4 for IF6, 2 for IF3), global_scale
 * 4 bytes. */
fp4q_status fp4q_dequantize(const fp4q_spec* spec, const uint8_t* codes,
                            const uint8_t* scales, const float* global_scale,
                            int64_t rows, int64_t cols, int32_t unrotate,
                            void* y, int32_t y_dtype, void* stream);

/* Reconstruction error in the caller's (un-rotated) domain:
 * out_host[0] = sum (x - x_hat)^2 / N, out_host[1] = sum w_col (x - x_hat)^2
 * / N (NaN when importance is NULL), accumulated in fp64 (ScaleSweep page,
 * Method 1: MSE and WMSE).  x_hat is the dequantized tensor, un-rotated when
 * spec->rotate is set.  Blocks until the two doubles are on the host.
 * Alignment: x 16, codes 8 (16 for MXFP4, 4 for IF6, 2 for IF3), workspace
 * 256, global_scale and importance 4 bytes. */
fp4q_status fp4q_error(const fp4q_spec* spec, const void* x, int32_t x_dtype,
                       int64_t rows, int64_t cols, const float* importance,
                       const uint8_t* codes, const uint8_t* scales,
                       const float* global_scale, void* workspace, size_t ws_bytes,
                       double out_host[2], void* stream);

const char* fp4q_status_string(fp4q_status status);
int fp4q_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* FP4Q_H */
