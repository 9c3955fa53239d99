// fp4q_capi.cpp -- the C ABI declared in include/fp4q.h.
//
// Every argument is validated on the host before anything reaches the HIP
// runtime, so a rejected call launches nothing and touches no output.
#include "fp4q.h"

#include <hip/hip_runtime.h>

#include <cmath>

#include "fp4q_launch.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int block_of(int32_t format) { return format == FP4Q_MXFP4 ? 32 : 16; }

bool is_adaptive(int32_t format)
{
    return format == FP4Q_IF4 || format == FP4Q_IF3 || format == FP4Q_IF6;
}

// alignment of the codes pointer: one block's codes are read and written as
// 8 (NVFP4, IF4), 16 (MXFP4), 12 (IF6, as 32-bit words) or 6 bytes (IF3, as
// 16-bit halves)
uintptr_t codes_align(int32_t format)
{
    switch (format) {
    case FP4Q_MXFP4: return 16;
    case FP4Q_IF6: return 4;
    case FP4Q_IF3: return 2;
    default: return 8;
    }
}

// common checks of a spec; the window is only meaningful for SWEEP
fp4q_status check_spec(const fp4q_spec* s, bool for_quantize)
{
    if (!s)
        return FP4Q_E_NULL;
    if (s->format != FP4Q_NVFP4 && s->format != FP4Q_MXFP4 && !is_adaptive(s->format))
        return FP4Q_E_ARG;
    if (s->block != block_of(s->format))
        return FP4Q_E_UNSUPPORTED;
    if (s->rotate != 0 && s->rotate != s->block)
        return FP4Q_E_ARG;
    if (!for_quantize)
        return FP4Q_OK;
    if (s->scale_rule != FP4Q_SCALE_ABSMAX && s->scale_rule != FP4Q_SCALE_SWEEP &&
        s->scale_rule != FP4Q_SCALE_FOUR_OVER_SIX)
        return FP4Q_E_ARG;
    if (s->objective != FP4Q_OBJ_MSE && s->objective != FP4Q_OBJ_WMSE)
        return FP4Q_E_ARG;
    if (s->global_scale_given != 0 && s->global_scale_given != 1)
        return FP4Q_E_ARG;
    if (s->scale_rule == FP4Q_SCALE_FOUR_OVER_SIX && s->format != FP4Q_NVFP4)
        return FP4Q_E_UNSUPPORTED;
    if (s->scale_rule == FP4Q_SCALE_SWEEP &&
        (s->sweep_lo > s->sweep_hi || s->sweep_lo < -126 || s->sweep_hi > 126))
        return FP4Q_E_ARG;
    return FP4Q_OK;
}

fp4q_status check_shape(int64_t rows, int64_t cols, int block)
{
    if (rows < 0 || cols < 0)
        return FP4Q_E_SHAPE;
    if (cols % block != 0)
        return FP4Q_E_SHAPE;
    if (cols != 0 && rows > INT64_MAX / cols)
        return FP4Q_E_SHAPE;
    return FP4Q_OK;
}

bool valid_dtype(int32_t d) { return d == FP4Q_F32 || d == FP4Q_BF16; }

// checks of every fp4q_quantize argument except the workspace, and the
// launch arguments they describe (workspace and stream left to the caller)
fp4q_status check_quantize(const fp4q_spec* spec, const void* x, int32_t x_dtype, int64_t rows,
                           int64_t cols, const float* importance, uint8_t* codes, uint8_t* scales,
                           float* global_scale, fp4q::QuantArgs& a)
{
    fp4q_status st = check_spec(spec, true);
    if (st != FP4Q_OK)
        return st;
    if ((st = check_shape(rows, cols, spec->block)) != FP4Q_OK)
        return st;
    if (!valid_dtype(x_dtype))
        return FP4Q_E_ARG;
    const bool has_gs = spec->format != FP4Q_MXFP4;
    // the weights matter wherever a block error decides between candidates
    const bool wants_imp = spec->objective == FP4Q_OBJ_WMSE &&
                           (spec->scale_rule != FP4Q_SCALE_ABSMAX || is_adaptive(spec->format));
    const bool empty = rows == 0 || cols == 0; // tensor pointers may then be NULL
    if ((!empty && (!x || !codes || !scales)) || (has_gs && !global_scale) ||
        (wants_imp && !empty && !importance))
        return FP4Q_E_NULL;
    if (!aligned(x, 16) || !aligned(codes, codes_align(spec->format)) ||
        (wants_imp && !aligned(importance, 16)) || (has_gs && !aligned(global_scale, 4)))
        return FP4Q_E_ALIGN;
    a.format = spec->format;
    a.rule = spec->scale_rule == FP4Q_SCALE_SWEEP ? fp4q::kSweep
           : spec->scale_rule == FP4Q_SCALE_FOUR_OVER_SIX ? fp4q::kFourSix : fp4q::kAbsMax;
    a.objective = wants_imp ? fp4q::kWMSE : fp4q::kMSE;
    a.lo = spec->sweep_lo;
    a.hi = spec->sweep_hi;
    a.rotate = spec->rotate;
    a.global_scale_given = spec->global_scale_given != 0;
    a.bf16 = x_dtype == FP4Q_BF16;
    a.x = x;
    a.rows = rows;
    a.cols = cols;
    a.importance = wants_imp ? importance : nullptr;
    a.codes = codes;
    a.scales = scales;
    a.global_scale = global_scale;
    return FP4Q_OK;
}

} // namespace

extern "C" {

int fp4q_abi_version(void) { return FP4Q_ABI_VERSION; }

const char* fp4q_status_string(fp4q_status s)
{
    switch (s) {
    case FP4Q_OK: return "ok";
    case FP4Q_E_NULL: return "a required pointer is NULL";
    case FP4Q_E_ARG: return "invalid argument (enum, window, rotation or workspace size)";
    case FP4Q_E_SHAPE: return "invalid shape (negative size, or cols not a multiple of the block)";
    case FP4Q_E_UNSUPPORTED: return "unsupported combination (block size, Four Over Six outside NVFP4, relaxed encode of IF3/IF4/IF6 or with rotation)";
    case FP4Q_E_HIP: return "the HIP runtime refused a launch or copy";
    case FP4Q_E_ALIGN: return "a tensor pointer is not aligned as required";
    case FP4Q_E_SCRATCH: return "the problem needs more scratch than fp4q_quantize_noalloc holds";
    }
    return "unknown status";
}

size_t fp4q_workspace_bytes(const fp4q_spec* spec, int64_t rows, int64_t cols)
{
    if (check_spec(spec, false) != FP4Q_OK || check_shape(rows, cols, spec->block) != FP4Q_OK)
        return 0;
    return fp4q::kWorkspaceBytes;
}

fp4q_status fp4q_quantize(const fp4q_spec* spec, const void* x, int32_t x_dtype, int64_t rows,
                          int64_t cols, const float* importance, uint8_t* codes, uint8_t* scales,
                          float* global_scale, void* workspace, size_t ws_bytes, void* stream)
{
    fp4q::QuantArgs a{};
    fp4q_status st = check_quantize(spec, x, x_dtype, rows, cols, importance, codes, scales,
                                    global_scale, a);
    if (st != FP4Q_OK)
        return st;
    if (!workspace)
        return FP4Q_E_NULL;
    if (ws_bytes < fp4q::kWorkspaceBytes)
        return FP4Q_E_ARG;
    if (!aligned(workspace, 256))
        return FP4Q_E_ALIGN;
    a.workspace = workspace;
    a.stream = static_cast<hipStream_t>(stream);
    return fp4q::launch_quantize(a) == hipSuccess ? FP4Q_OK : FP4Q_E_HIP;
}

fp4q_status fp4q_quantize_noalloc(const fp4q_spec* spec, const void* x, int32_t x_dtype,
                                  int64_t rows, int64_t cols, const float* importance,
                                  uint8_t* codes, uint8_t* scales, float* global_scale,
                                  void* stream)
{
    fp4q::QuantArgs a{};
    fp4q_status st = check_quantize(spec, x, x_dtype, rows, cols, importance, codes, scales,
                                    global_scale, a);
    if (st != FP4Q_OK)
        return st;
    if (fp4q_workspace_bytes(spec, rows, cols) > (size_t)FP4Q_NOALLOC_SCRATCH_BYTES)
        return FP4Q_E_SCRATCH;
    a.stream = static_cast<hipStream_t>(stream);
    if (fp4q::static_scratch(a.stream, &a.workspace) != hipSuccess)
        return FP4Q_E_HIP;
    return fp4q::launch_quantize(a) == hipSuccess ? FP4Q_OK : FP4Q_E_HIP;
}

fp4q_status fp4q_quantize_relaxed(const fp4q_spec* spec, const void* x, int32_t x_dtype,
                                  int64_t rows, int64_t cols, const float* coef, int32_t coef_group,
                                  int32_t scales_given, uint8_t* codes, uint8_t* scales,
                                  float* global_scale, void* workspace, size_t ws_bytes, void* stream)
{
    fp4q_status st = check_spec(spec, false);
    if (st != FP4Q_OK)
        return st;
    if ((st = check_shape(rows, cols, spec->block)) != FP4Q_OK)
        return st;
    if (is_adaptive(spec->format) || spec->rotate != 0)
        return FP4Q_E_UNSUPPORTED;
    if (!valid_dtype(x_dtype) || (coef_group != 8 && coef_group != spec->block) ||
        (scales_given != 0 && scales_given != 1) ||
        (spec->global_scale_given != 0 && spec->global_scale_given != 1))
        return FP4Q_E_ARG;
    const bool has_gs = spec->format != FP4Q_MXFP4;
    const bool empty = rows == 0 || cols == 0;
    if ((!empty && (!x || !coef || !codes || !scales)) || !workspace || (has_gs && !global_scale))
        return FP4Q_E_NULL;
    if (ws_bytes < fp4q::kWorkspaceBytes)
        return FP4Q_E_ARG;
    if (!aligned(x, 16) || !aligned(codes, spec->block == 32 ? 16 : 8) || !aligned(coef, 4) ||
        !aligned(workspace, 256) || (has_gs && !aligned(global_scale, 4)))
        return FP4Q_E_ALIGN;
    fp4q::RelaxArgs a{};
    a.format = spec->format;
    a.group = coef_group;
    a.global_scale_given = spec->global_scale_given != 0;
    a.scales_given = scales_given != 0;
    a.bf16 = x_dtype == FP4Q_BF16;
    a.x = x;
    a.rows = rows;
    a.cols = cols;
    a.coef = coef;
    a.codes = codes;
    a.scales = scales;
    a.global_scale = global_scale;
    a.workspace = workspace;
    a.stream = static_cast<hipStream_t>(stream);
    return fp4q::launch_quantize_relaxed(a) == hipSuccess ? FP4Q_OK : FP4Q_E_HIP;
}

fp4q_status fp4q_dequantize(const fp4q_spec* spec, const uint8_t* codes, const uint8_t* scales,
                            const float* global_scale, int64_t rows, int64_t cols, int32_t unrotate,
                            void* y, int32_t y_dtype, void* stream)
{
    fp4q_status st = check_spec(spec, false);
    if (st != FP4Q_OK)
        return st;
    if ((st = check_shape(rows, cols, spec->block)) != FP4Q_OK)
        return st;
    if (!valid_dtype(y_dtype) || (unrotate != 0 && unrotate != spec->block))
        return FP4Q_E_ARG;
    const bool has_gs = spec->format != FP4Q_MXFP4;
    const bool empty = rows == 0 || cols == 0;
    if ((!empty && (!codes || !scales || !y)) || (has_gs && !empty && !global_scale))
        return FP4Q_E_NULL;
    if (!aligned(codes, codes_align(spec->format)) || !aligned(y, 16) ||
        (has_gs && !aligned(global_scale, 4)))
        return FP4Q_E_ALIGN;
    fp4q::DequantArgs a{};
    a.format = spec->format;
    a.unrotate = unrotate;
    a.out_bf16 = y_dtype == FP4Q_BF16;
    a.codes = codes;
    a.scales = scales;
    a.global_scale = global_scale;
    a.rows = rows;
    a.cols = cols;
    a.y = y;
    a.stream = static_cast<hipStream_t>(stream);
    return fp4q::launch_dequantize(a) == hipSuccess ? FP4Q_OK : FP4Q_E_HIP;
}

fp4q_status fp4q_error(const fp4q_spec* spec, const void* x, int32_t x_dtype, int64_t rows,
                       int64_t cols, const float* importance, const uint8_t* codes,
                       const uint8_t* scales, const float* global_scale, void* workspace,
                       size_t ws_bytes, double out_host[2], void* stream)
{
    fp4q_status st = check_spec(spec, false);
    if (st != FP4Q_OK)
        return st;
    if ((st = check_shape(rows, cols, spec->block)) != FP4Q_OK)
        return st;
    if (!valid_dtype(x_dtype))
        return FP4Q_E_ARG;
    const bool has_gs = spec->format != FP4Q_MXFP4;
    const bool empty = rows == 0 || cols == 0;
    if ((!empty && (!x || !codes || !scales || (has_gs && !global_scale))) || !workspace || !out_host)
        return FP4Q_E_NULL;
    if (ws_bytes < fp4q::kWorkspaceBytes)
        return FP4Q_E_ARG;
    if (!aligned(x, 16) || !aligned(codes, codes_align(spec->format)) || !aligned(workspace, 256) ||
        (has_gs && !aligned(global_scale, 4)) || !aligned(importance, 4))
        return FP4Q_E_ALIGN;
    fp4q::ErrorArgs a{};
    a.format = spec->format;
    a.rotate = spec->rotate;
    a.bf16 = x_dtype == FP4Q_BF16;
    a.x = x;
    a.rows = rows;
    a.cols = cols;
    a.importance = importance;
    a.codes = codes;
    a.scales = scales;
    a.global_scale = global_scale;
    a.workspace = workspace;
    a.stream = static_cast<hipStream_t>(stream);
    double* out_dev = reinterpret_cast<double*>(static_cast<char*>(workspace) + fp4q::kErrorOutOffset);
    if (fp4q::launch_error(a, out_dev) != hipSuccess)
        return FP4Q_E_HIP;
    if (hipMemcpyAsync(out_host, out_dev, 2 * sizeof(double), hipMemcpyDeviceToHost, a.stream) != hipSuccess)
        return FP4Q_E_HIP;
    if (hipStreamSynchronize(a.stream) != hipSuccess)
        return FP4Q_E_HIP;
    return FP4Q_OK;
}

} // extern "C"
