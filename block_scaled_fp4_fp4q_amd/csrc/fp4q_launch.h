// fp4q_launch.h -- internal interface between the C ABI (fp4q_capi.cpp) and
// the kernel launchers (fp4q_kernels.hip).  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4q {

enum { kNVFP4 = 0, kMXFP4 = 1, kIF4 = 2, kIF3 = 3, kIF6 = 4 };
enum { kAbsMax = 0, kSweep = 1, kFourSix = 2 };
enum { kMSE = 0, kWMSE = 1 };

// workspace layout (bytes): [0, 16384) partial maxima (float, <= 1024) or
// partial error sums (double2, <= 1024); [16384, 16400) the two error sums
constexpr int kErrorGroups = 1024;
constexpr size_t kErrorOutOffset = 16384;
constexpr size_t kWorkspaceBytes = 32768;

struct QuantArgs {
    int format, rule, objective, lo, hi, rotate;
    bool global_scale_given, bf16;
    const void* x;
    int64_t rows, cols;
    const float* importance;
    uint8_t* codes;
    uint8_t* scales;
    float* global_scale;
    void* workspace;
    hipStream_t stream;
};

struct DequantArgs {
    int format, unrotate;
    bool out_bf16;
    const uint8_t* codes;
    const uint8_t* scales;
    const float* global_scale;
    int64_t rows, cols;
    void* y;
    hipStream_t stream;
};

struct ErrorArgs {
    int format, rotate;
    bool bf16;
    const void* x;
    int64_t rows, cols;
    const float* importance;
    const uint8_t* codes;
    const uint8_t* scales;
    const float* global_scale;
    void* workspace;
    hipStream_t stream;
};

// codes from a relaxed step D*c, stored scales unchanged
struct RelaxArgs {
    int format, group;
    bool global_scale_given, scales_given, bf16;
    const void* x;
    int64_t rows, cols;
    const float* coef;
    uint8_t* codes;
    uint8_t* scales;
    float* global_scale;
    void* workspace;
    hipStream_t stream;
};

// Device address, on the GPU that runs `stream` (the current device for the
// null stream), of the library's static scratch array of kWorkspaceBytes:
// the workspace of the entry point that allocates nothing.  Looked up once
// per device and kept.
hipError_t static_scratch(hipStream_t stream, void** out);

hipError_t launch_quantize(const QuantArgs& a);
hipError_t launch_quantize_relaxed(const RelaxArgs& a);
hipError_t launch_dequantize(const DequantArgs& a);
hipError_t launch_error(const ErrorArgs& a, double* out_dev);

} // namespace fp4q
