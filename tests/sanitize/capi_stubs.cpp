// capi_stubs.cpp -- stand-ins for the kernel launchers and the two HIP
// runtime calls of the C ABI, so that its host-side argument handling can be
// built and run under -fsanitize=address,undefined without a GPU.  A stub
// records the call and never dereferences a device pointer.
#include <cstring>

#include "fp4q_launch.h"

namespace fp4q {

int stub_launches = 0;

hipError_t static_scratch(hipStream_t, void** out)
{
    static unsigned char fake[1];
    *out = fake; // never dereferenced: the launchers are stubs
    return hipSuccess;
}

hipError_t launch_quantize(const QuantArgs& a)
{
    ++stub_launches;
    return a.rows >= 0 && a.cols >= 0 ? hipSuccess : hipErrorInvalidValue;
}

hipError_t launch_quantize_relaxed(const RelaxArgs& a)
{
    ++stub_launches;
    return a.group > 0 ? hipSuccess : hipErrorInvalidValue;
}

hipError_t launch_dequantize(const DequantArgs&)
{
    ++stub_launches;
    return hipSuccess;
}

hipError_t launch_error(const ErrorArgs&, double*)
{
    ++stub_launches;
    return hipSuccess;
}

} // namespace fp4q

// the two runtime calls fp4q_error makes after its launch
hipError_t hipMemcpyAsync(void* dst, const void*, size_t bytes, hipMemcpyKind, hipStream_t)
{
    std::memset(dst, 0, bytes); // the host destination only
    return hipSuccess;
}

hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
