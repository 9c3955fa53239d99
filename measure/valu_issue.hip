// valu_issue.hip -- issue cost of the VALU instructions the quantizers are
// built from, measured on the device this runs on, and of two that a cheaper
// error estimate would need (a decode to packed f16 and a binary32 fma with
// an f16 operand).  Binary32 fma, mul, add and sub issue at twice the rate of
// most other VALU instructions on this chip (rounding, min/max, integer and
// bit operations, f16), so one representative of that slower class each
// (v_rndne_f32, v_min_f32, v_add_u32) is measured too, written as single
// inline-asm instructions so that the compiler cannot fold the chains.
//
// Each kernel keeps eight independent dependency chains per lane and runs
// eight waves per SIMD, so the SIMD always has an instruction ready and the
// time per instruction is its issue cost, not its latency.  The loop body is
// 64 instructions of one kind (a short loop adds branch overhead that a long
// straight-line kernel body does not have).  The core clock
// during each kernel is read from the shader-clock counter (s_memtime) against
// the 100 MHz real-time counter (s_memrealtime); a ~0.3 s warm-up precedes the
// measurements so that the clock has settled.  Printed: one JSON line with the
// clock and the cost of one wave64 instruction in core-clock cycles per SIMD.
//
// This is a measurement tool for the quantizers' VALU roofline, not part of
// the library.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <vector>

namespace {

constexpr int kThreads = 256;
constexpr int kChains = 8;

enum Kind { kFma32, kMul32, kEncode, kDecodeXor, kXor, kFma64, kDecodeF16Xor, kFmaMix, kRndne32, kMin32, kAddU32 };

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

template <int KIND>
__global__ __launch_bounds__(kThreads) void chains(uint32_t* __restrict__ out, uint64_t* __restrict__ clk,
                                                    int iters, float seed)
{
    float f[kChains], g[kChains];
    uint32_t u[kChains];
    double d[kChains];
#pragma unroll
    for (int i = 0; i < kChains; ++i) {
        f[i] = seed * (float)(threadIdx.x + i + 1);
        g[i] = 0.5f + 0.01f * (float)i;
        u[i] = (threadIdx.x + 1u) * 2654435761u + (uint32_t)i;
        d[i] = (double)f[i];
    }
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
#pragma unroll 8
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < kChains; ++i) {
            if constexpr (KIND == kFma32)
                f[i] = __builtin_fmaf(g[i], 0.999f, f[i]);
            if constexpr (KIND == kMul32)
                f[i] = f[i] * g[i];
            if constexpr (KIND == kEncode)
                u[i] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(u[i], f[i], g[i], 1.0f, 0);
            if constexpr (KIND == kDecodeXor) {
                const auto t = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(u[i], 1.0f, 0);
                u[i] ^= __float_as_uint(t[0]);
            }
            if constexpr (KIND == kDecodeF16Xor) { // decode to two packed f16 values
                const half2_t t = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(u[i], 1.0f, 0);
                u[i] ^= __builtin_bit_cast(uint32_t, t);
            }
            if constexpr (KIND == kFmaMix) { // binary32 fma with one f16 operand
                const half2_t t = __builtin_bit_cast(half2_t, __float_as_uint(f[(i + 1) % kChains]));
                f[i] = __builtin_fmaf(g[i], (float)t[1], f[i]);
            }
            if constexpr (KIND == kXor)
                u[i] ^= u[(i + 1) % kChains];
            if constexpr (KIND == kFma64)
                d[i] = __builtin_fma(d[i], 0.999, 0.001);
            if constexpr (KIND == kRndne32)
                asm volatile("v_rndne_f32 %0, %0" : "+v"(f[i]));
            if constexpr (KIND == kMin32)
                asm volatile("v_min_f32 %0, %0, %1" : "+v"(f[i]) : "v"(g[i]));
            if constexpr (KIND == kAddU32)
                asm volatile("v_add_u32 %0, %0, %1" : "+v"(u[i]) : "v"(u[(i + 1) % kChains]));
        }
    }
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    uint32_t acc = 0;
#pragma unroll
    for (int i = 0; i < kChains; ++i)
        acc ^= u[i] ^ __float_as_uint(f[i]) ^ (uint32_t)__double_as_longlong(d[i]);
    out[(size_t)blockIdx.x * kThreads + threadIdx.x] = acc; // out holds grid * kThreads words
    if (threadIdx.x == 0) {
        clk[2 * (size_t)blockIdx.x] = t1 - t0; // clk holds 2 * grid words
        clk[2 * (size_t)blockIdx.x + 1] = r1 - r0;
    }
}

#define CHECK(call)                                                                       \
    do {                                                                                  \
        hipError_t e_ = (call);                                                           \
        if (e_ != hipSuccess) {                                                           \
            fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));                    \
            return -1.0;                                                                  \
        }                                                                                 \
    } while (0)

struct Setup {
    int grid, simds;
    uint32_t* out;
    uint64_t* clk;
    double clock_hz; // of the last measurement
};

// mean time of `reps` launches, and the core clock seen by the waves
template <int KIND>
double run(Setup& s, int iters, int reps)
{
    hipEvent_t a, b;
    CHECK(hipEventCreate(&a));
    CHECK(hipEventCreate(&b));
    hipLaunchKernelGGL(chains<KIND>, dim3(s.grid), dim3(kThreads), 0, 0, s.out, s.clk, iters, 1.0f);
    CHECK(hipGetLastError());
    CHECK(hipEventRecord(a, 0));
    for (int r = 0; r < reps; ++r)
        hipLaunchKernelGGL(chains<KIND>, dim3(s.grid), dim3(kThreads), 0, 0, s.out, s.clk, iters, 1.0f);
    CHECK(hipGetLastError());
    CHECK(hipEventRecord(b, 0));
    CHECK(hipEventSynchronize(b));
    float ms = 0.0f;
    CHECK(hipEventElapsedTime(&ms, a, b));
    std::vector<uint64_t> c(2 * (size_t)s.grid);
    CHECK(hipMemcpy(c.data(), s.clk, c.size() * sizeof(uint64_t), hipMemcpyDeviceToHost));
    double cyc = 0.0, rt = 0.0;
    for (int i = 0; i < s.grid; ++i) {
        cyc += (double)c[2 * i];
        rt += (double)c[2 * i + 1];
    }
    s.clock_hz = rt > 0.0 ? cyc / rt * 100e6 : 0.0; // s_memrealtime ticks at 100 MHz
    CHECK(hipEventDestroy(a));
    CHECK(hipEventDestroy(b));
    return ms / reps * 1e-3;
}

// core-clock cycles one SIMD spends per wave64 instruction of the kernel
template <int KIND>
double cost(Setup& s, int iters, int reps, double instr_per_chain_step)
{
    const double sec = run<KIND>(s, iters, reps);
    const double waves = (double)s.grid * (kThreads / 64);
    const double instr = waves * iters * kChains * instr_per_chain_step;
    return sec * s.clock_hz * s.simds / instr;
}

} // namespace

int main()
{
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, 0) != hipSuccess) {
        fprintf(stderr, "no device\n");
        return 2;
    }
    Setup s;
    s.simds = p.multiProcessorCount * 4;
    s.grid = p.multiProcessorCount * 8; // eight waves per SIMD
    s.clock_hz = 0.0;
    if (hipMalloc(&s.out, sizeof(uint32_t) * (size_t)s.grid * kThreads) != hipSuccess ||
        hipMalloc(&s.clk, sizeof(uint64_t) * 2 * (size_t)s.grid) != hipSuccess) {
        fprintf(stderr, "hipMalloc failed\n");
        return 2;
    }
    const int iters = 16384;
    // warm-up: ~0.3 s of sustained VALU load
    if (run<kFma32>(s, iters, 300) < 0.0)
        return 1;
    const double fma = cost<kFma32>(s, iters, 20, 1.0);
    const double fma_clk = s.clock_hz;
    const double mul = cost<kMul32>(s, iters, 20, 1.0);
    const double enc = cost<kEncode>(s, iters, 20, 1.0);
    const double enc_clk = s.clock_hz;
    const double dx = cost<kDecodeXor>(s, iters, 20, 1.0);
    const double x = cost<kXor>(s, iters, 20, 1.0);
    const double f64 = cost<kFma64>(s, iters / 4, 20, 1.0);
    const double dhx = cost<kDecodeF16Xor>(s, iters, 20, 1.0);
    const double mix = cost<kFmaMix>(s, iters, 20, 1.0);
    const double rnd = cost<kRndne32>(s, iters, 20, 1.0);
    const double mn = cost<kMin32>(s, iters, 20, 1.0);
    const double au = cost<kAddU32>(s, iters, 20, 1.0);
    if (fma < 0.0 || mul < 0.0 || enc < 0.0 || dx < 0.0 || x < 0.0 || f64 < 0.0 || dhx < 0.0 || mix < 0.0 ||
        rnd < 0.0 || mn < 0.0 || au < 0.0)
        return 1;
    printf("{\"device\": \"%s\", \"simds\": %d, \"clock_ghz_fma32\": %.3f, \"clock_ghz_encode\": %.3f, "
           "\"cycles_per_wave64_instr\": {\"v_fma_f32\": %.3f, \"v_mul_f32\": %.3f, "
           "\"v_cvt_scalef32_pk_fp4_f32\": %.3f, \"v_cvt_scalef32_pk_f32_fp4\": %.3f, "
           "\"v_xor_b32\": %.3f, \"v_fma_f64\": %.3f, \"v_cvt_scalef32_pk_f16_fp4\": %.3f, "
           "\"v_fma_mix_f32\": %.3f, \"v_rndne_f32\": %.3f, \"v_min_f32\": %.3f, \"v_add_u32\": %.3f}}\n",
           p.gcnArchName, s.simds, fma_clk * 1e-9, enc_clk * 1e-9, fma, mul, enc, dx - x, x, f64, dhx - x, mix,
           rnd, mn, au);
    (void)hipFree(s.out);
    (void)hipFree(s.clk);
    return 0;
}
