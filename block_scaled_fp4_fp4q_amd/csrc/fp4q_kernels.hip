// fp4q_kernels.hip -- HIP kernels for block-scaled 4-bit quantization on
// gfx950 (MI355X), and the host launchers the C ABI calls.
//
// Data flow of one quantize call (NVFP4 / IF4 with a computed global scale):
//   amax_*      one read of x (rotated on the fly when asked) -> one partial
//               maximum per workgroup in the workspace;
//   finalize    one workgroup reduces the partials to G and writes
//               S = max(G/1536, 2^-117) (1 for G == 0) to the caller's
//               global_scale (ScaleSweep page, Method 2: S = max|x|/(256*6));
//   *_quant     one lane per block: load + widen, optional Hadamard, block
//               max, base scale, candidate search, encode, packed store.
// MXFP4 and a caller-supplied S skip the first two kernels.
//
// Block decisions are exact: candidate errors are accumulated in binary64
// over the same binary32 encode sequence the method defines, and ties keep
// the smaller scale byte (the FP4 branch for IF4).
#include "fp4q_device.h"
#include "fp4q_launch.h"

namespace fp4q {

constexpr int kThreads = 256;
constexpr int kAmaxGroups = 1024; // partial maxima per call (<= kMaxPartials)

// ---------------------------------------------------------------------------
// global maximum
// ---------------------------------------------------------------------------

__device__ __forceinline__ void store_group_max(float m, float* partials)
{
    __shared__ float red[kThreads / 64];
    m = wave_max(m);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0)
        red[wave] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        float g = red[0];
#pragma unroll
        for (int w = 1; w < kThreads / 64; ++w)
            g = __builtin_fmaxf(g, red[w]);
        partials[blockIdx.x] = g;
    }
}

// un-rotated tensor: a flat, perfectly coalesced pass over 16-byte vectors
template <bool BF16>
__global__ __launch_bounds__(kThreads) void amax_flat(const uint4* __restrict__ x, int64_t nvec,
                                                      float* __restrict__ partials)
{
    float m = 0.0f;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nvec;
         i += (int64_t)gridDim.x * kThreads) {
        const uint4 w = x[i];
        if constexpr (BF16) {
            m = __builtin_fmaxf(m, __builtin_fabsf(bf16_lo(w.x)));
            m = __builtin_fmaxf(m, __builtin_fabsf(bf16_hi(w.x)));
            m = __builtin_fmaxf(m, __builtin_fabsf(bf16_lo(w.y)));
            m = __builtin_fmaxf(m, __builtin_fabsf(bf16_hi(w.y)));
            m = __builtin_fmaxf(m, __builtin_fabsf(bf16_lo(w.z)));
            m = __builtin_fmaxf(m, __builtin_fabsf(bf16_hi(w.z)));
            m = __builtin_fmaxf(m, __builtin_fabsf(bf16_lo(w.w)));
            m = __builtin_fmaxf(m, __builtin_fabsf(bf16_hi(w.w)));
        } else {
            m = __builtin_fmaxf(m, __builtin_fabsf(__uint_as_float(w.x)));
            m = __builtin_fmaxf(m, __builtin_fabsf(__uint_as_float(w.y)));
            m = __builtin_fmaxf(m, __builtin_fabsf(__uint_as_float(w.z)));
            m = __builtin_fmaxf(m, __builtin_fabsf(__uint_as_float(w.w)));
        }
    }
    store_group_max(m, partials);
}

// rotated tensor: one lane per block so the Hadamard stays in registers
template <int B, bool BF16>
__global__ __launch_bounds__(kThreads) void amax_rot(const void* __restrict__ x, int64_t nblocks,
                                                     float* __restrict__ partials)
{
    float m = 0.0f;
    for (int64_t blk = (int64_t)blockIdx.x * kThreads + threadIdx.x; blk < nblocks;
         blk += (int64_t)gridDim.x * kThreads) {
        float v[B];
        load_block<B, BF16, false>(x, blk, v);
        fwht<B>(v);
        m = __builtin_fmaxf(m, block_absmax<B>(v));
    }
    store_group_max(m, partials);
}

// G = max of the partials; S = G / 1536, floored at 2^-117 (so every
// D = s*S is a normal binary32 with a finite reciprocal), 1 when G == 0
__global__ __launch_bounds__(1024) void finalize_scale(const float* __restrict__ partials, int n,
                                                       float* __restrict__ S_out)
{
    __shared__ float red[1024 / 64];
    float m = 0.0f;
    for (int i = threadIdx.x; i < n; i += 1024)
        m = __builtin_fmaxf(m, partials[i]);
    m = wave_max(m);
    if ((threadIdx.x & 63) == 0)
        red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        float g = 0.0f;
        for (int w = 0; w < 1024 / 64; ++w)
            g = __builtin_fmaxf(g, red[w]);
        float s = g / 1536.0f;
        s = __builtin_fmaxf(s, 0x1p-117f);
        *S_out = (g == 0.0f) ? 1.0f : s;
    }
}

// ---------------------------------------------------------------------------
// encoders
// ---------------------------------------------------------------------------

// the 16 nibbles of an NVFP4 block encoded with step D (reciprocal r)
__device__ __forceinline__ uint2 encode16_fp4(const float* v, float r)
{
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t sgn = __float_as_uint(v[i]) >> 31;
        const float q = e2m1_q(__builtin_fabsf(v[i]) * r);
        const uint32_t nib = (sgn << 3) | e2m1_code(q);
        if (i < 8)
            lo |= nib << (4 * i);
        else
            hi |= nib << (4 * (i - 8));
    }
    return make_uint2(lo, hi);
}

__device__ __forceinline__ uint2 sign_only16(const float* v)
{
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t nib = (__float_as_uint(v[i]) >> 31) << 3;
        if (i < 8)
            lo |= nib << (4 * i);
        else
            hi |= nib << (4 * (i - 8));
    }
    return make_uint2(lo, hi);
}

// block error of the FP4 encoding with step D, reciprocal r, in binary64
template <bool WMSE>
__device__ __forceinline__ double fp4_error16(const float* v, const float* w, float D, float r)
{
    double E = 0.0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float a = __builtin_fabsf(v[i]);
        const float xh = e2m1_q(a * r) * D;
        const double d = (double)a - (double)xh;
        double t = d * d;
        if constexpr (WMSE)
            t = (double)w[i] * t;
        E = E + t;
    }
    return E;
}

template <bool WMSE>
__device__ __forceinline__ double int4_error16(const float* v, const float* w, float Di, float ri)
{
    double E = 0.0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float a = __builtin_fabsf(v[i]);
        const float q = __builtin_fminf(__builtin_rintf(a * ri), 7.0f);
        const float xh = q * Di;
        const double d = (double)a - (double)xh;
        double t = d * d;
        if constexpr (WMSE)
            t = (double)w[i] * t;
        E = E + t;
    }
    return E;
}

__device__ __forceinline__ uint2 encode16_int4(const float* v, float ri)
{
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float q = __builtin_fminf(__builtin_rintf(__builtin_fabsf(v[i]) * ri), 7.0f);
        int qi = (int)q;
        if (__float_as_uint(v[i]) >> 31)
            qi = -qi;
        const uint32_t nib = (uint32_t)qi & 0xFu;
        if (i < 8)
            lo |= nib << (4 * i);
        else
            hi |= nib << (4 * (i - 8));
    }
    return make_uint2(lo, hi);
}

__device__ __forceinline__ void load_weights16(const float* __restrict__ imp, int64_t col0, float* w)
{
    const float4* p = reinterpret_cast<const float4*>(imp + col0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float4 t = p[q];
        w[4 * q + 0] = t.x; w[4 * q + 1] = t.y; w[4 * q + 2] = t.z; w[4 * q + 3] = t.w;
    }
}

// ---------------------------------------------------------------------------
// NVFP4: AbsMax or ScaleSweep (MSE / WMSE)
// ---------------------------------------------------------------------------

template <bool BF16, bool ROT, bool SWEEP, bool WMSE>
__global__ __launch_bounds__(kThreads) void nvfp4_quant(
    const void* __restrict__ x, int64_t nblocks, int64_t blocks_per_row,
    const float* __restrict__ imp, const float* __restrict__ Sp, int lo, int hi,
    uint2* __restrict__ codes, uint8_t* __restrict__ scales)
{
    __shared__ float sD[128], sR[128];
    const float S = *Sp;
    if constexpr (SWEEP) {
        // per-candidate step D = fl32(s*S) and reciprocal fl32(1/D), shared
        for (int c = threadIdx.x; c < 128; c += kThreads) {
            const float D = e4m3_value((uint32_t)(c < 0x7F ? c : 0x7E)) * S;
            sD[c] = D;
            sR[c] = 1.0f / D;
        }
        __syncthreads();
    }
    const float S6 = 6.0f * S;
    for (int64_t blk = (int64_t)blockIdx.x * kThreads + threadIdx.x; blk < nblocks;
         blk += (int64_t)gridDim.x * kThreads) {
        float v[16];
        load_block<16, BF16>(x, blk, v);
        if constexpr (ROT)
            fwht<16>(v);
        const float a = block_absmax<16>(v);
        uint2 packed;
        uint32_t sbyte;
        if (a == 0.0f) {
            sbyte = 0;
            packed = sign_only16(v);
        } else {
            uint32_t sb = e4m3_round(a / S6);
            sb = sb < 1u ? 1u : sb;
            uint32_t cb = sb;
            if constexpr (SWEEP) {
                float w[16];
                if constexpr (WMSE)
                    load_weights16(imp, (blk % blocks_per_row) * 16, w);
                const int c0 = max(1, (int)sb + lo), c1 = min(0x7E, (int)sb + hi);
                double best = __builtin_huge_val();
                for (int c = c0; c <= c1; ++c) {
                    const double E = fp4_error16<WMSE>(v, w, sD[c], sR[c]);
                    if (E < best) {
                        best = E;
                        cb = (uint32_t)c;
                    }
                }
            }
            const float D = e4m3_value(cb) * S;
            const float r = 1.0f / D;
            sbyte = cb;
            packed = encode16_fp4(v, r);
        }
        codes[blk] = packed;
        scales[blk] = (uint8_t)sbyte;
    }
}

// ---------------------------------------------------------------------------
// IF4: per block FP4 vs INT4 (6/7 step), indicator in the scale's bit 7
// ---------------------------------------------------------------------------

template <bool BF16, bool ROT, bool WMSE>
__global__ __launch_bounds__(kThreads) void if4_quant(
    const void* __restrict__ x, int64_t nblocks, int64_t blocks_per_row,
    const float* __restrict__ imp, const float* __restrict__ Sp,
    uint2* __restrict__ codes, uint8_t* __restrict__ scales)
{
    const float S = *Sp;
    const float S6 = 6.0f * S;
    for (int64_t blk = (int64_t)blockIdx.x * kThreads + threadIdx.x; blk < nblocks;
         blk += (int64_t)gridDim.x * kThreads) {
        float v[16];
        load_block<16, BF16>(x, blk, v);
        if constexpr (ROT)
            fwht<16>(v);
        const float a = block_absmax<16>(v);
        uint2 packed;
        uint32_t sbyte;
        if (a == 0.0f) {
            sbyte = 0;
            packed = sign_only16(v);
        } else {
            uint32_t sb = e4m3_round(a / S6);
            sb = sb < 1u ? 1u : sb;
            float w[16];
            if constexpr (WMSE)
                load_weights16(imp, (blk % blocks_per_row) * 16, w);
            const float D = e4m3_value(sb) * S;
            const float r = 1.0f / D;
            const float Di = D * kInt4Step;
            const float ri = 1.0f / Di;
            const double ef = fp4_error16<WMSE>(v, w, D, r);
            const double ei = int4_error16<WMSE>(v, w, Di, ri);
            if (ei < ef) {
                sbyte = sb | 0x80u;
                packed = encode16_int4(v, ri);
            } else {
                sbyte = sb;
                packed = encode16_fp4(v, r);
            }
        }
        codes[blk] = packed;
        scales[blk] = (uint8_t)sbyte;
    }
}

// ---------------------------------------------------------------------------
// MXFP4: E8M0 scale 2^(floor(log2 max) - 2) per 32 elements
// ---------------------------------------------------------------------------

__device__ __forceinline__ int floor_log2_f32(float a)
{
    const uint32_t u = __float_as_uint(a);
    if (u >= 0x00800000u)
        return (int)(u >> 23) - 127;
    return -149 + (31 - __clz((int)u)); // subnormal, u != 0
}

template <bool BF16, bool ROT>
__global__ __launch_bounds__(kThreads) void mxfp4_quant(
    const void* __restrict__ x, int64_t nblocks, uint4* __restrict__ codes,
    uint8_t* __restrict__ scales)
{
    for (int64_t blk = (int64_t)blockIdx.x * kThreads + threadIdx.x; blk < nblocks;
         blk += (int64_t)gridDim.x * kThreads) {
        float v[32];
        load_block<32, BF16>(x, blk, v);
        if constexpr (ROT)
            fwht<32>(v);
        const float a = block_absmax<32>(v);
        int e = (a == 0.0f) ? -127 : floor_log2_f32(a) - 2;
        e = e < -127 ? -127 : (e > 127 ? 127 : e);
        const float r = __uint_as_float((uint32_t)(127 - e) << 23); // 2^-e, -e <= 127
        uint32_t wds[4] = {0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const uint32_t sgn = __float_as_uint(v[i]) >> 31;
            const float q = e2m1_q(__builtin_fabsf(v[i]) * r);
            wds[i >> 3] |= ((sgn << 3) | e2m1_code(q)) << (4 * (i & 7));
        }
        codes[blk] = make_uint4(wds[0], wds[1], wds[2], wds[3]);
        scales[blk] = (uint8_t)(e + 127);
    }
}

// ---------------------------------------------------------------------------
// dequantize and error
// ---------------------------------------------------------------------------

// decode one block's B values (before any un-rotation)
template <int FMT, int B>
__device__ __forceinline__ void decode_block(const uint32_t* wds, uint32_t sb, float S, float* o)
{
    if constexpr (FMT == kMXFP4) {
        const float D = (sb == 0xFFu) ? __builtin_nanf("")
                        : (sb == 0u ? __uint_as_float(0x00400000u) : __uint_as_float(sb << 23));
#pragma unroll
        for (int i = 0; i < B; ++i) {
            const uint32_t nib = (wds[i >> 3] >> (4 * (i & 7))) & 0xFu;
            const float val = e2m1_value(nib & 7u) * D;
            o[i] = (nib & 8u) ? -val : val;
        }
    } else {
        const uint32_t mag = sb & 0x7Fu;
        float s = (mag == 0x7Fu) ? __builtin_nanf("") : e4m3_value(mag);
        const bool int4 = (FMT == kIF4) && (sb & 0x80u);
        if (FMT == kNVFP4 && (sb & 0x80u))
            s = -s;
        const float D = s * S;
        if (int4) {
            const float Di = D * kInt4Step;
#pragma unroll
            for (int i = 0; i < B; ++i) {
                const uint32_t nib = (wds[i >> 3] >> (4 * (i & 7))) & 0xFu;
                const int q = (nib & 8u) ? (int)nib - 16 : (int)nib;
                o[i] = (float)q * Di;
            }
        } else {
#pragma unroll
            for (int i = 0; i < B; ++i) {
                const uint32_t nib = (wds[i >> 3] >> (4 * (i & 7))) & 0xFu;
                const float val = e2m1_value(nib & 7u) * D;
                o[i] = (nib & 8u) ? -val : val;
            }
        }
    }
}

template <int B>
__device__ __forceinline__ void load_codes(const uint8_t* __restrict__ codes, int64_t blk, uint32_t* wds)
{
    if constexpr (B == 16) {
        const uint2 c = reinterpret_cast<const uint2*>(codes)[blk];
        wds[0] = c.x;
        wds[1] = c.y;
    } else {
        const uint4 c = reinterpret_cast<const uint4*>(codes)[blk];
        wds[0] = c.x; wds[1] = c.y; wds[2] = c.z; wds[3] = c.w;
    }
}

template <int FMT, int B, bool ROT, bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void dequant(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const float* __restrict__ Sp, int64_t nblocks, void* __restrict__ y)
{
    const float S = (FMT == kMXFP4) ? 1.0f : *Sp;
    for (int64_t blk = (int64_t)blockIdx.x * kThreads + threadIdx.x; blk < nblocks;
         blk += (int64_t)gridDim.x * kThreads) {
        uint32_t wds[B / 8];
        load_codes<B>(codes, blk, wds);
        float o[B];
        decode_block<FMT, B>(wds, scales[blk], S, o);
        if constexpr (ROT)
            fwht<B>(o);
        if constexpr (OUT_BF16) {
            u32x4* p = reinterpret_cast<u32x4*>(y) + blk * (B / 8);
#pragma unroll
            for (int q = 0; q < B / 8; ++q) {
                u32x4 t;
                t.x = f32_to_bf16(o[8 * q + 0]) | (f32_to_bf16(o[8 * q + 1]) << 16);
                t.y = f32_to_bf16(o[8 * q + 2]) | (f32_to_bf16(o[8 * q + 3]) << 16);
                t.z = f32_to_bf16(o[8 * q + 4]) | (f32_to_bf16(o[8 * q + 5]) << 16);
                t.w = f32_to_bf16(o[8 * q + 6]) | (f32_to_bf16(o[8 * q + 7]) << 16);
                __builtin_nontemporal_store(t, p + q);
            }
        } else {
            f32x4* p = reinterpret_cast<f32x4*>(y) + blk * (B / 4);
#pragma unroll
            for (int q = 0; q < B / 4; ++q) {
                const f32x4 t = {o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]};
                __builtin_nontemporal_store(t, p + q);
            }
        }
    }
}

template <int FMT, int B, bool BF16, bool ROT, bool IMP>
__global__ __launch_bounds__(kThreads) void error_partial(
    const void* __restrict__ x, const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const float* __restrict__ Sp, const float* __restrict__ imp, int64_t nblocks,
    int64_t blocks_per_row, double2* __restrict__ partials)
{
    const float S = (FMT == kMXFP4) ? 1.0f : *Sp;
    double s = 0.0, ws = 0.0;
    for (int64_t blk = (int64_t)blockIdx.x * kThreads + threadIdx.x; blk < nblocks;
         blk += (int64_t)gridDim.x * kThreads) {
        float v[B], o[B];
        load_block<B, BF16>(x, blk, v);
        uint32_t wds[B / 8];
        load_codes<B>(codes, blk, wds);
        decode_block<FMT, B>(wds, scales[blk], S, o);
        if constexpr (ROT)
            fwht<B>(o);
        const float* w = IMP ? imp + (blk % blocks_per_row) * B : nullptr;
#pragma unroll
        for (int i = 0; i < B; ++i) {
            const double d = (double)v[i] - (double)o[i];
            const double t = d * d;
            s += t;
            if constexpr (IMP)
                ws += (double)w[i] * t;
        }
    }
    __shared__ double red[2][kThreads / 64];
    s = wave_sum(s);
    ws = wave_sum(ws);
    if ((threadIdx.x & 63) == 0) {
        red[0][threadIdx.x >> 6] = s;
        red[1][threadIdx.x >> 6] = ws;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        double a = 0.0, b = 0.0;
        for (int w = 0; w < kThreads / 64; ++w) {
            a += red[0][w];
            b += red[1][w];
        }
        partials[blockIdx.x] = make_double2(a, b);
    }
}

__global__ __launch_bounds__(64) void error_final(const double2* __restrict__ partials, int n,
                                                  double inv_n, int has_imp, double* __restrict__ out)
{
    double a = 0.0, b = 0.0;
    for (int i = threadIdx.x; i < n; i += 64) {
        a += partials[i].x;
        b += partials[i].y;
    }
    a = wave_sum(a);
    b = wave_sum(b);
    if (threadIdx.x == 0) {
        out[0] = a * inv_n;
        out[1] = has_imp ? b * inv_n : __builtin_nan("");
    }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------

static int grid_for(int64_t items, int cap)
{
    const int64_t g = (items + kThreads - 1) / kThreads;
    return (int)(g < 1 ? 1 : (g > cap ? cap : g));
}

constexpr int kQuantGroupCap = 16384;

template <bool BF16, bool ROT>
static void launch_nvfp4(const QuantArgs& a, int64_t nb, const float* Sp, int grid)
{
    const int64_t bpr = a.cols / 16;
    uint2* codes = reinterpret_cast<uint2*>(a.codes);
    if (a.rule == kAbsMax)
        hipLaunchKernelGGL((nvfp4_quant<BF16, ROT, false, false>), grid, kThreads, 0, a.stream,
                           a.x, nb, bpr, a.importance, Sp, 0, 0, codes, a.scales);
    else if (a.objective == kWMSE)
        hipLaunchKernelGGL((nvfp4_quant<BF16, ROT, true, true>), grid, kThreads, 0, a.stream,
                           a.x, nb, bpr, a.importance, Sp, a.lo, a.hi, codes, a.scales);
    else
        hipLaunchKernelGGL((nvfp4_quant<BF16, ROT, true, false>), grid, kThreads, 0, a.stream,
                           a.x, nb, bpr, a.importance, Sp, a.lo, a.hi, codes, a.scales);
}

template <bool BF16, bool ROT>
static void launch_if4(const QuantArgs& a, int64_t nb, const float* Sp, int grid)
{
    const int64_t bpr = a.cols / 16;
    uint2* codes = reinterpret_cast<uint2*>(a.codes);
    if (a.objective == kWMSE)
        hipLaunchKernelGGL((if4_quant<BF16, ROT, true>), grid, kThreads, 0, a.stream,
                           a.x, nb, bpr, a.importance, Sp, codes, a.scales);
    else
        hipLaunchKernelGGL((if4_quant<BF16, ROT, false>), grid, kThreads, 0, a.stream,
                           a.x, nb, bpr, a.importance, Sp, codes, a.scales);
}

template <bool BF16>
static void launch_amax(const QuantArgs& a, float* partials, int groups)
{
    const int64_t n = a.rows * a.cols;
    if (a.rotate == 0) {
        const int64_t nvec = n * (BF16 ? 2 : 4) / 16;
        hipLaunchKernelGGL((amax_flat<BF16>), groups, kThreads, 0, a.stream,
                           reinterpret_cast<const uint4*>(a.x), nvec, partials);
    } else {
        hipLaunchKernelGGL((amax_rot<16, BF16>), groups, kThreads, 0, a.stream, a.x, n / 16, partials);
    }
}

hipError_t launch_quantize(const QuantArgs& a)
{
    const int64_t n = a.rows * a.cols;
    const int B = (a.format == kMXFP4) ? 32 : 16;
    const int64_t nb = n / B;
    float* partials = reinterpret_cast<float*>(a.workspace);
    const float* Sp = a.global_scale;
    if (a.format != kMXFP4 && !a.global_scale_given) {
        int groups = 0;
        if (n > 0) {
            const int64_t items = (a.rotate == 0) ? n * (a.bf16 ? 2 : 4) / 16 : nb;
            groups = grid_for(items, kAmaxGroups);
            if (a.bf16)
                launch_amax<true>(a, partials, groups);
            else
                launch_amax<false>(a, partials, groups);
        }
        hipLaunchKernelGGL(finalize_scale, 1, 1024, 0, a.stream, partials, groups, a.global_scale);
    }
    if (nb > 0) {
        const int grid = grid_for(nb, kQuantGroupCap);
        const bool rot = a.rotate != 0;
        if (a.format == kNVFP4) {
            if (a.bf16)
                rot ? launch_nvfp4<true, true>(a, nb, Sp, grid) : launch_nvfp4<true, false>(a, nb, Sp, grid);
            else
                rot ? launch_nvfp4<false, true>(a, nb, Sp, grid) : launch_nvfp4<false, false>(a, nb, Sp, grid);
        } else if (a.format == kIF4) {
            if (a.bf16)
                rot ? launch_if4<true, true>(a, nb, Sp, grid) : launch_if4<true, false>(a, nb, Sp, grid);
            else
                rot ? launch_if4<false, true>(a, nb, Sp, grid) : launch_if4<false, false>(a, nb, Sp, grid);
        } else {
            uint4* codes = reinterpret_cast<uint4*>(a.codes);
            if (a.bf16) {
                if (rot)
                    hipLaunchKernelGGL((mxfp4_quant<true, true>), grid, kThreads, 0, a.stream, a.x, nb, codes, a.scales);
                else
                    hipLaunchKernelGGL((mxfp4_quant<true, false>), grid, kThreads, 0, a.stream, a.x, nb, codes, a.scales);
            } else {
                if (rot)
                    hipLaunchKernelGGL((mxfp4_quant<false, true>), grid, kThreads, 0, a.stream, a.x, nb, codes, a.scales);
                else
                    hipLaunchKernelGGL((mxfp4_quant<false, false>), grid, kThreads, 0, a.stream, a.x, nb, codes, a.scales);
            }
        }
    }
    return hipGetLastError();
}

template <int FMT, int B>
static void launch_dequant_fmt(const DequantArgs& a, int64_t nb, int grid)
{
    if (a.unrotate) {
        if (a.out_bf16)
            hipLaunchKernelGGL((dequant<FMT, B, true, true>), grid, kThreads, 0, a.stream, a.codes, a.scales, a.global_scale, nb, a.y);
        else
            hipLaunchKernelGGL((dequant<FMT, B, true, false>), grid, kThreads, 0, a.stream, a.codes, a.scales, a.global_scale, nb, a.y);
    } else {
        if (a.out_bf16)
            hipLaunchKernelGGL((dequant<FMT, B, false, true>), grid, kThreads, 0, a.stream, a.codes, a.scales, a.global_scale, nb, a.y);
        else
            hipLaunchKernelGGL((dequant<FMT, B, false, false>), grid, kThreads, 0, a.stream, a.codes, a.scales, a.global_scale, nb, a.y);
    }
}

hipError_t launch_dequantize(const DequantArgs& a)
{
    const int B = (a.format == kMXFP4) ? 32 : 16;
    const int64_t nb = a.rows * a.cols / B;
    if (nb == 0)
        return hipSuccess;
    const int grid = grid_for(nb, kQuantGroupCap);
    if (a.format == kNVFP4)
        launch_dequant_fmt<kNVFP4, 16>(a, nb, grid);
    else if (a.format == kIF4)
        launch_dequant_fmt<kIF4, 16>(a, nb, grid);
    else
        launch_dequant_fmt<kMXFP4, 32>(a, nb, grid);
    return hipGetLastError();
}

template <int FMT, int B, bool BF16>
static void launch_error_fmt(const ErrorArgs& a, int64_t nb, int grid, double2* partials)
{
    const int64_t bpr = a.cols / B;
    const bool imp = a.importance != nullptr;
    const bool rot = a.rotate != 0;
#define FP4Q_ERR(R, I)                                                                          \
    hipLaunchKernelGGL((error_partial<FMT, B, BF16, R, I>), grid, kThreads, 0, a.stream, a.x,  \
                       a.codes, a.scales, a.global_scale, a.importance, nb, bpr, partials)
    if (rot) {
        if (imp) FP4Q_ERR(true, true); else FP4Q_ERR(true, false);
    } else {
        if (imp) FP4Q_ERR(false, true); else FP4Q_ERR(false, false);
    }
#undef FP4Q_ERR
}

hipError_t launch_error(const ErrorArgs& a, double* out_dev)
{
    const int B = (a.format == kMXFP4) ? 32 : 16;
    const int64_t n = a.rows * a.cols;
    const int64_t nb = n / B;
    double2* partials = reinterpret_cast<double2*>(a.workspace);
    int grid = 0;
    if (nb > 0) {
        grid = grid_for(nb, kErrorGroups);
        if (a.format == kNVFP4)
            a.bf16 ? launch_error_fmt<kNVFP4, 16, true>(a, nb, grid, partials)
                   : launch_error_fmt<kNVFP4, 16, false>(a, nb, grid, partials);
        else if (a.format == kIF4)
            a.bf16 ? launch_error_fmt<kIF4, 16, true>(a, nb, grid, partials)
                   : launch_error_fmt<kIF4, 16, false>(a, nb, grid, partials);
        else
            a.bf16 ? launch_error_fmt<kMXFP4, 32, true>(a, nb, grid, partials)
                   : launch_error_fmt<kMXFP4, 32, false>(a, nb, grid, partials);
    }
    const double inv_n = n > 0 ? 1.0 / (double)n : 0.0;
    hipLaunchKernelGGL(error_final, 1, 64, 0, a.stream, partials, grid, inv_n,
                       a.importance != nullptr ? 1 : 0, out_dev);
    return hipGetLastError();
}

} // namespace fp4q
