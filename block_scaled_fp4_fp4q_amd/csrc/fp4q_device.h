// fp4q_device.h -- device-side number formats and block helpers for gfx950.
//
// Every helper here is a fixed sequence of IEEE binary32 operations (the
// library is built with -ffp-contract=off, correctly rounded division and
// denormals kept), so a block quantized here is bit-identical to the same
// sequence evaluated anywhere else.
//
// Formats: E2M1 (FP4 elements), E4M3FN (NVFP4/IF4 scales: bias 7, 0x7F NaN,
// 126 positive finite values -- ScaleSweep page, Method 2), E8M0 (MXFP4
// scales: a biased power of two -- "Bridging the Gap ... Microscaling FP4"
// page, Problem).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4q {

// native clang vectors (the nontemporal builtins take these, not HIP's structs)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---- bf16 ---------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// round-to-nearest-even fp32 -> bf16 bits (NaN stays a quiet NaN)
__device__ __forceinline__ uint32_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return (u >> 16) | 0x40u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// two binary32 values rounded to bf16 (nearest even) and packed, first value
// in the low half: one v_cvt_pk_bf16_f32 on gfx950
__device__ __forceinline__ uint32_t bf16_pair(float a, float b)
{
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// ---- E4M3FN --------------------------------------------------------------

// value of a non-negative E4M3 pattern 0x00..0x7E
__device__ __forceinline__ float e4m3_value(uint32_t b)
{
    const uint32_t e = b >> 3, m = b & 7u;
    return e == 0 ? (float)m * 0x1p-9f : __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// nearest E4M3 pattern to t >= 0 with ties to even, saturating at 448 (0x7E)
__device__ __forceinline__ uint32_t e4m3_round(float t)
{
    if (t >= 448.0f)
        return 0x7Eu;
    if (t < 0x1p-6f) // subnormal range: multiples of 2^-9, exact scaling then RNE
        return (uint32_t)__builtin_rintf(t * 512.0f);
    uint32_t u = __float_as_uint(t);
    u += 0x7FFFFu + ((u >> 20) & 1u); // round the 23-bit mantissa to 3 bits
    return (u >> 20) - (120u << 3);
}

// ---- E2M1 -----------------------------------------------------------------

// nearest E2M1 magnitude {0,.5,1,1.5,2,3,4,6} to y >= 0, ties to the even
// code, saturating at 6.  Adding 2^22 / 2^23 / 2^24 makes the binary32 ulp
// equal to the grid spacing of [0,2) / [2,4) / [4,inf), so the hardware's
// round-to-nearest-even performs the rounding.
__device__ __forceinline__ float e2m1_q(float y)
{
    const float M = y < 2.0f ? 0x1p22f : (y < 4.0f ? 0x1p23f : 0x1p24f);
    const float v = (y + M) - M;
    return __builtin_fminf(v, 6.0f);
}

// ---- gfx950 FP4 conversion instructions ------------------------------------
// v_cvt_scalef32_pk_fp4_f32 with a unit scale rounds two binary32 values to
// the nearest E2M1 value (ties to the even code), saturates at +-6 and keeps
// the sign (also of zero): exactly e2m1_q, applied to signed values.  It
// writes the two codes as nibbles (first value low) into byte SEL of `old`.
// v_cvt_scalef32_pk_f32_fp4 decodes byte SEL of a packed word.
template <int SEL>
__device__ __forceinline__ uint32_t fp4_pack2(uint32_t old, float a, float b)
{
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, SEL);
}

template <int SEL>
__device__ __forceinline__ void fp4_unpack2(uint32_t packed, float& a, float& b)
{
    const auto t = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, 1.0f, SEL);
    a = t[0];
    b = t[1];
}

// the same with a power-of-two scale P: codes of a/P and b/P, and P times the
// decoded values (the hardware applies only the exponent of P, exactly)
template <int SEL>
__device__ __forceinline__ uint32_t fp4_pack2_scaled(uint32_t old, float a, float b, float P)
{
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, P, SEL);
}

template <int SEL>
__device__ __forceinline__ void fp4_unpack2_scaled(uint32_t packed, float& a, float& b, float P)
{
    const auto t = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, P, SEL);
    a = t[0];
    b = t[1];
}

// A register of unspecified value, to start a packed code word whose four
// bytes the following conversions all overwrite.  The empty asm emits
// nothing; taking `tie` as an input keeps each use a statement of its own, so
// that the compiler neither merges two of them (a conversion would then copy
// the shared register first) nor has to materialize a constant.
__device__ __forceinline__ uint32_t fresh_word(float tie)
{
    uint32_t w;
    asm("" : "=v"(w) : "v"(tie));
    return w;
}

// the 16 sign|magnitude nibbles of E2M1(v[i] * r), element 2k in the low
// nibble of byte k
__device__ __forceinline__ uint2 fp4_encode16(const float* v, float r)
{
    // every byte of both words is written: start from any value
    uint32_t lo = __builtin_nondeterministic_value(0u), hi = __builtin_nondeterministic_value(0u);
    lo = fp4_pack2<0>(lo, v[0] * r, v[1] * r);
    lo = fp4_pack2<1>(lo, v[2] * r, v[3] * r);
    lo = fp4_pack2<2>(lo, v[4] * r, v[5] * r);
    lo = fp4_pack2<3>(lo, v[6] * r, v[7] * r);
    hi = fp4_pack2<0>(hi, v[8] * r, v[9] * r);
    hi = fp4_pack2<1>(hi, v[10] * r, v[11] * r);
    hi = fp4_pack2<2>(hi, v[12] * r, v[13] * r);
    hi = fp4_pack2<3>(hi, v[14] * r, v[15] * r);
    return make_uint2(lo, hi);
}

// INT4 step factor of IF4's 6/7 method: fl32(6/7)
constexpr float kInt4Step = 0.857142865657806396484375f; // 0x3F5B6DB7

// ---- block Hadamard ---------------------------------------------------------

// In-register Sylvester Hadamard of one n-block, butterfly stage widths
// 1, 2, ..., n/2, then one multiplication by fl32(1/sqrt(n)).
template <int N>
__device__ __forceinline__ void fwht(float* v)
{
#pragma unroll
    for (int h = 1; h < N; h *= 2)
#pragma unroll
        for (int i = 0; i < N; i += 2 * h)
#pragma unroll
            for (int j = i; j < i + h; ++j) {
                const float a = v[j], b = v[j + h];
                v[j] = a + b;
                v[j + h] = a - b;
            }
    const float c = (N == 16) ? 0.25f : __uint_as_float(0x3E3504F3u); // fl32(1/sqrt(32))
#pragma unroll
    for (int k = 0; k < N; ++k)
        v[k] = v[k] * c;
}

// ---- block loads -------------------------------------------------------------

// load the B elements of block `blk` of a contiguous tensor, widened to f32;
// NT marks the last read of the data (nontemporal: do not keep it in cache)
template <int B, bool BF16, bool NT = true>
__device__ __forceinline__ void load_block(const void* __restrict__ x, int64_t blk, float* v)
{
    if constexpr (BF16) {
        const u32x4* p = reinterpret_cast<const u32x4*>(x) + blk * (B / 8);
#pragma unroll
        for (int q = 0; q < B / 8; ++q) {
            const u32x4 w = NT ? __builtin_nontemporal_load(p + q) : p[q];
            v[8 * q + 0] = bf16_lo(w.x); v[8 * q + 1] = bf16_hi(w.x);
            v[8 * q + 2] = bf16_lo(w.y); v[8 * q + 3] = bf16_hi(w.y);
            v[8 * q + 4] = bf16_lo(w.z); v[8 * q + 5] = bf16_hi(w.z);
            v[8 * q + 6] = bf16_lo(w.w); v[8 * q + 7] = bf16_hi(w.w);
        }
    } else {
        const f32x4* p = reinterpret_cast<const f32x4*>(x) + blk * (B / 4);
#pragma unroll
        for (int q = 0; q < B / 4; ++q) {
            const f32x4 w = NT ? __builtin_nontemporal_load(p + q) : p[q];
            v[4 * q + 0] = w.x; v[4 * q + 1] = w.y; v[4 * q + 2] = w.z; v[4 * q + 3] = w.w;
        }
    }
}

// The input of a grid-stride loop that handles one block per lane and
// iteration.  With AHEAD (bf16 only) the block's raw words are loaded one
// iteration ahead (B/2 VGPRs), so that the load's latency overlaps the
// arithmetic on the previous block; otherwise each block is loaded in place.
// Loading ahead pays where the extra registers do not cost a wave per SIMD.
template <int B, bool BF16, bool AHEAD>
struct BlockStream {
    static constexpr bool kAhead = BF16 && AHEAD;
    u32x4 w[kAhead ? B / 8 : 1];

    // start the load of block `blk`, if it exists
    __device__ __forceinline__ void prefetch(const void* __restrict__ x, int64_t blk, int64_t nblocks)
    {
        if constexpr (kAhead) {
            if (blk < nblocks) {
                const u32x4* p = reinterpret_cast<const u32x4*>(x) + blk * (B / 8);
#pragma unroll
                for (int q = 0; q < B / 8; ++q)
                    w[q] = __builtin_nontemporal_load(p + q);
            }
        }
    }

    // the B elements of block `blk`, widened to f32 (loaded ahead: the block
    // the last prefetch loaded)
    __device__ __forceinline__ void take(const void* __restrict__ x, int64_t blk, float* v) const
    {
        if constexpr (kAhead) {
#pragma unroll
            for (int q = 0; q < B / 8; ++q) {
                v[8 * q + 0] = bf16_lo(w[q].x); v[8 * q + 1] = bf16_hi(w[q].x);
                v[8 * q + 2] = bf16_lo(w[q].y); v[8 * q + 3] = bf16_hi(w[q].y);
                v[8 * q + 4] = bf16_lo(w[q].z); v[8 * q + 5] = bf16_hi(w[q].z);
                v[8 * q + 6] = bf16_lo(w[q].w); v[8 * q + 7] = bf16_hi(w[q].w);
            }
        } else {
            load_block<B, BF16>(x, blk, v);
        }
    }
};

template <int B>
__device__ __forceinline__ float block_absmax(const float* v)
{
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < B; ++i)
        a = __builtin_fmaxf(a, __builtin_fabsf(v[i]));
    return a;
}

// ---- quad exchange (lanes 4k..4k+3) -------------------------------------------

// the same register of lane (lane ^ X) within this lane's quad, X = 1 or 2
// (DPP quad_perm [1,0,3,2] or [2,3,0,1]; every lane of the quad must be active)
template <int X>
__device__ __forceinline__ float quad_xor(float v)
{
    static_assert(X == 1 || X == 2, "quad exchange partner");
    constexpr int ctrl = X == 1 ? 0xB1 : 0x4E;
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), ctrl, 0xF, 0xF, true));
}

// ---- wave reductions (64 lanes) -------------------------------------------------

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        v = __builtin_fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

__device__ __forceinline__ double wave_sum(double v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        v += __shfl_xor(v, off, 64);
    return v;
}

} // namespace fp4q
