// fp4q_kernels.hip -- HIP kernels for block-scaled 4-bit quantization on
// gfx950 (MI355X), and the host launchers the C ABI calls.
//
// Data flow of one quantize call (NVFP4 / IF4 with a computed global scale):
//   amax_*      one read of x (rotated on the fly when asked) -> one partial
//               maximum per workgroup in the workspace;
//   *_quant,    every workgroup reduces the partials to G, S = max(G/1536,
//   *_sweep     2^-117) (1 for G == 0; ScaleSweep page, Method 2: S =
//               max|x|/(256*6)), and workgroup 0 publishes S; then per block:
//               load + widen, optional Hadamard, block max, base scale,
//               candidate search, encode, packed store.  Most kernels give a
//               block to one lane; the streaming bf16 MXFP4 ones give it to
//               four (lanes per block, below).
// MXFP4 and a caller-supplied S skip the first kernel.
//
// Block decisions equal the method's binary64 argmin (ties keep the smaller
// scale byte, the FP4 branch for IF4): candidates are compared by binary32
// estimates over the method's own codes, certified by a rigorous error bound,
// and blocks the bound leaves undecided take the exact binary64 evaluation.
#include "fp4q_device.h"
#include "fp4q_launch.h"

#include <mutex>

namespace fp4q {

constexpr int kThreads = 256;
constexpr int kAmaxGroups = 1024; // partial maxima per call (4 KiB of the 32 KiB workspace)

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

// un-rotated tensor: a flat, perfectly coalesced pass over 16-byte vectors,
// four loads in flight per lane
template <bool BF16>
__device__ __forceinline__ float vec_absmax(const uint4 w)
{
    if constexpr (BF16) {
        const float a = __builtin_fmaxf(__builtin_fabsf(bf16_lo(w.x)), __builtin_fabsf(bf16_hi(w.x)));
        const float b = __builtin_fmaxf(__builtin_fabsf(bf16_lo(w.y)), __builtin_fabsf(bf16_hi(w.y)));
        const float c = __builtin_fmaxf(__builtin_fabsf(bf16_lo(w.z)), __builtin_fabsf(bf16_hi(w.z)));
        const float d = __builtin_fmaxf(__builtin_fabsf(bf16_lo(w.w)), __builtin_fabsf(bf16_hi(w.w)));
        return __builtin_fmaxf(__builtin_fmaxf(a, b), __builtin_fmaxf(c, d));
    } else {
        const float a = __builtin_fmaxf(__builtin_fabsf(__uint_as_float(w.x)), __builtin_fabsf(__uint_as_float(w.y)));
        const float b = __builtin_fmaxf(__builtin_fabsf(__uint_as_float(w.z)), __builtin_fabsf(__uint_as_float(w.w)));
        return __builtin_fmaxf(a, b);
    }
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void amax_flat(const uint4* __restrict__ x, int64_t nvec,
                                                      float* __restrict__ partials)
{
    float m = 0.0f;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    for (; i + 3 * stride < nvec; i += 4 * stride) {
        const uint4 w0 = x[i], w1 = x[i + stride], w2 = x[i + 2 * stride], w3 = x[i + 3 * stride];
        m = __builtin_fmaxf(m, __builtin_fmaxf(__builtin_fmaxf(vec_absmax<BF16>(w0), vec_absmax<BF16>(w1)),
                                               __builtin_fmaxf(vec_absmax<BF16>(w2), vec_absmax<BF16>(w3))));
    }
    for (; i < nvec; i += stride)
        m = __builtin_fmaxf(m, vec_absmax<BF16>(x[i]));
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
// D = s*S is a normal binary32 with a finite reciprocal), 1 when G == 0.
// Launched for an empty tensor only (n == 0 partials: S = 1), where no
// quantize kernel runs to publish S.
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

// The global scale seen by a quantize kernel: with npart > 0 every workgroup
// reduces the partial maxima itself (a few KiB from L2, instead of a separate
// one-workgroup launch) and workgroup 0 publishes S; with npart == 0 it is
// read from *Sp (the caller supplied it).
__device__ __forceinline__ float global_scale(const float* __restrict__ partials, int npart,
                                              float* __restrict__ Sp)
{
    if (npart == 0)
        return *Sp;
    __shared__ float red[kThreads / 64];
    float m = 0.0f;
    for (int i = threadIdx.x; i < npart; i += kThreads)
        m = __builtin_fmaxf(m, partials[i]);
    m = wave_max(m);
    if ((threadIdx.x & 63) == 0)
        red[threadIdx.x >> 6] = m;
    __syncthreads();
    float g = red[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w)
        g = __builtin_fmaxf(g, red[w]);
    float s = g / 1536.0f;
    s = __builtin_fmaxf(s, 0x1p-117f);
    s = (g == 0.0f) ? 1.0f : s;
    if (blockIdx.x == 0 && threadIdx.x == 0)
        *Sp = s;
    return s;
}

// ---------------------------------------------------------------------------
// encoders
// ---------------------------------------------------------------------------

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
    // RNE is odd-symmetric, so clamping rint(v ri) to [-7, 7] gives
    // sign(v) min(RNE(|v| ri), 7) (a signed zero gives 0).  q + 8, in [1, 15],
    // goes to byte k of ev (element 8h + 2k) or od (element 8h + 2k + 1) by a
    // byte conversion; byte k of ev | od << 4 then holds elements 2k and
    // 2k + 1, and (q + 8) XOR 8 is q's two's complement nibble
    uint32_t out[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        uint32_t ev = __builtin_nondeterministic_value(0u), od = __builtin_nondeterministic_value(0u);
#pragma unroll
        for (int j = 0; j < 8; ++j) { // every byte of ev and od is written
            const float q = __builtin_amdgcn_fmed3f(__builtin_rintf(v[8 * h + j] * ri), -7.0f, 7.0f);
            if (j & 1)
                od = __builtin_amdgcn_cvt_pk_u8_f32(q + 8.0f, j / 2, od);
            else
                ev = __builtin_amdgcn_cvt_pk_u8_f32(q + 8.0f, j / 2, ev);
        }
        out[h] = (ev | (od << 4)) ^ 0x88888888u;
    }
    return make_uint2(out[0], out[1]);
}

// fp4_error16 and int4_error16 (MSE) of one block together, element by
// element from a per-lane LDS copy of the block (loop not unrolled): the same
// terms and order of summation with a few live registers, for the rare blocks
// whose estimates do not decide -- so that this path does not set the
// register budget, and with it the occupancy, of the common path
__device__ __forceinline__ void if4_exact_errors_lds(const float* slot, float D, float r, float Di,
                                                     float ri, double& ef, double& ei)
{
    ef = 0.0;
    ei = 0.0;
#pragma unroll 1
    for (int i = 0; i < 16; ++i) {
        const float a = __builtin_fabsf(slot[i]);
        const float xf = e2m1_q(a * r) * D;
        const double df = (double)a - (double)xf;
        const float xi = __builtin_fminf(__builtin_rintf(a * ri), 7.0f) * Di;
        const double di = (double)a - (double)xi;
        ef = ef + df * df;
        ei = ei + di * di;
    }
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

// ---- importance square roots -------------------------------------------------

constexpr int kRootCols = 4096; // importance columns whose square roots fit in LDS

// sqrt(w) of every column and the weight sum of every 16 columns, into LDS,
// when there are at most kRootCols columns; returns whether it did (the
// caller synchronizes the workgroup before use)
__device__ __forceinline__ bool roots_prologue(const float* __restrict__ imp, int64_t cols,
                                               float* root, float* wsum)
{
    if (cols > kRootCols)
        return false;
    for (int j = threadIdx.x; j < (int)cols; j += kThreads)
        root[j] = __builtin_sqrtf(imp[j]);
    for (int j = threadIdx.x; j < (int)(cols / 16); j += kThreads) {
        float W = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            W += imp[16 * j + i];
        wsum[j] = W;
    }
    return true;
}

// b = sqrt(w) of the N columns from col0 (a multiple of 16) and their weight
// sum W (rounded: the bounds carry slack for it)
template <int N>
__device__ __forceinline__ void block_roots(const float* __restrict__ imp, const float* root,
                                            const float* wsum, bool in_lds, int64_t col0, float* b,
                                            float& W)
{
    if (in_lds) {
        const float4* rp = reinterpret_cast<const float4*>(root + col0);
#pragma unroll
        for (int q = 0; q < N / 4; ++q) {
            const float4 t = rp[q];
            b[4 * q + 0] = t.x; b[4 * q + 1] = t.y; b[4 * q + 2] = t.z; b[4 * q + 3] = t.w;
        }
        W = wsum[col0 / 16];
        if constexpr (N == 32)
            W += wsum[col0 / 16 + 1];
    } else {
#pragma unroll
        for (int q = 0; q < N / 16; ++q)
            load_weights16(imp, col0 + 16 * q, b + 16 * q);
        W = 0.0f;
#pragma unroll
        for (int i = 0; i < N; ++i) {
            W += b[i];
            b[i] = __builtin_sqrtf(b[i]);
        }
    }
}

// ---- certified binary32 estimates ------------------------------------------
//
// A candidate's block error is estimated in binary32 in units of a fixed step
// (S^2 for E4M3 scales, the lowest step^2 for E8M0 windows): the conversion
// gives the method's own codes, and each term is (b y - b q)^2 with
// b = sqrt(w) (or (y - q)^2).  The binary64 error then lies within
// est_bound(estimate) of the estimate, where A bounds |x| and 6 D (7 D_int)
// over the candidates and W the weight sum, all in the same units, and rel
// the relative part (derivation at the ScaleSweep kernel).

__device__ __forceinline__ float est_bound(float E, float A, float W, float rel)
{
    constexpr float u = 0x1p-24f;
    return 16.0f * u * A * __builtin_amdgcn_sqrtf(W * E) * 1.0001f + rel * E + 64.0f * u * u * A * A * W;
}

// INT4 estimate of IF4's 6/7 method in units of the INT4 step, with q the
// method's integer min(RNE(fl(|x| ri)), 7), also packing the method's INT4
// nibbles.  z = fl(v ri) and t = fl(z + 1.5 2^23) = RNE(z) + 1.5 2^23 (the
// binary32 ulp there is 1; rounding to nearest even is odd-symmetric, so
// RNE(z) is sign(v) RNE(|v| ri)); CLAMP saturates t at +-7, which the caller
// leaves out where |v| ri stays below 7.5.  Then q = t - 1.5 2^23, the term
// (z - q)^2, and q + 8 = t - (1.5 2^23 - 8) in [1, 15] packed as bytes.
template <bool WMSE, bool CLAMP>
__device__ __forceinline__ float int4_est16_codes(const float* v, const float* b, float ri, uint2& words)
{
    constexpr float M = 12582912.0f;
    float F = 0.0f;
    uint32_t out[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        // q + 8 as byte k of ev (element 8h + 2k) or od (element 8h + 2k + 1);
        // every byte is written
        uint32_t ev = 0u, od = 0u;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int i = 8 * h + j;
            const float z = v[i] * ri;
            float t = z + M;
            if constexpr (CLAMP)
                t = __builtin_amdgcn_fmed3f(t, M - 7.0f, M + 7.0f);
            const float q = t - M;
            float d;
            if constexpr (WMSE)
                d = __builtin_fmaf(-b[i], q, b[i] * z);
            else
                d = z - q;
            F = __builtin_fmaf(d, d, F);
            const float q8 = t - (M - 8.0f);
            if (j & 1)
                od = __builtin_amdgcn_cvt_pk_u8_f32(q8, j / 2, od);
            else
                ev = __builtin_amdgcn_cvt_pk_u8_f32(q8, j / 2, ev);
        }
        // byte k of ev | od << 4 holds q + 8 of elements 2k (low nibble) and
        // 2k+1; (q + 8) XOR 8 is q mod 16, the two's complement nibble
        out[h] = (ev | (od << 4)) ^ 0x88888888u;
    }
    words = make_uint2(out[0], out[1]);
    return F;
}

// the 32 sign|magnitude nibbles of E2M1(v[i] * r) (hardware conversion)
__device__ __forceinline__ uint4 fp4_encode32(const float* v, float r)
{
    const uint2 lo = fp4_encode16(v, r), hi = fp4_encode16(v + 16, r);
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
}

// the 32 sign|magnitude nibbles of E2M1(y[i] / P) for a power of two P, which
// the conversion applies exactly
__device__ __forceinline__ uint4 fp4_encode32_scaled(const float* y, float P)
{
    uint32_t w[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        uint32_t c = __builtin_nondeterministic_value(0u); // every byte is written
        c = fp4_pack2_scaled<0>(c, y[8 * g + 0], y[8 * g + 1], P);
        c = fp4_pack2_scaled<1>(c, y[8 * g + 2], y[8 * g + 3], P);
        c = fp4_pack2_scaled<2>(c, y[8 * g + 4], y[8 * g + 5], P);
        c = fp4_pack2_scaled<3>(c, y[8 * g + 6], y[8 * g + 7], P);
        w[g] = c;
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// ---------------------------------------------------------------------------
// NVFP4 AbsMax
// ---------------------------------------------------------------------------

template <bool BF16, bool ROT>
__global__ __launch_bounds__(kThreads) void nvfp4_absmax(
    const void* __restrict__ x, int64_t nblocks, const float* __restrict__ partials, int npart,
    float* __restrict__ Sp, uint2* __restrict__ codes, uint8_t* __restrict__ scales)
{
    const float S = global_scale(partials, npart, Sp);
    const float S6 = 6.0f * S;
    for (int64_t blk = (int64_t)blockIdx.x * kThreads + threadIdx.x; blk < nblocks;
         blk += (int64_t)gridDim.x * kThreads) {
        float v[16];
        load_block<16, BF16>(x, blk, v);
        if constexpr (ROT)
            fwht<16>(v);
        const float a = block_absmax<16>(v);
        uint32_t sb = 0;
        float r = 1.0f; // an all-zero block keeps only its signs
        if (a != 0.0f) {
            sb = e4m3_round(a / S6);
            sb = sb < 1u ? 1u : sb;
            r = 1.0f / (e4m3_value(sb) * S);
        }
        codes[blk] = fp4_encode16(v, r);
        scales[blk] = (uint8_t)sb;
    }
}

// ---------------------------------------------------------------------------
// NVFP4 ScaleSweep (MSE / WMSE)
//
// Fast path, per block: every candidate's error is estimated in binary32 (y =
// |x| r with the method's own r = fl32(1/D), codes from the hardware E2M1
// conversion, which rounds exactly like the method, so each code is the
// method's code; only the error arithmetic is shortened).  The sum is formed
// in units of the candidate's step D and carried in units of S^2 (times the
// pattern's exact s*s), which stays normal for any global scale.  A rigorous
// bound T on |binary64 error / S^2 - estimate| then certifies the pick:
// when the runner-up minus its bound exceeds the best plus its bound, the
// binary64 argmin (ties to the smaller byte) is the estimated one.  Blocks
// that are not certified -- exact ties, near ties, all-on-grid blocks -- go to
// a per-wave queue in LDS that the wave drains with the exact binary64
// evaluation, so the result equals the binary64 sweep for every block.
// ---------------------------------------------------------------------------

// binary32 estimates of sum_i w_i (y_i - E2M1(y_i))^2 for y_i = v_i * r and,
// when PAIR, also for y_i / 2 (the pattern eight steps up, whose step is
// exactly 2D) in units of the first step: the hardware conversion applies the
// power-of-two scale 2 exactly, so one multiply serves both candidates.
// With weights, b holds sqrt(w) and each term is formed as (b y - b q)^2, so
// that the product b y serves both candidates of a pair as well.
// Every code word starts from a fresh register of unspecified value (all four
// bytes are written): a word handed on from the previous candidate would tie
// each candidate's conversions to the end of the previous one's decodes.
// With `words`, the first candidate's two code words (its 16 nibbles, the
// method's codes) are stored there.
template <bool WMSE, bool PAIR>
__device__ __forceinline__ void fp4_err32(const float* v, const float* b, float r, float& F1, float& F2,
                                          uint32_t* words = nullptr)
{
    F1 = 0.0f;
    F2 = 0.0f;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
        float y[8], q[8], h[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            y[j] = v[8 * g + j] * r;
        uint32_t c = fresh_word(y[0]), c2 = fresh_word(y[1]);
        // the half block's conversions are issued as one group, between
        // scheduling barriers: interleaving FP4 conversions with binary32
        // arithmetic costs more issue cycles than grouping them (measured:
        // the sweep 3.5% faster on a bf16 KV cache, 4.6% on a weighted
        // 14336x4096 weight)
        __builtin_amdgcn_sched_barrier(0);
        c = fp4_pack2<0>(c, y[0], y[1]);
        c = fp4_pack2<1>(c, y[2], y[3]);
        c = fp4_pack2<2>(c, y[4], y[5]);
        c = fp4_pack2<3>(c, y[6], y[7]);
        if constexpr (PAIR) {
            c2 = fp4_pack2_scaled<0>(c2, y[0], y[1], 2.0f);
            c2 = fp4_pack2_scaled<1>(c2, y[2], y[3], 2.0f);
            c2 = fp4_pack2_scaled<2>(c2, y[4], y[5], 2.0f);
            c2 = fp4_pack2_scaled<3>(c2, y[6], y[7], 2.0f);
        }
        fp4_unpack2<0>(c, q[0], q[1]);
        fp4_unpack2<1>(c, q[2], q[3]);
        fp4_unpack2<2>(c, q[4], q[5]);
        fp4_unpack2<3>(c, q[6], q[7]);
        if constexpr (PAIR) {
            fp4_unpack2_scaled<0>(c2, h[0], h[1], 2.0f);
            fp4_unpack2_scaled<1>(c2, h[2], h[3], 2.0f);
            fp4_unpack2_scaled<2>(c2, h[4], h[5], 2.0f);
            fp4_unpack2_scaled<3>(c2, h[6], h[7], 2.0f);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (words)
            words[g] = c;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if constexpr (WMSE) {
                const float bj = b[8 * g + j];
                const float by = bj * y[j];
                const float d = __builtin_fmaf(-bj, q[j], by);
                F1 = __builtin_fmaf(d, d, F1);
                if constexpr (PAIR) {
                    const float e = __builtin_fmaf(-bj, h[j], by);
                    F2 = __builtin_fmaf(e, e, F2);
                }
            } else {
                const float d = y[j] - q[j];
                F1 = __builtin_fmaf(d, d, F1);
                if constexpr (PAIR) {
                    const float e = y[j] - h[j];
                    F2 = __builtin_fmaf(e, e, F2);
                }
            }
        }
    }
}

// clamp a window pattern into [0x01, 0x7E]: a pattern past an end stands for
// the end pattern itself
__device__ __forceinline__ int clamp_pattern(int c) { return c < 1 ? 1 : (c > 0x7E ? 0x7E : c); }

// keep the least and the second least estimate; ties keep the earlier one
__device__ __forceinline__ void keep_best(float E, int c, float& e1, float& e2, int& cb)
{
    const bool better = E < e1;
    e2 = better ? e1 : __builtin_fminf(e2, E);
    cb = better ? c : cb;
    e1 = better ? E : e1;
}

// keep the two least of non-negative estimates whose low four mantissa bits
// carry the window offset: as unsigned integers such patterns order like the
// values (+inf and NaN from overflow order last), and the offset moves each
// estimate by at most 15 ulp (30u relative)
__device__ __forceinline__ void keep_best_packed(float E, uint32_t k, uint32_t& p1, uint32_t& p2)
{
    const uint32_t p = (__float_as_uint(E) & ~0xFu) | k;
    const uint32_t hi = p1 > p ? p1 : p; // p1 <= p2 throughout
    p2 = p2 < hi ? p2 : hi;
    p1 = p1 < p ? p1 : p;
}

// one pattern's constants: the pair every candidate reads (r, s*s) first,
// so that it is one aligned 8-byte LDS load with an immediate offset
struct alignas(16) SweepPattern {
    float r;    // fl32(1/D)
    float s2;   // s*s, exact
    float D;    // fl32(s S)
    float pair; // 1 when the pattern eight steps up has exactly twice this step
};

// the whole window [LO, HI] known at compile time, every pattern sb+k normal
// and finite, and every pair (k, k+8) an exact doubling: fully unrolled, no
// clamps or masks.  Returns the two least packed estimates (see above); only
// a strict gap beyond the error bounds is certified, so the order among
// near-equal estimates never decides a result.
template <bool WMSE, int LO, int HI>
__device__ __forceinline__ void sweep_fixed(const float* v, const float* b, const SweepPattern* tab, int sb,
                                            uint32_t& p1, uint32_t& p2)
{
    static_assert(HI - LO < 16, "the window offset must fit in four bits");
#pragma unroll
    for (int k = LO; k <= HI; ++k) {
        if (((k - LO) & 15) >= 8)
            continue; // evaluated with its partner k-8
        const SweepPattern t = tab[sb + k];
        float F1, F2;
        if (k + 8 <= HI) {
            fp4_err32<WMSE, true>(v, b, t.r, F1, F2);
            keep_best_packed(F1 * t.s2, (uint32_t)(k - LO), p1, p2);
            keep_best_packed(F2 * t.s2, (uint32_t)(k + 8 - LO), p1, p2);
        } else {
            fp4_err32<WMSE, false>(v, b, t.r, F1, F2);
            keep_best_packed(F1 * t.s2, (uint32_t)(k - LO), p1, p2);
        }
    }
}

template <bool BF16, bool ROT, bool WMSE, int WIN>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void nvfp4_sweep(
    const void* __restrict__ x, int64_t nblocks, int64_t blocks_per_row,
    const float* __restrict__ imp, const float* __restrict__ partials, int npart,
    float* __restrict__ Sp, int lo, int hi, uint2* __restrict__ codes, uint8_t* __restrict__ scales)
{
    // per pattern: r = fl32(1/D), s*s (exact), D = fl32(s S), and 1 when the
    // pattern eight steps up has exactly twice this step (so one product
    // serves both), else 0.  Estimates are kept in units of S^2: s*s is
    // normal for every pattern, while D*D would underflow for small S.
    __shared__ SweepPattern tab[128];
    // uncertified blocks, one queue per wave: a wave appends at most 64 per
    // iteration and drains its queue once it holds more than 64
    __shared__ int64_t queue[kThreads / 64][128];
    __shared__ float stage[kThreads / 16][WMSE ? 2 : 1][16]; // a queued block and its weights per group
    // sqrt(importance) per column and the importance sum per block column
    __shared__ __attribute__((aligned(16))) float root[WMSE ? kRootCols : 1]; // read as float4
    __shared__ float wsum[WMSE ? kRootCols / 16 : 1];
    const float S = global_scale(partials, npart, Sp);
    for (int c = threadIdx.x; c < 128; c += kThreads) {
        const float sc = e4m3_value((uint32_t)(c < 0x7E ? c : 0x7E));
        const float D = sc * S;
        const float D8 = e4m3_value((uint32_t)(c + 8 < 0x7E ? c + 8 : 0x7E)) * S;
        const bool twice = c >= 8 && c + 8 <= 0x7E && D8 == 2.0f * D && (1.0f / D8) == 0.5f * (1.0f / D);
        tab[c] = SweepPattern{1.0f / D, sc * sc, D, twice ? 1.0f : 0.0f};
    }
    bool roots_in_lds = false;
    if constexpr (WMSE)
        roots_in_lds = roots_prologue(imp, blocks_per_row * 16, root, wsum);
    __syncthreads();
    // every pair (c, c+8) with c in [8, 0x76] an exact doubling (true unless S
    // pushes the steps to the ends of the binary32 range)
    const bool pairs_exact = __syncthreads_and(threadIdx.x < 8 || threadIdx.x > 0x76 || tab[threadIdx.x].pair != 0.0f);
    constexpr int FLO = WIN == 1 ? -3 : -8, FHI = 7;
    const float S6 = 6.0f * S;
    const float invS = 1.0f / S;
    constexpr float u = 0x1p-24f; // unit roundoff of binary32
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    // importance column of this lane's block, advanced incrementally
    int64_t col = 0, col_step = 0;
    if constexpr (WMSE) {
        col = ((int64_t)blockIdx.x * kThreads + threadIdx.x) % blocks_per_row;
        col_step = stride % blocks_per_row;
    }

    // Exact binary64 sweep of a wave's queued blocks, candidate-parallel:
    // sixteen lanes share a block, each evaluates every sixteenth offset of
    // the window, and the group keeps the least (error, pattern) pair -- the
    // same choice as a scan in ascending order that keeps the first least
    // error.  The block (and its weights) pass through LDS and each error sum
    // runs element by element in a loop that is not unrolled, with the terms
    // and order of fp4_error16: few live registers, so this rare path does
    // not set the register budget of the common one.  A wave's queue and
    // drain involve that wave alone: the grid-stride loop has no workgroup
    // barrier.
    const int wv = threadIdx.x >> 6;
    auto wave_sync = [] {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };
    auto drain = [&](uint32_t n) {
        const int grp = threadIdx.x >> 4, sub = threadIdx.x & 15;
        for (uint32_t j0 = 0; j0 < n; j0 += 4) {
            const uint32_t j = j0 + (uint32_t)(grp & 3);
            const bool active = j < n;
            const int64_t blk = queue[wv][active ? j : 0];
            uint32_t sb;
            {
                float v[16];
                load_block<16, BF16, false>(x, blk, v);
                if constexpr (ROT)
                    fwht<16>(v);
                const float a = block_absmax<16>(v);
                sb = e4m3_round(a / S6);
                sb = sb < 1u ? 1u : sb;
                if (sub == 0) {
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        stage[grp][0][i] = v[i];
                    if constexpr (WMSE) {
                        const int64_t col0 = (blk % blocks_per_row) * 16;
#pragma unroll
                        for (int i = 0; i < 16; ++i)
                            stage[grp][WMSE ? 1 : 0][i] = imp[col0 + i];
                    }
                }
            }
            wave_sync();
            const float* xs = stage[grp][0];
            const float* ws = stage[grp][WMSE ? 1 : 0]; // read only with weights
            double best = __builtin_huge_val();
            int cb = 0x7F;
            for (int k = lo + sub; k <= hi; k += 16) {
                const int c = clamp_pattern((int)sb + k);
                const SweepPattern t = tab[c];
                double E = 0.0;
#pragma unroll 1
                for (int i = 0; i < 16; ++i) {
                    const float a = __builtin_fabsf(xs[i]);
                    const float xh = e2m1_q(a * t.r) * t.D;
                    const double d = (double)a - (double)xh;
                    double tt = d * d;
                    if constexpr (WMSE)
                        tt = (double)ws[i] * tt;
                    E = E + tt;
                }
                if (E < best || (E == best && c < cb)) {
                    best = E;
                    cb = c;
                }
            }
#pragma unroll
            for (int off = 8; off > 0; off >>= 1) {
                const double E2 = __shfl_xor(best, off, 64);
                const int c2 = __shfl_xor(cb, off, 64);
                if (E2 < best || (E2 == best && c2 < cb)) {
                    best = E2;
                    cb = c2;
                }
            }
            if (active && sub == 0) {
                float v[16];
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    v[i] = xs[i];
                codes[blk] = fp4_encode16(v, tab[cb].r);
                scales[blk] = (uint8_t)cb;
            }
            wave_sync(); // the stage is rewritten next round
        }
    };
    uint32_t wq = 0; // entries in this wave's queue (the same in every lane)

    // every lane of a wave runs the same number of iterations, so the queue
    // count and the drain stay wave-uniform
    // with weights, bf16 input of this lane's next block is loaded one
    // iteration ahead so that its latency overlaps the current block's
    // arithmetic; without them those registers would cost the kernel its
    // sixth wave per SIMD (79 against 90 VGPRs), and six waves without the
    // early load measured 0.3-1.2% faster.  Binary32 input loads in place.
    constexpr bool ahead = BF16 && WMSE;
    u32x4 pre[2];
    if constexpr (ahead) {
        const int64_t b0 = (int64_t)blockIdx.x * kThreads + threadIdx.x;
        if (b0 < nblocks) {
            const u32x4* p = reinterpret_cast<const u32x4*>(x) + b0 * 2;
            pre[0] = __builtin_nontemporal_load(p);
            pre[1] = __builtin_nontemporal_load(p + 1);
        }
    }
    for (int64_t base = (int64_t)blockIdx.x * kThreads; base < nblocks; base += stride) {
        const int64_t blk = base + threadIdx.x;
        bool queued = false;
        if (blk < nblocks) {
            float v[16];
            if constexpr (ahead) {
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const u32x4 w = pre[q];
                    v[8 * q + 0] = bf16_lo(w.x); v[8 * q + 1] = bf16_hi(w.x);
                    v[8 * q + 2] = bf16_lo(w.y); v[8 * q + 3] = bf16_hi(w.y);
                    v[8 * q + 4] = bf16_lo(w.z); v[8 * q + 5] = bf16_hi(w.z);
                    v[8 * q + 6] = bf16_lo(w.w); v[8 * q + 7] = bf16_hi(w.w);
                }
                if (blk + stride < nblocks) {
                    const u32x4* p = reinterpret_cast<const u32x4*>(x) + (blk + stride) * 2;
                    pre[0] = __builtin_nontemporal_load(p);
                    pre[1] = __builtin_nontemporal_load(p + 1);
                }
            } else {
                load_block<16, BF16>(x, blk, v);
            }
            if constexpr (ROT)
                fwht<16>(v);
            const float a = block_absmax<16>(v);
            if (a == 0.0f) {
                codes[blk] = fp4_encode16(v, 1.0f); // signs only
                scales[blk] = 0;
            } else {
                uint32_t sb = e4m3_round(a / S6);
                sb = sb < 1u ? 1u : sb;
                // this lane's offsets that land on finite patterns
                const int klo = max(lo, 1 - (int)sb), khi = min(hi, 0x7E - (int)sb);
                float b[16];
                float W = 16.0f;
                if constexpr (WMSE)
                    block_roots<16>(imp, root, wsum, roots_in_lds, col * 16, b, W);
                float e1 = __builtin_huge_valf(), e2 = __builtin_huge_valf();
                int cb = 1;
                float rel = 32.0f * u; // relative part of the bound
                const bool interior = WIN != 0 && pairs_exact && (int)sb + FLO >= 8 && (int)sb + FHI <= 0x7E;
                if (WIN != 0 && __builtin_amdgcn_ballot_w64(!interior) == 0) {
                    uint32_t p1 = 0x7F800000u, p2 = 0x7F800000u;
                    sweep_fixed<WMSE, FLO, FHI>(v, b, tab, (int)sb, p1, p2);
                    // an overflowed estimate (pattern >= +inf) is never certified
                    e1 = p1 < 0x7F800000u ? __uint_as_float(p1) : __builtin_huge_valf();
                    e2 = p2 < 0x7F800000u ? __uint_as_float(p2) : __builtin_huge_valf();
                    cb = (int)sb + FLO + (int)(p1 & 0xFu);
                    rel = 64.0f * u; // + 30u from the packed offsets
                } else {
                    // offsets k and k+8 pair up in runs of eight; the rest are singles
                    for (int k = lo; k <= hi; ++k) {
                        if (((k - lo) & 15) >= 8)
                            continue; // evaluated with its partner k-8 (uniform branch)
                        const bool ok1 = k >= klo && k <= khi;
                        const int c = clamp_pattern((int)sb + k);
                        const SweepPattern t = tab[c];
                        if (k + 8 <= hi) {
                            const bool ok2 = k + 8 >= klo && k + 8 <= khi;
                            const int c8 = clamp_pattern((int)sb + k + 8);
                            float F1, F2, E2;
                            if (__builtin_amdgcn_ballot_w64(t.pair == 0.0f) == 0) {
                                // every lane's pair is an exact doubling: shared product
                                fp4_err32<WMSE, true>(v, b, t.r, F1, F2);
                                E2 = F2 * t.s2;
                            } else {
                                float unused;
                                fp4_err32<WMSE, false>(v, b, t.r, F1, unused);
                                fp4_err32<WMSE, false>(v, b, tab[c8].r, F2, unused);
                                E2 = F2 * tab[c8].s2;
                            }
                            keep_best(ok1 ? F1 * t.s2 : __builtin_huge_valf(), c, e1, e2, cb);
                            keep_best(ok2 ? E2 : __builtin_huge_valf(), c8, e1, e2, cb);
                        } else {
                            float F1, unused;
                            fp4_err32<WMSE, false>(v, b, t.r, F1, unused);
                            keep_best(ok1 ? F1 * t.s2 : __builtin_huge_valf(), c, e1, e2, cb);
                        }
                    }
                }
                // |binary64 error / S^2 - estimate| <= T(estimate): a few u
                // relative per element from the shortened arithmetic (products
                // b*y formed from the rounded y), summed by Cauchy-Schwarz, plus
                // the binary32 accumulation and the gap between fl(s S)^2 and
                // s^2 S^2.  A bounds |x| / S and 6 D / S over the window;
                // underflow of y or b*y adds at most 2^-149 per element, which
                // the A-term covers whenever W > 0 (W == 0 gives exact ties,
                // never certified).  The constants carry >= 40% slack.
                const float A = __builtin_fmaxf(a * invS * (1.0f + 4.0f * u),
                                                6.0f * e4m3_value((uint32_t)clamp_pattern((int)sb + hi))) *
                                (1.0f + 4.0f * u);
                const float tail = 64.0f * u * u * A * A * W;
                const float s1 = __builtin_amdgcn_sqrtf(W * e1) * 1.0001f;
                const float s2 = __builtin_amdgcn_sqrtf(W * e2) * 1.0001f;
                const float t1 = 16.0f * u * A * s1 + rel * e1 + tail;
                const float t2 = 16.0f * u * A * s2 + rel * e2 + tail;
                // 6 D of the window's top pattern finite: no candidate's
                // reconstruction overflows (the exact path handles those)
                const bool finite_top = 6.0f * tab[clamp_pattern((int)sb + hi)].D < __builtin_huge_valf();
                const bool certain = klo <= khi && finite_top && e1 < __builtin_huge_valf() &&
                                     ((e2 == __builtin_huge_valf()) || (e2 - t2 > e1 + t1));
                if (certain) {
                    codes[blk] = fp4_encode16(v, tab[cb].r);
                    scales[blk] = (uint8_t)cb;
                } else {
                    queued = true;
                }
            }
        }
        {
            const uint64_t m = __builtin_amdgcn_ballot_w64(queued);
            if (queued) {
                const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
                queue[wv][wq + below] = blk;
            }
            wq += (uint32_t)__builtin_popcountll(m);
        }
        if constexpr (WMSE) {
            col += col_step;
            col = col >= blocks_per_row ? col - blocks_per_row : col;
        }
        if (wq > 64u) {
            wave_sync();
            drain(wq);
            wq = 0;
        }
    }
    wave_sync();
    drain(wq);
}

// ---------------------------------------------------------------------------
// IF4: per block FP4 vs INT4 (6/7 step), indicator in the scale's bit 7
// ---------------------------------------------------------------------------

template <bool BF16, bool ROT, bool WMSE>
__global__ __launch_bounds__(kThreads) void if4_quant(
    const void* __restrict__ x, int64_t nblocks, int64_t blocks_per_row,
    const float* __restrict__ imp, const float* __restrict__ partials, int npart,
    float* __restrict__ Sp, uint2* __restrict__ codes, uint8_t* __restrict__ scales)
{
    __shared__ __attribute__((aligned(16))) float root[WMSE ? kRootCols : 1]; // read as float4
    __shared__ float wsum[WMSE ? kRootCols / 16 : 1];
    // MSE: each lane's current block for the exact path (a stride of 20 floats
    // keeps the 16-byte stores of eight consecutive lanes on distinct banks).
    // With weights the roots table already bounds the workgroups per CU, so
    // the block stays in registers there.
    __shared__ __attribute__((aligned(16))) float xslot[WMSE ? 4 : kThreads * 20];
    float* slot = xslot + (WMSE ? 0 : threadIdx.x * 20);
    const float S = global_scale(partials, npart, Sp);
    bool roots_in_lds = false;
    if constexpr (WMSE)
        roots_in_lds = roots_prologue(imp, blocks_per_row * 16, root, wsum);
    __syncthreads();
    const float S6 = 6.0f * S, invS = 1.0f / S;
    constexpr float u = 0x1p-24f;
    for (int64_t blk = (int64_t)blockIdx.x * kThreads + threadIdx.x; blk < nblocks;
         blk += (int64_t)gridDim.x * kThreads) {
        float v[16];
        load_block<16, BF16>(x, blk, v);
        if constexpr (ROT)
            fwht<16>(v);
        const float a = block_absmax<16>(v);
        if constexpr (!WMSE) {
            // stored now so that v is dead after the estimates (the register
            // budget of the common path), read back only by the exact path
#pragma unroll
            for (int i = 0; i < 16; i += 4)
                *reinterpret_cast<float4*>(slot + i) = make_float4(v[i], v[i + 1], v[i + 2], v[i + 3]);
        }
        uint2 packed;
        uint32_t sbyte;
        if (a == 0.0f) {
            sbyte = 0;
            packed = fp4_encode16(v, 1.0f); // signs only
        } else {
            uint32_t sb = e4m3_round(a / S6);
            sb = sb < 1u ? 1u : sb;
            const int64_t col0 = (blk % blocks_per_row) * 16;
            const float sv = e4m3_value(sb);
            const float D = sv * S;
            const float r = 1.0f / D;
            const float Di = D * kInt4Step;
            const float ri = 1.0f / Di;
            // binary32 estimates in units of S^2, certified when separated
            // by more than their bounds (INT4 must be strictly lower)
            float b[16];
            float W = 16.0f;
            if constexpr (WMSE)
                block_roots<16>(imp, root, wsum, roots_in_lds, col0, b, W);
            // the estimates also produce both candidates' codes: the FP4
            // conversion words (of y = v r, as the encode) and the INT4 nibbles
            uint32_t cw[2];
            float Ff, unused;
            fp4_err32<WMSE, false>(v, b, r, Ff, unused, cw);
            // at s_base |x| ri < 7 (17/16) < 7.5 unless s_base is subnormal
            // or saturated (a given S)
            uint2 int4_words;
            const float Fi = __builtin_amdgcn_ballot_w64(sb < 8u || sb >= 0x7Eu) != 0
                                 ? int4_est16_codes<WMSE, true>(v, b, ri, int4_words)
                                 : int4_est16_codes<WMSE, false>(v, b, ri, int4_words);
            const float sz = sv * kInt4Step;
            const float Ef = Ff * (sv * sv), Ei = Fi * (sz * sz);
            const float A = __builtin_fmaxf(a * invS * (1.0f + 4.0f * u), 6.0f * sv) * (1.0f + 4.0f * u);
            const float Tf = est_bound(Ef, A, W, 40.0f * u), Ti = est_bound(Ei, A, W, 40.0f * u);
            // reconstructions 6 D and 7 D_int finite (the exact path sees overflow)
            const bool finite = 6.0f * D < __builtin_huge_valf() && 7.0f * Di < __builtin_huge_valf();
            int choice = -1; // 0 FP4, 1 INT4, -1 undecided
            if (finite) {
                if (Ei + Ti < Ef - Tf)
                    choice = 1;
                else if (Ef + Tf <= Ei - Ti)
                    choice = 0;
            }
            if (choice < 0) { // exact binary64 comparison (rare)
                double ef, ei;
                if constexpr (WMSE) {
                    float w[16];
                    load_weights16(imp, col0, w);
                    ef = fp4_error16<true>(v, w, D, r);
                    ei = int4_error16<true>(v, w, Di, ri);
                } else {
                    if4_exact_errors_lds(slot, D, r, Di, ri, ef, ei);
                }
                choice = ei < ef ? 1 : 0;
            }
            if (choice == 1) {
                sbyte = sb | 0x80u;
                packed = int4_words;
            } else {
                sbyte = sb;
                packed = make_uint2(cw[0], cw[1]);
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

// one lane per block (binary32 input): block maximum, E8M0 exponent, the
// hardware encode of |v| 2^-e
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
        // 2^-e exactly (a finite maximum gives e <= 125), so |v| 2^-e is the
        // method's own product and the hardware conversion its own code
        const float r = __uint_as_float((uint32_t)(127 - e) << 23);
        codes[blk] = fp4_encode32(v, r);
        scales[blk] = (uint8_t)(e + 127);
    }
}

// eight bf16 values of a 16-byte piece, widened
__device__ __forceinline__ void unpack8_bf16(const u32x4 w, float* v)
{
    v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x);
    v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
    v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z);
    v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
}

// 32-point Hadamard of a block spread over a quad (lane s holds elements
// 8s..8s+7): butterfly widths 1, 2, 4 inside the lane, then 8 and 16 across
// the quad -- the in-register transform's order and roundings.  Across lanes
// the lower partner keeps a + b and the upper a - b, each as one rounding of
// fma(+-1, own, partner's).
__device__ __forceinline__ void fwht32_quad(float* v, int s)
{
#pragma unroll
    for (int h = 1; h < 8; h *= 2)
#pragma unroll
        for (int i = 0; i < 8; i += 2 * h)
#pragma unroll
            for (int j = i; j < i + h; ++j) {
                const float a = v[j], b = v[j + h];
                v[j] = a + b;
                v[j + h] = a - b;
            }
    const float sg1 = (s & 1) ? -1.0f : 1.0f, sg2 = (s & 2) ? -1.0f : 1.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k)
        v[k] = __builtin_fmaf(sg1, v[k], quad_xor<1>(v[k]));
#pragma unroll
    for (int k = 0; k < 8; ++k)
        v[k] = __builtin_fmaf(sg2, v[k], quad_xor<2>(v[k]));
    const float c = __uint_as_float(0x3E3504F3u); // fl32(1/sqrt(32))
#pragma unroll
    for (int k = 0; k < 8; ++k)
        v[k] = v[k] * c;
}

// the block maximum of a quad's 32 values
__device__ __forceinline__ float quad_absmax(const float* v)
{
    float a = block_absmax<8>(v);
    a = __builtin_fmaxf(a, quad_xor<1>(a));
    return __builtin_fmaxf(a, quad_xor<2>(a));
}

// MXFP4 quantize of bf16 input with four lanes per block: lane s of a quad holds
// elements 8s..8s+7, so every load instruction reads 1 KiB contiguous (one
// 16-byte piece per lane) instead of 16-byte pieces 64 bytes apart.  The block
// maximum and the Hadamard's two widest stages cross the quad through DPP;
// each lane writes its four code bytes.
template <bool ROT>
__global__ __launch_bounds__(kThreads) void mxfp4_quant_quad(
    const void* __restrict__ x, int64_t nblocks, uint32_t* __restrict__ codes,
    uint8_t* __restrict__ scales)
{
    const int s = threadIdx.x & 3;
    const u32x4* xp = reinterpret_cast<const u32x4*>(x);
    // a quad's lanes are consecutive and nblocks * 4 is a multiple of 4, so a
    // quad is active or inactive as a whole (the DPP exchanges need that)
    for (int64_t q = (int64_t)blockIdx.x * kThreads + threadIdx.x; q < nblocks * 4;
         q += (int64_t)gridDim.x * kThreads) {
        float v[8];
        unpack8_bf16(__builtin_nontemporal_load(xp + q), v);
        if constexpr (ROT)
            fwht32_quad(v, s);
        const float a = quad_absmax(v);
        int e = (a == 0.0f) ? -127 : floor_log2_f32(a) - 2;
        e = e < -127 ? -127 : (e > 127 ? 127 : e);
        const float r = __uint_as_float((uint32_t)(127 - e) << 23);
        // every byte of the word is written: start from any value
        uint32_t c = __builtin_nondeterministic_value(0u);
        c = fp4_pack2<0>(c, v[0] * r, v[1] * r);
        c = fp4_pack2<1>(c, v[2] * r, v[3] * r);
        c = fp4_pack2<2>(c, v[4] * r, v[5] * r);
        c = fp4_pack2<3>(c, v[6] * r, v[7] * r);
        codes[q] = c; // codes holds nblocks * 4 words
        if (s == 0)
            scales[q >> 2] = (uint8_t)(e + 127);
    }
}

// 2^k as binary32, exact for k in [-149, 127]
__device__ __forceinline__ float pow2f(int k)
{
    return k >= -126 ? __uint_as_float((uint32_t)(k + 127) << 23) : __uint_as_float(1u << (k + 149));
}

// OCP E8M0 exponent of a block maximum, clamped to [-127, 127]
__device__ __forceinline__ int mx_exponent(float a)
{
    const int e = (a == 0.0f) ? -127 : floor_log2_f32(a) - 2;
    return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// binary64 block error of the MXFP4 encoding with exponent e
template <bool WMSE>
__device__ __forceinline__ double mx_error32(const float* v, const float* w, int e)
{
    const float D = pow2f(e), r = pow2f(-e);
    double E = 0.0;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        float a = __builtin_fabsf(v[i]);
        // treated as redefined here, so that a caller's loop over exponents
        // does not keep all 32 widened values live (64 VGPRs) across it
        asm volatile("" : "+v"(a));
        const float xh = e2m1_q(a * r) * D;
        const double d = (double)a - (double)xh;
        double t = d * d;
        if constexpr (WMSE)
            t = (double)w[i] * t;
        E = E + t;
    }
    return E;
}

__device__ __forceinline__ void load_weights32(const float* __restrict__ imp, int64_t col0, float* w)
{
    load_weights16(imp, col0, w);
    load_weights16(imp, col0 + 16, w + 16);
}

// binary32 estimate of the MXFP4 error at exponent e_lo + j in units of
// 2^(2 e_lo): y = v 2^-e_lo is exact, the conversion with scale P = 2^j gives
// the codes of y / P and the decode with the same scale P q, exactly
template <bool WMSE>
__device__ __forceinline__ float mx_est32(const float* y, const float* by, const float* b, float P,
                                          uint32_t (&cw)[4])
{
    float F = 0.0f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        uint32_t c = cw[g];
        c = fp4_pack2_scaled<0>(c, y[8 * g + 0], y[8 * g + 1], P);
        c = fp4_pack2_scaled<1>(c, y[8 * g + 2], y[8 * g + 3], P);
        c = fp4_pack2_scaled<2>(c, y[8 * g + 4], y[8 * g + 5], P);
        c = fp4_pack2_scaled<3>(c, y[8 * g + 6], y[8 * g + 7], P);
        float q[8];
        fp4_unpack2_scaled<0>(c, q[0], q[1], P);
        fp4_unpack2_scaled<1>(c, q[2], q[3], P);
        fp4_unpack2_scaled<2>(c, q[4], q[5], P);
        fp4_unpack2_scaled<3>(c, q[6], q[7], P);
        cw[g] = c;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int i = 8 * g + j;
            float d;
            if constexpr (WMSE)
                d = __builtin_fmaf(-b[i], q[j], by[i]);
            else
                d = y[i] - q[j];
            F = __builtin_fmaf(d, d, F);
        }
    }
    return F;
}

// MXFP4 with a window of E8M0 exponents around the OCP one, binary64 argmin
// (first least in ascending exponent) -- "Bridging the Gap ... Microscaling
// FP4" page, Method 2: format-specific scale search for E8M0.  Windows of at
// most 16 unclamped exponents take certified binary32 estimates; the rest,
// and every block they leave undecided, the exact binary64 search.
template <bool BF16, bool ROT, bool WMSE>
__global__ __launch_bounds__(kThreads) void mxfp4_sweep(
    const void* __restrict__ x, int64_t nblocks, int64_t blocks_per_row,
    const float* __restrict__ imp, int lo, int hi, uint4* __restrict__ codes,
    uint8_t* __restrict__ scales)
{
    __shared__ __attribute__((aligned(16))) float root[WMSE ? kRootCols : 1]; // read as float4
    __shared__ float wsum[WMSE ? kRootCols / 16 : 1];
    bool roots_in_lds = false;
    if constexpr (WMSE)
        roots_in_lds = roots_prologue(imp, blocks_per_row * 32, root, wsum);
    __syncthreads();
    constexpr float u = 0x1p-24f;
    const int K = hi - lo + 1;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    int64_t blk = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    BlockStream<32, BF16, WMSE> in; // ahead only where it costs no wave per SIMD
    in.prefetch(x, blk, nblocks);
    for (; blk < nblocks; blk += stride) {
        float v[32];
        in.take(x, blk, v);
        in.prefetch(x, blk + stride, nblocks);
        if constexpr (ROT)
            fwht<32>(v);
        const float a = block_absmax<32>(v);
        const int e0 = mx_exponent(a);
        const int64_t col0 = (blk % blocks_per_row) * 32;
        int eb = 1000; // chosen exponent; 1000 = undecided
        uint4 out = make_uint4(0u, 0u, 0u, 0u);
        // fast path: no clamping, and 6 * 2^e of the top exponent finite.  It
        // works on y = v 2^-e_lo alone (exact), so v is dead from here on and
        // the rare exact path below loads the block again.
        if (a != 0.0f && K <= 16 && e0 + lo >= -127 && e0 + hi <= 125) {
            const int el = e0 + lo;
            const float rl = pow2f(-el);
            float y[32], b[32], by[32];
            float W = 32.0f;
#pragma unroll
            for (int i = 0; i < 32; ++i)
                y[i] = v[i] * rl;
            if constexpr (WMSE) {
                block_roots<32>(imp, root, wsum, roots_in_lds, col0, b, W);
#pragma unroll
                for (int i = 0; i < 32; ++i)
                    by[i] = b[i] * y[i];
            }
            uint32_t cw[4] = {0u, 0u, 0u, 0u};
            float e1 = __builtin_huge_valf(), e2 = __builtin_huge_valf();
            int jb = 0;
            float P = 1.0f;
            for (int j = 0; j < K; ++j, P *= 2.0f) {
                const float E = mx_est32<WMSE>(y, by, b, P, cw);
                keep_best(E, j, e1, e2, jb);
            }
            const float A = __builtin_fmaxf(a * rl, 6.0f * pow2f(K - 1)) * (1.0f + 4.0f * u);
            const float t1 = est_bound(e1, A, W, 32.0f * u), t2 = est_bound(e2, A, W, 32.0f * u);
            if (e1 < __builtin_huge_valf() && (K == 1 || e2 - t2 > e1 + t1)) {
                eb = el + jb;
            } else if (K == 2) {
                // Two exponents whose reconstructions agree element by element
                // (both exact multiples of 2^el) have equal binary64 errors, and
                // the first wins: a block of one dominant element over values
                // that round to zero either way.
                bool same = true;
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    uint32_t c1 = cw[g], c2 = cw[g];
                    float q1[8], q2[8];
                    c1 = fp4_pack2_scaled<0>(c1, y[8 * g + 0], y[8 * g + 1], 1.0f);
                    c1 = fp4_pack2_scaled<1>(c1, y[8 * g + 2], y[8 * g + 3], 1.0f);
                    c1 = fp4_pack2_scaled<2>(c1, y[8 * g + 4], y[8 * g + 5], 1.0f);
                    c1 = fp4_pack2_scaled<3>(c1, y[8 * g + 6], y[8 * g + 7], 1.0f);
                    c2 = fp4_pack2_scaled<0>(c2, y[8 * g + 0], y[8 * g + 1], 2.0f);
                    c2 = fp4_pack2_scaled<1>(c2, y[8 * g + 2], y[8 * g + 3], 2.0f);
                    c2 = fp4_pack2_scaled<2>(c2, y[8 * g + 4], y[8 * g + 5], 2.0f);
                    c2 = fp4_pack2_scaled<3>(c2, y[8 * g + 6], y[8 * g + 7], 2.0f);
                    fp4_unpack2_scaled<0>(c1, q1[0], q1[1], 1.0f);
                    fp4_unpack2_scaled<1>(c1, q1[2], q1[3], 1.0f);
                    fp4_unpack2_scaled<2>(c1, q1[4], q1[5], 1.0f);
                    fp4_unpack2_scaled<3>(c1, q1[6], q1[7], 1.0f);
                    fp4_unpack2_scaled<0>(c2, q2[0], q2[1], 2.0f);
                    fp4_unpack2_scaled<1>(c2, q2[2], q2[3], 2.0f);
                    fp4_unpack2_scaled<2>(c2, q2[4], q2[5], 2.0f);
                    fp4_unpack2_scaled<3>(c2, q2[6], q2[7], 2.0f);
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        same = same && q1[j] == q2[j];
                }
                if (same)
                    eb = el;
            }
            // codes of v 2^-eb = y / 2^(eb - el): the conversion applies the
            // power-of-two scale exactly
            if (eb != 1000)
                out = fp4_encode32_scaled(y, pow2f(eb - el));
        }
        if (eb == 1000) { // exact binary64 search over the clamped window
            load_block<32, BF16, false>(x, blk, v);
            if constexpr (ROT)
                fwht<32>(v);
            float w[32];
            if constexpr (WMSE)
                load_weights32(imp, col0, w);
            double best = 0.0;
            int eprev = 1000;
            eb = e0;
            for (int k = lo; k <= hi; ++k) {
                int e = e0 + k;
                e = e < -127 ? -127 : (e > 127 ? 127 : e);
                if (e == eprev)
                    continue;
                const double E = mx_error32<WMSE>(v, w, e);
                if (eprev == 1000 || E < best) { // the first exponent is always taken
                    best = E;
                    eb = e;
                }
                eprev = e;
            }
            out = fp4_encode32(v, pow2f(-eb));
        }
        codes[blk] = out;
        scales[blk] = (uint8_t)(eb + 127);
    }
}

// NVFP4 Four Over Six: the block maximum onto 6 (AbsMax) or onto 4, the
// lower binary64 error kept, a tie keeps 6 (Adaptive Block-Scaled Data Types
// page, Problem; ScaleSweep page, Problem definition).  Certified binary32
// estimates decide when separated; the rest compare exactly.
template <bool BF16, bool ROT, bool WMSE>
__global__ __launch_bounds__(kThreads) void nvfp4_foursix(
    const void* __restrict__ x, int64_t nblocks, int64_t blocks_per_row,
    const float* __restrict__ imp, const float* __restrict__ partials, int npart,
    float* __restrict__ Sp, uint2* __restrict__ codes, uint8_t* __restrict__ scales)
{
    __shared__ __attribute__((aligned(16))) float root[WMSE ? kRootCols : 1]; // read as float4
    __shared__ float wsum[WMSE ? kRootCols / 16 : 1];
    __shared__ float2 tab[128]; // per pattern: D = fl32(s S) and r = fl32(1/D)
    const float S = global_scale(partials, npart, Sp);
    for (int c = threadIdx.x; c < 128; c += kThreads) {
        const float D = e4m3_value((uint32_t)(c < 0x7E ? c : 0x7E)) * S;
        tab[c] = make_float2(D, 1.0f / D);
    }
    bool roots_in_lds = false;
    if constexpr (WMSE)
        roots_in_lds = roots_prologue(imp, blocks_per_row * 16, root, wsum);
    __syncthreads();
    const float S6 = 6.0f * S, S4 = 4.0f * S, invS = 1.0f / S;
    constexpr float u = 0x1p-24f;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    int64_t blk = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    BlockStream<16, BF16, true> in;
    in.prefetch(x, blk, nblocks);
    for (; blk < nblocks; blk += stride) {
        float v[16];
        in.take(x, blk, v);
        in.prefetch(x, blk + stride, nblocks);
        if constexpr (ROT)
            fwht<16>(v);
        const float a = block_absmax<16>(v);
        uint32_t cb = 0;
        float r = 1.0f;
        uint2 packed = make_uint2(0u, 0u);
        bool have = false; // packed holds the chosen codes
        if (a != 0.0f) {
            uint32_t s6 = e4m3_round(a / S6), s4 = e4m3_round(a / S4);
            s6 = s6 < 1u ? 1u : s6;
            s4 = s4 < 1u ? 1u : s4;
            const float v6 = e4m3_value(s6), v4 = e4m3_value(s4);
            const float2 t6 = tab[s6];
            const float D6 = t6.x, r6 = t6.y;
            cb = s6;
            r = r6;
            if (s4 != s6) {
                const int64_t col0 = (blk % blocks_per_row) * 16;
                const float2 t4 = tab[s4];
                const float D4 = t4.x, r4 = t4.y;
                float b[16];
                float W = 16.0f;
                if constexpr (WMSE)
                    block_roots<16>(imp, root, wsum, roots_in_lds, col0, b, W);
                // the estimates' conversion words are each candidate's codes
                uint32_t cw[2];
                float F6, F4, unused;
                fp4_err32<WMSE, false>(v, b, r6, F6, unused, cw);
                const uint2 codes6 = make_uint2(cw[0], cw[1]);
                fp4_err32<WMSE, false>(v, b, r4, F4, unused, cw);
                const uint2 codes4 = make_uint2(cw[0], cw[1]);
                const float E6 = F6 * (v6 * v6), E4 = F4 * (v4 * v4);
                const float A = __builtin_fmaxf(a * invS * (1.0f + 4.0f * u), 6.0f * __builtin_fmaxf(v6, v4)) *
                                (1.0f + 4.0f * u);
                const float T6 = est_bound(E6, A, W, 32.0f * u), T4 = est_bound(E4, A, W, 32.0f * u);
                const bool finite = 6.0f * __builtin_fmaxf(D6, D4) < __builtin_huge_valf();
                int four = -1; // 1: s4 strictly lower, 0: s6 kept, -1 undecided
                if (finite) {
                    if (E4 + T4 < E6 - T6)
                        four = 1;
                    else if (E6 + T6 <= E4 - T4)
                        four = 0;
                }
                if (four < 0) { // exact binary64 comparison
                    float w[16];
                    if constexpr (WMSE)
                        load_weights16(imp, col0, w);
                    four = fp4_error16<WMSE>(v, w, D4, r4) < fp4_error16<WMSE>(v, w, D6, r6) ? 1 : 0;
                }
                if (four)
                    cb = s4;
                packed = four ? codes4 : codes6;
                have = true;
            }
        }
        codes[blk] = have ? packed : fp4_encode16(v, r);
        scales[blk] = (uint8_t)cb;
    }
}

// INT4 estimate in units of the INT4 step from binary32 fma, add and sub
// only (the rounding instruction and min issue at half their rate):
// t = fl(|x| r_int + M), M = 1.5 2^23, holds the exact product rounded to the
// nearest integer (ties to even) while the product is below 2^22, q = t - M
// exactly, and d = fl(|x| r_int - q) with a single rounding.  This q differs
// from the method's RNE(fl(|x| r_int)) only where fl(|x| r_int) is a tie
// that the exact product is not; |d| then moves by less than one rounding of
// the product, which the bound's per-element term covers.  CLAMP applies the
// saturation at 7, needed only where |x| r_int can reach 7.5; without it
// the product stays below 7.5 by the caller's choice of patterns.
template <bool WMSE, bool CLAMP>
__device__ __forceinline__ float int4_est16(const float* v, const float* b, float ri)
{
    constexpr float M = 12582912.0f;
    float F = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float a = __builtin_fabsf(v[i]);
        float t = __builtin_fmaf(a, ri, M);
        if constexpr (CLAMP)
            t = __builtin_fminf(t, M + 7.0f);
        const float q = t - M;
        float d = __builtin_fmaf(a, ri, -q);
        if constexpr (WMSE)
            d = b[i] * d;
        F = __builtin_fmaf(d, d, F);
    }
    return F;
}

// the two least of non-negative estimates whose low five mantissa bits carry
// the candidate's place in the window, 2 (k - lo) + (1 for INT4): the place
// moves an estimate by at most 31 ulp (62u relative), and as unsigned
// integers +inf and NaN (masked candidates, overflow) order last
__device__ __forceinline__ void keep_best_packed5(float E, uint32_t k, uint32_t& p1, uint32_t& p2)
{
    const uint32_t p = (__float_as_uint(E) & ~0x1Fu) | k;
    const uint32_t hi = p1 > p ? p1 : p; // p1 <= p2 throughout
    p2 = p2 < hi ? p2 : hi;
    p1 = p1 < p ? p1 : p;
}

// the FP4 and INT4 estimates of one pattern, e = (r, r_int, s^2, (s fl(6/7))^2)
template <bool WMSE, bool CLAMP>
__device__ __forceinline__ void if4_pattern(const float* v, const float* b, float4 e, uint32_t place,
                                            uint32_t& p1, uint32_t& p2)
{
    float Ff, unused;
    fp4_err32<WMSE, false>(v, b, e.x, Ff, unused);
    keep_best_packed5(Ff * e.z, place, p1, p2);
    keep_best_packed5(int4_est16<WMSE, CLAMP>(v, b, e.y) * e.w, place + 1u, p1, p2);
}

// IF4 over a window of patterns: per pattern the FP4 then the INT4 encoding,
// the first least binary64 error kept.  Certified binary32 estimates decide
// when the two least are separated; the other blocks join a per-wave LDS
// queue that the wave drains with the exact search, sixteen lanes per block.
// A wave's queue and its drain involve that wave alone, so the grid-stride
// loop has no workgroup barrier and the waves of a workgroup never wait for
// each other.  Six waves per SIMD for MSE (80 VGPRs, one of them spilled
// once per block) ran faster than the five the compiler picks by itself.
template <bool BF16, bool ROT, bool WMSE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(WMSE ? 4 : 6))) void if4_sweep(
    const void* __restrict__ x, int64_t nblocks, int64_t blocks_per_row,
    const float* __restrict__ imp, const float* __restrict__ partials, int npart,
    float* __restrict__ Sp, int lo, int hi, uint2* __restrict__ codes, uint8_t* __restrict__ scales)
{
    __shared__ float4 tab[128]; // D, r, D_int = fl32(D 6/7), r_int
    // per index c = clamp(s_base + k, 0, 127): r, r_int and the estimates'
    // units s^2 and (s fl(6/7))^2 over S^2.  Indices 0 and 127 stand for
    // offsets past patterns 0x01 and 0x7E, which repeat an end pattern: their
    // units are +inf, so those candidates order last.
    __shared__ float4 est[128];
    __shared__ int64_t queue[kThreads / 64][128]; // per wave: uncertified blocks
    __shared__ float stage[kThreads / 16][WMSE ? 2 : 1][16]; // a queued block and its weights per group
    __shared__ __attribute__((aligned(16))) float root[WMSE ? kRootCols : 1]; // read as float4
    __shared__ float wsum[WMSE ? kRootCols / 16 : 1];
    const float S = global_scale(partials, npart, Sp);
    for (int c = threadIdx.x; c < 128; c += kThreads) {
        const int ce = c < 1 ? 1 : (c > 0x7E ? 0x7E : c);
        const float sv = e4m3_value((uint32_t)ce);
        const float D = sv * S;
        const float Di = D * kInt4Step;
        tab[c] = make_float4(D, 1.0f / D, Di, 1.0f / Di);
        const float sz = sv * kInt4Step;
        const float inf = __builtin_huge_valf();
        est[c] = make_float4(1.0f / D, 1.0f / Di, c == ce ? sv * sv : inf, c == ce ? sz * sz : inf);
    }
    bool roots_in_lds = false;
    if constexpr (WMSE)
        roots_in_lds = roots_prologue(imp, blocks_per_row * 16, root, wsum);
    __syncthreads();
    const float S6 = 6.0f * S, invS = 1.0f / S;
    constexpr float u = 0x1p-24f;
    const bool packed = hi - lo <= 15; // 2 (hi - lo + 1) places fit five bits

    // exact binary64 search of the queued blocks: lane `sub` of a group of 16
    // takes the offsets lo + sub, lo + sub + 16, ...; the group keeps the
    // least (error, 2 c + type) pair, which is the first least error in the
    // method's order (patterns ascending, FP4 before INT4).  The block (and
    // its weights) pass through LDS and the error sums run element by
    // element in a loop that is not unrolled: the same terms in the same
    // order as fp4_error16 / int4_error16 with few live registers, so that
    // this rare path does not set the kernel's register budget.
    const int wv = threadIdx.x >> 6;
    auto wave_sync = [] {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };
    auto drain = [&](uint32_t n) {
        const int grp = threadIdx.x >> 4, sub = threadIdx.x & 15;
        for (uint32_t j0 = 0; j0 < n; j0 += 4) {
            const uint32_t j = j0 + (uint32_t)(grp & 3);
            const bool active = j < n;
            const int64_t blk = queue[wv][active ? j : 0];
            uint32_t sb;
            {
                float v[16];
                load_block<16, BF16, false>(x, blk, v);
                if constexpr (ROT)
                    fwht<16>(v);
                const float a = block_absmax<16>(v);
                sb = e4m3_round(a / S6);
                sb = sb < 1u ? 1u : sb;
                if (sub == 0) {
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        stage[grp][0][i] = v[i];
                    if constexpr (WMSE) {
                        const int64_t col0 = (blk % blocks_per_row) * 16;
#pragma unroll
                        for (int i = 0; i < 16; ++i)
                            stage[grp][WMSE ? 1 : 0][i] = imp[col0 + i];
                    }
                }
            }
            wave_sync();
            const float* xs = stage[grp][0];
            const float* ws = stage[grp][WMSE ? 1 : 0]; // read only with weights
            double best = __builtin_huge_val();
            int key = 0x7FFF;
            for (int k = lo + sub; k <= hi; k += 16) {
                const int c = clamp_pattern((int)sb + k);
                const float4 t = tab[c];
                double ef = 0.0, ei = 0.0;
#pragma unroll 1
                for (int i = 0; i < 16; ++i) {
                    const float a = __builtin_fabsf(xs[i]);
                    const float xf = e2m1_q(a * t.y) * t.x;
                    const float xi = __builtin_fminf(__builtin_rintf(a * t.w), 7.0f) * t.z;
                    const double df = (double)a - (double)xf;
                    const double di = (double)a - (double)xi;
                    double tf = df * df, ti = di * di;
                    if constexpr (WMSE) {
                        const double wi = (double)ws[i];
                        tf = wi * tf;
                        ti = wi * ti;
                    }
                    ef = ef + tf;
                    ei = ei + ti;
                }
                if (ef < best || (ef == best && 2 * c < key)) {
                    best = ef;
                    key = 2 * c;
                }
                if (ei < best || (ei == best && 2 * c + 1 < key)) {
                    best = ei;
                    key = 2 * c + 1;
                }
            }
#pragma unroll
            for (int off = 8; off > 0; off >>= 1) {
                const double E2 = __shfl_xor(best, off, 64);
                const int k2 = __shfl_xor(key, off, 64);
                if (E2 < best || (E2 == best && k2 < key)) {
                    best = E2;
                    key = k2;
                }
            }
            if (active && sub == 0) {
                float v[16];
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    v[i] = xs[i];
                const float4 t = tab[key >> 1];
                codes[blk] = (key & 1) ? encode16_int4(v, t.w) : fp4_encode16(v, t.y);
                scales[blk] = (uint8_t)((key >> 1) | ((key & 1) << 7));
            }
            wave_sync(); // the stage is rewritten next round
        }
    };

    // every lane of a wave runs the same number of iterations, so the
    // wave-wide queue count and drain stay uniform
    uint32_t wq = 0; // entries in this wave's queue (the same in every lane)
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t base = (int64_t)blockIdx.x * kThreads; base < nblocks; base += stride) {
        const int64_t blk = base + threadIdx.x;
        bool queued = false;
        if (blk < nblocks) {
            float v[16];
            load_block<16, BF16>(x, blk, v);
            if constexpr (ROT)
                fwht<16>(v);
            const float a = block_absmax<16>(v);
            if (a == 0.0f) {
                codes[blk] = fp4_encode16(v, 1.0f); // signs only
                scales[blk] = 0;
            } else {
                uint32_t sb = e4m3_round(a / S6);
                sb = sb < 1u ? 1u : sb;
                const int64_t col0 = (blk % blocks_per_row) * 16;
                const int ctop = clamp_pattern((int)sb + hi);
                float b[16];
                float W = 16.0f;
                if constexpr (WMSE)
                    block_roots<16>(imp, root, wsum, roots_in_lds, col0, b, W);
                float e1, e2, rel;
                int cb;
                if (packed) {
                    uint32_t p1 = 0x7F800000u, p2 = 0x7F800000u;
                    // below s_base |x| r_int can reach 7.5: saturate
                    for (int k = lo; k <= (hi < -1 ? hi : -1); ++k)
                        if4_pattern<WMSE, true>(v, b, est[(int)sb + k < 0 ? 0 : (int)sb + k],
                                                2u * (uint32_t)(k - lo), p1, p2);
                    if (lo <= 0 && hi >= 0) {
                        // at s_base, |x| r_int < 7 (17/16) < 7.5 unless
                        // s_base is subnormal or saturated
                        const float4 e = est[sb];
                        if (__builtin_amdgcn_ballot_w64(sb < 8u || sb >= 0x7Eu) != 0)
                            if4_pattern<WMSE, true>(v, b, e, 2u * (uint32_t)(-lo), p1, p2);
                        else
                            if4_pattern<WMSE, false>(v, b, e, 2u * (uint32_t)(-lo), p1, p2);
                    }
                    // above s_base, |x| r_int < 7 (31/32) < 7
                    for (int k = lo > 1 ? lo : 1; k <= hi; ++k)
                        if4_pattern<WMSE, false>(v, b, est[(int)sb + k > 127 ? 127 : (int)sb + k],
                                                 2u * (uint32_t)(k - lo), p1, p2);
                    e1 = p1 < 0x7F800000u ? __uint_as_float(p1) : __builtin_huge_valf();
                    e2 = p2 < 0x7F800000u ? __uint_as_float(p2) : __builtin_huge_valf();
                    const uint32_t place = p1 & 0x1Fu;
                    cb = ((int)sb + lo + (int)(place >> 1)) | ((place & 1u) ? 0x80 : 0);
                    rel = 104.0f * u; // 40u, + 62u from the packed places
                } else {
                    // wide windows: every distinct pattern once, in order
                    e1 = __builtin_huge_valf();
                    e2 = __builtin_huge_valf();
                    cb = (int)sb;
                    int cprev = -1;
                    for (int k = lo; k <= hi; ++k) {
                        const int c = clamp_pattern((int)sb + k);
                        if (c == cprev)
                            continue;
                        cprev = c;
                        const float4 e = est[c];
                        float Ff, unused;
                        fp4_err32<WMSE, false>(v, b, e.x, Ff, unused);
                        keep_best(Ff * e.z, c, e1, e2, cb);
                        keep_best(int4_est16<WMSE, true>(v, b, e.y) * e.w, c | 0x80, e1, e2, cb);
                    }
                    rel = 40.0f * u;
                }
                const float A = __builtin_fmaxf(a * invS * (1.0f + 4.0f * u),
                                                6.0f * e4m3_value((uint32_t)ctop)) * (1.0f + 4.0f * u);
                const float t1 = est_bound(e1, A, W, rel), t2 = est_bound(e2, A, W, rel);
                const float4 tt = tab[ctop];
                // the top pattern's reconstructions finite (the exact search
                // sees overflow)
                const bool finite = 6.0f * tt.x < __builtin_huge_valf() && 7.0f * tt.z < __builtin_huge_valf();
                const bool certain = finite && e1 < __builtin_huge_valf() &&
                                     (e2 == __builtin_huge_valf() || e2 - t2 > e1 + t1);
                if (certain) {
                    const float4 t = tab[cb & 0x7F];
                    codes[blk] = (cb & 0x80) ? encode16_int4(v, t.w) : fp4_encode16(v, t.y);
                    scales[blk] = (uint8_t)cb;
                } else {
                    queued = true;
                }
            }
        }
        {
            const uint64_t m = __builtin_amdgcn_ballot_w64(queued);
            if (queued) {
                const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
                queue[wv][wq + below] = blk;
            }
            wq += (uint32_t)__builtin_popcountll(m);
            if (wq > 64u) { // at most 64 join per iteration: drain before overflow
                wave_sync();
                drain(wq);
                wq = 0;
            }
        }
    }
    wave_sync();
    drain(wq);
}

// the eight codes of v[0..7] * r, r = fl32(1 / D_q).  When D_q is below
// 2^-128, r is +inf: every nonzero element saturates, and a zero element
// keeps a sign-only code as |x| / D_q = 0 does (0 * inf would be NaN, which
// the conversion turns into the saturated code)
__device__ __forceinline__ uint32_t relaxed_word(const float* v, float r)
{
    float y[8];
    if (r == __builtin_huge_valf()) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            y[j] = v[j] == 0.0f ? v[j] : v[j] * r;
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            y[j] = v[j] * r;
    }
    uint32_t wv = 0;
    wv = fp4_pack2<0>(wv, y[0], y[1]);
    wv = fp4_pack2<1>(wv, y[2], y[3]);
    wv = fp4_pack2<2>(wv, y[4], y[5]);
    wv = fp4_pack2<3>(wv, y[6], y[7]);
    return wv;
}

// FOCUS deploy-side encode: codes from the relaxed step D_q = fl32(D c)
// (one coefficient per GROUP elements), the stored scale S_dq unchanged
// (FOCUS page, Method 2: S_q = S_dq c_i; Method 3: c_k per sub-block of 8)
template <int FMT, bool BF16, int GROUP, bool GIVEN>
__global__ __launch_bounds__(kThreads) void relaxed_quant(
    const void* __restrict__ x, int64_t nblocks, const float* __restrict__ coef,
    const float* __restrict__ partials, int npart, float* __restrict__ Sp,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales)
{
    constexpr int B = (FMT == kMXFP4) ? 32 : 16;
    constexpr int NG = B / GROUP;
    const float S = (FMT == kMXFP4) ? 1.0f : global_scale(partials, npart, Sp);
    const float S6 = 6.0f * S;
    for (int64_t blk = (int64_t)blockIdx.x * kThreads + threadIdx.x; blk < nblocks;
         blk += (int64_t)gridDim.x * kThreads) {
        float v[B];
        load_block<B, BF16>(x, blk, v);
        uint32_t byte;
        float D;
        if constexpr (GIVEN) {
            // a given byte is a finite non-negative pattern (E8M0 below
            // 0xFF, E4M3 up to 0x7E)
            byte = scales[blk];
            if constexpr (FMT == kMXFP4)
                D = pow2f((int)byte - 127);
            else
                D = e4m3_value(byte) * S;
        } else if constexpr (FMT == kMXFP4) {
            const int e = mx_exponent(block_absmax<B>(v));
            byte = (uint32_t)(e + 127);
            D = pow2f(e);
        } else {
            const float a = block_absmax<B>(v);
            byte = 0;
            D = 0.0f;
            if (a != 0.0f) {
                byte = e4m3_round(a / S6);
                byte = byte < 1u ? 1u : byte;
                D = e4m3_value(byte) * S;
            }
        }
        float c[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g)
            c[g] = coef[blk * NG + g];
        uint32_t wds[B / 8];
#pragma unroll
        for (int q = 0; q < B / 8; ++q) {
            // one coefficient covers GROUP >= 8 consecutive elements
            const float cg = c[(8 * q) / GROUP];
            const float r = (D == 0.0f) ? 0.0f : 1.0f / (D * cg); // a zero step keeps signs only
            wds[q] = relaxed_word(v + 8 * q, r);
        }
        if constexpr (B == 16)
            reinterpret_cast<uint2*>(codes)[blk] = make_uint2(wds[0], wds[1]);
        else
            reinterpret_cast<uint4*>(codes)[blk] = make_uint4(wds[0], wds[1], wds[2], wds[3]);
        if constexpr (!GIVEN)
            scales[blk] = (uint8_t)byte;
    }
}

// The same encode for bf16 input with L = B/8 lanes per block (four for
// MXFP4, two for NVFP4): lane s holds elements 8s..8s+7 from one coalesced
// 16-byte load, and the coefficient of its group; the block maximum crosses
// the lanes through DPP, and each lane writes its four code bytes.
template <int FMT, int GROUP, bool GIVEN>
__global__ __launch_bounds__(kThreads) void relaxed_quant_lanes(
    const void* __restrict__ x, int64_t nblocks, const float* __restrict__ coef,
    const float* __restrict__ partials, int npart, float* __restrict__ Sp,
    uint32_t* __restrict__ codes, uint8_t* __restrict__ scales)
{
    constexpr int B = (FMT == kMXFP4) ? 32 : 16;
    constexpr int L = B / 8;
    constexpr int NG = B / GROUP;
    const int s = threadIdx.x & (L - 1);
    const float S = (FMT == kMXFP4) ? 1.0f : global_scale(partials, npart, Sp);
    const float S6 = 6.0f * S;
    const u32x4* xp = reinterpret_cast<const u32x4*>(x);
    // a block's lanes are consecutive and nblocks * L is a multiple of L, so
    // they are active or inactive together (the DPP exchanges need that)
    for (int64_t q = (int64_t)blockIdx.x * kThreads + threadIdx.x; q < nblocks * L;
         q += (int64_t)gridDim.x * kThreads) {
        const int64_t blk = q / L;
        float v[8];
        unpack8_bf16(__builtin_nontemporal_load(xp + q), v);
        uint32_t byte;
        float D;
        if constexpr (GIVEN) {
            byte = scales[blk];
            if constexpr (FMT == kMXFP4)
                D = pow2f((int)byte - 127);
            else
                D = e4m3_value(byte) * S;
        } else {
            float a = block_absmax<8>(v);
            a = __builtin_fmaxf(a, quad_xor<1>(a));
            if constexpr (L == 4)
                a = __builtin_fmaxf(a, quad_xor<2>(a));
            if constexpr (FMT == kMXFP4) {
                const int e = mx_exponent(a);
                byte = (uint32_t)(e + 127);
                D = pow2f(e);
            } else {
                byte = 0;
                D = 0.0f;
                if (a != 0.0f) {
                    byte = e4m3_round(a / S6);
                    byte = byte < 1u ? 1u : byte;
                    D = e4m3_value(byte) * S;
                }
            }
        }
        const float cg = coef[blk * NG + (8 * s) / GROUP];
        const float r = (D == 0.0f) ? 0.0f : 1.0f / (D * cg); // a zero step keeps signs only
        codes[q] = relaxed_word(v, r); // codes holds nblocks * L words
        if constexpr (!GIVEN)
            if (s == 0)
                scales[blk] = (uint8_t)byte;
    }
}

// ---------------------------------------------------------------------------
// IF3 / IF6: the adaptive FP-or-INT type at 3 and 6 bits
//
// Adaptive Block-Scaled Data Types, Methodology: the per-block pick between
// an FP grid and a scaled INT grid applies to 3- and 6-bit types as well.
// The n-bit type here is the one whose n = 4 case is IF4: FP element E2M(n-3)
// (E2M0 magnitudes {0, 1, 2, 4}; OCP E2M3, 1/8 steps below 2, 1/4 below 4,
// 1/2 up to 7.5), INT element in [-(2^(n-1)-1), 2^(n-1)-1] with step
// D fl32(FPmax/INTmax), E4M3 block scale with the indicator in bit 7, base
// scale E4M3(max|x| / (FPmax S)) and S = max|x| / (256 FPmax).  Codes are
// n-bit fields, element e at bits n e .. n e + n - 1, least significant bit
// first (IF6: 12 bytes per block, IF3: 6).  With two candidates per pattern
// the block errors are evaluated in binary64 directly, in the method's order
// of operations, so each pick equals the method's.
// ---------------------------------------------------------------------------

template <int N>
struct IfnFormat {
    static constexpr int kTop = (1 << (N - 1)) - 1;                 // INT maximum
    static constexpr float kFpMax = N == 6 ? 7.5f : 4.0f;           // FP maximum
    static constexpr float kScaleDen = 256.0f * kFpMax;             // S = G / (256 FPmax)
    static constexpr int kWords = N == 6 ? 3 : 2;                   // 32-bit words per block's codes
};

// fl32(FPmax / INTmax): fl32(7.5/31) and fl32(4/3)
template <int N>
__device__ __forceinline__ float ifn_step() { return IfnFormat<N>::kFpMax / (float)IfnFormat<N>::kTop; }

// nearest FP magnitude to y >= 0 (ties to the even code, saturating at the
// largest); returns the value and sets its magnitude code
template <int N>
__device__ __forceinline__ float fpn_round(float y, uint32_t& code)
{
    if constexpr (N == 6) {
        // adding 2^20 / 2^21 / 2^22 makes the binary32 ulp equal to the E2M3
        // step of [0,2) / [2,4) / [4,inf): round-to-nearest-even does the rest
        const float M = y < 2.0f ? 0x1p20f : (y < 4.0f ? 0x1p21f : 0x1p22f);
        const float q = __builtin_fminf((y + M) - M, 7.5f);
        const uint32_t u = __float_as_uint(q);
        // subnormal codes 0..7 are 8 q; above, (exponent field + 1) << 3 | mantissa
        code = q < 1.0f ? (uint32_t)(q * 8.0f) : ((((u >> 23) - 126u) << 3) | ((u >> 20) & 7u));
        return q;
    } else {
        // E2M0 {0, 1, 2, 4}, the midpoints 0.5, 1.5 and 3 going to the even
        // codes 0, 2, 2: up to 3 that is min(RNE(y), 2) (adding 2^23 makes the
        // binary32 ulp 1), above 3 it is 4
        const float q = __builtin_fminf((y + 0x1p23f) - 0x1p23f, 2.0f);
        const bool top = y > 3.0f;
        code = top ? 3u : (uint32_t)q;
        return top ? 4.0f : q;
    }
}

// binary64 block error of the FP grid with step D, reciprocal r; with codes,
// also the block's sign|magnitude codes
template <int N, bool WMSE>
__device__ __forceinline__ double fpn_error16(const float* v, const float* w, float D, float r,
                                             uint32_t* codes)
{
    double E = 0.0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float a = __builtin_fabsf(v[i]);
        uint32_t m;
        const float xh = fpn_round<N>(a * r, m) * D;
        const double d = (double)a - (double)xh;
        double t = d * d;
        if constexpr (WMSE)
            t = (double)w[i] * t;
        E = E + t;
        if (codes)
            codes[i] = ((__float_as_uint(v[i]) >> 31) << (N - 1)) | m;
    }
    return E;
}

// the same for the INT grid with step Di, reciprocal ri: q = min(RNE(|x| ri),
// INTmax); codes are the n-bit two's complement of +-q.  A zero element has
// q = 0 (|x| / D_int = 0), also where D_int < 2^-128 makes ri infinite and
// |x| ri would be NaN (IF6's step 7.5/31 is below 1/4, so that happens for
// the smallest patterns under the smallest global scales).
template <int N, bool WMSE>
__device__ __forceinline__ double intn_error16(const float* v, const float* w, float Di, float ri,
                                              uint32_t* codes)
{
    double E = 0.0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float a = __builtin_fabsf(v[i]);
        const float q = a == 0.0f ? 0.0f
                                  : __builtin_fminf(__builtin_rintf(a * ri), (float)IfnFormat<N>::kTop);
        const float xh = q * Di;
        const double d = (double)a - (double)xh;
        double t = d * d;
        if constexpr (WMSE)
            t = (double)w[i] * t;
        E = E + t;
        if (codes) {
            const int sq = (__float_as_uint(v[i]) >> 31) ? -(int)q : (int)q;
            codes[i] = (uint32_t)sq & ((1u << N) - 1u);
        }
    }
    return E;
}

// gfx950's FP6 conversions.  v_cvt_scalef32_2xpk16_fp6_f32 (scale 1) rounds
// 32 binary32 values to E2M3 exactly as IF6's FP grid does here (nearest,
// ties to the even code, saturating at 7.5, the sign kept; an in-bounds
// probe matched the exact rounding at every midpoint +-1 ulp, on the grid,
// far beyond 7.5 and on signed zeros) and packs the 6-bit codes least
// significant first, value j of its first operand in field 2j and value j of
// its second in field 2j + 1; v_cvt_scalef32_pk32_f32_fp6 decodes the 32
// fields in order.  So elements 2j and 2j + 1 of a block go to value j of
// the two operands, and fields 0..15 -- the first three words -- are the
// block's IF6 FP codes in the stored layout.  Values 8..15 of both operands
// are unspecified padding whose codes are ignored.
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x32 __attribute__((ext_vector_type(32)));
typedef uint32_t u32x6 __attribute__((ext_vector_type(6)));

__device__ __forceinline__ u32x6 fp6_encode16(const float* v, float r, f32x16& a, f32x16& b)
{
    a = __builtin_nondeterministic_value(a);
    b = __builtin_nondeterministic_value(b);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        a[j] = v[2 * j] * r;
        b[j] = v[2 * j + 1] * r;
    }
    return __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(a, b, 1.0f);
}

// IF6's FP estimate through the hardware rounding: y = fl(v r) (signed, the
// same magnitude as fl(|x| r)), q its decoded E2M3 value, d = y - q
template <bool WMSE>
__device__ __forceinline__ float fp6_est16(const float* v, const float* bw, float r)
{
    f32x16 a, b;
    const u32x6 c = fp6_encode16(v, r, a, b);
    const f32x32 q = __builtin_amdgcn_cvt_scalef32_pk32_f32_fp6(c, 1.0f);
    float F = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        float d = ((e & 1) ? b[e / 2] : a[e / 2]) - q[e];
        if constexpr (WMSE)
            d = bw[e] * d;
        F = __builtin_fmaf(d, d, F);
    }
    return F;
}

// binary32 estimate of the FP grid's block error in units of D^2, from the
// method's own codes (the FP rounding of fl(|x| r)): d = y - q, with weights
// b d (b = sqrt(w)).  Same per-element error terms as the FP4 estimate.
template <int N, bool WMSE>
__device__ __forceinline__ float fpn_est16(const float* v, const float* b, float r)
{
    float F = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        uint32_t m;
        const float y = __builtin_fabsf(v[i]) * r;
        float d = y - fpn_round<N>(y, m);
        if constexpr (WMSE)
            d = b[i] * d;
        F = __builtin_fmaf(d, d, F);
    }
    return F;
}

// the INT grid's estimate in units of D_int^2: t = fl(|x| ri + 1.5 2^23)
// holds the exact product rounded to the nearest integer, saturated at
// INTmax, q = t - 1.5 2^23, d = fl(|x| ri - q) with one rounding (q differs
// from the method's only where fl(|x| ri) is a tie; |d| then moves by less
// than one rounding of the product).  An infinite ri (D_int below 2^-128)
// gives NaN or +inf, which the caller treats as undecided.
template <int N, bool WMSE>
__device__ __forceinline__ float intn_est16(const float* v, const float* b, float ri)
{
    constexpr float M = 12582912.0f;
    float F = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float a = __builtin_fabsf(v[i]);
        const float t = __builtin_fminf(__builtin_fmaf(a, ri, M), M + (float)IfnFormat<N>::kTop);
        float d = __builtin_fmaf(a, ri, -(t - M));
        if constexpr (WMSE)
            d = b[i] * d;
        F = __builtin_fmaf(d, d, F);
    }
    return F;
}

// the method's n-bit codes of the block on the FP grid (reciprocal r) or the
// INT grid (reciprocal ri)
template <int N>
__device__ __forceinline__ void fpn_codes16(const float* v, float r, uint32_t* codes)
{
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t xb = __float_as_uint(v[i]);
        const float y = __builtin_fabsf(v[i]) * r;
        if constexpr (N == 3) {
            // E2M0: t = fl(y + 2^23) - 2^23 is RNE(y); min(RNE(y), 2) is the
            // code up to 3 and 3 (the value 4) above it, so the low two bits
            // of t clamped to 2^23 + 2 (or 2^23 + 3 above 3) are the
            // magnitude code; the sign goes to bit 2
            const float t = y > 3.0f ? 0x1p23f + 3.0f : __builtin_fminf(y + 0x1p23f, 0x1p23f + 2.0f);
            codes[i] = (__float_as_uint(t) & 3u) | ((xb >> 29) & ~3u); // xb >> 29 < 8
        } else {
            uint32_t m;
            fpn_round<N>(y, m);
            codes[i] = ((xb >> 31) << (N - 1)) | m;
        }
    }
}

// INT codes are the n-bit two's complement of sign(x) min(RNE(fl(|x| ri)),
// INTmax).  With a finite ri, t = fl(fl(x ri) + 1.5 2^23) holds that signed
// integer plus 1.5 2^23 (the binary32 ulp there is 1, and rounding to nearest
// even is symmetric about 1.5 2^23, which is even); clamped to 1.5 2^23 +-
// INTmax, the low n bits of t are the code.  An infinite ri (D_int below
// 2^-128) takes the plain form, where a zero element stays 0.
template <int N>
__device__ __forceinline__ void intn_codes16(const float* v, float ri, uint32_t* codes)
{
    constexpr float M = 12582912.0f, T = (float)IfnFormat<N>::kTop;
    if (ri < __builtin_huge_valf()) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float t = __builtin_amdgcn_fmed3f(v[i] * ri + M, M - T, M + T);
            codes[i] = __float_as_uint(t) & ((1u << N) - 1u);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float a = __builtin_fabsf(v[i]);
            const float q = a == 0.0f ? 0.0f : T;
            const int sq = (__float_as_uint(v[i]) >> 31) ? -(int)q : (int)q;
            codes[i] = (uint32_t)sq & ((1u << N) - 1u);
        }
    }
}

// the block's 16 n-bit codes as 32-bit words, code i at bits n i .. n i + n - 1
template <int N>
__device__ __forceinline__ void pack_ifn(const uint32_t* c, uint32_t* w)
{
    uint64_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int sh = N * i;
        if (sh < 64) {
            lo |= (uint64_t)c[i] << sh;
            if (sh + N > 64)
                hi |= (uint64_t)c[i] >> (64 - sh);
        } else {
            hi |= (uint64_t)c[i] << (sh - 64);
        }
    }
    w[0] = (uint32_t)lo;
    w[1] = (uint32_t)(lo >> 32);
    if constexpr (N == 6)
        w[2] = (uint32_t)hi;
}

template <int N>
__device__ __forceinline__ void store_ifn(uint8_t* __restrict__ codes, int64_t blk, const uint32_t* w)
{
    if constexpr (N == 6) { // 12 bytes, 4-byte aligned
        uint32_t* p = reinterpret_cast<uint32_t*>(codes) + 3 * blk;
        p[0] = w[0];
        p[1] = w[1];
        p[2] = w[2];
    } else {                // 6 bytes, 2-byte aligned
        uint16_t* p = reinterpret_cast<uint16_t*>(codes) + 3 * blk;
        p[0] = (uint16_t)w[0];
        p[1] = (uint16_t)(w[0] >> 16);
        p[2] = (uint16_t)w[1];
    }
}

// One lane per block.  Patterns of the window (one for the base scale alone)
// are tried in ascending order, each with the FP grid and then the INT grid;
// the first least binary64 error wins.
template <int N, bool BF16, bool ROT, bool WMSE>
__global__ __launch_bounds__(kThreads) void ifn_quant(
    const void* __restrict__ x, int64_t nblocks, int64_t blocks_per_row,
    const float* __restrict__ imp, const float* __restrict__ partials, int npart,
    float* __restrict__ Sp, int lo, int hi, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales)
{
    using F = IfnFormat<N>;
    // per pattern: D = fl32(s S), r = fl32(1/D), D_int = fl32(D step), r_int,
    // and the estimates' units over S^2: s^2 and (s step)^2
    __shared__ float4 tab[128];
    __shared__ float2 units[128];
    __shared__ __attribute__((aligned(16))) float root[WMSE ? kRootCols : 1]; // read as float4
    __shared__ float wsum[WMSE ? kRootCols / 16 : 1];
    float S;
    if (npart == 0) {
        S = *Sp;
    } else { // S = G / (256 FPmax), floored at 2^-117 (1 for G == 0)
        __shared__ float red[kThreads / 64];
        float m = 0.0f;
        for (int i = threadIdx.x; i < npart; i += kThreads)
            m = __builtin_fmaxf(m, partials[i]);
        m = wave_max(m);
        if ((threadIdx.x & 63) == 0)
            red[threadIdx.x >> 6] = m;
        __syncthreads();
        float g = red[0];
#pragma unroll
        for (int w = 1; w < kThreads / 64; ++w)
            g = __builtin_fmaxf(g, red[w]);
        float s = g / F::kScaleDen;
        s = __builtin_fmaxf(s, 0x1p-117f);
        S = (g == 0.0f) ? 1.0f : s;
        if (blockIdx.x == 0 && threadIdx.x == 0)
            *Sp = S;
    }
    const float step = ifn_step<N>();
    for (int c = threadIdx.x; c < 128; c += kThreads) {
        const float sv = e4m3_value((uint32_t)(c < 0x7E ? c : 0x7E));
        const float D = sv * S;
        const float Di = D * step;
        tab[c] = make_float4(D, 1.0f / D, Di, 1.0f / Di);
        const float sz = sv * step;
        units[c] = make_float2(sv * sv, sz * sz);
    }
    bool roots_in_lds = false;
    if constexpr (WMSE)
        roots_in_lds = roots_prologue(imp, blocks_per_row * 16, root, wsum);
    __syncthreads();
    const float SM = F::kFpMax * S;
    const float invS = 1.0f / S;
    constexpr float u = 0x1p-24f;
    for (int64_t blk = (int64_t)blockIdx.x * kThreads + threadIdx.x; blk < nblocks;
         blk += (int64_t)gridDim.x * kThreads) {
        float v[16];
        load_block<16, BF16>(x, blk, v);
        if constexpr (ROT)
            fwht<16>(v);
        const float a = block_absmax<16>(v);
        uint32_t cds[16], words[F::kWords];
        uint32_t sbyte = 0;
        if (a == 0.0f) { // scale 0, codes keep only the signs
#pragma unroll
            for (int i = 0; i < 16; ++i)
                cds[i] = (__float_as_uint(v[i]) >> 31) << (N - 1);
        } else {
            const int64_t col0 = (blk % blocks_per_row) * 16;
            uint32_t sb = e4m3_round(a / SM);
            sb = sb < 1u ? 1u : sb;
            // binary32 estimates of every (pattern, grid) in the method's
            // order, in units of S^2, certified by the bound of the FP4
            // estimates (A bounds |x| / S and FPmax D / S over the window;
            // 40u covers the units (s fl(step))^2 against fl(fl(s S) step)^2)
            float b[16];
            float W = 16.0f;
            if constexpr (WMSE)
                block_roots<16>(imp, root, wsum, roots_in_lds, col0, b, W);
            float e1 = __builtin_huge_valf(), e2 = __builtin_huge_valf();
            int cb = (int)sb;
            bool defined = true;
            int prev = -1;
            for (int k = lo; k <= hi; ++k) {
                const int c = clamp_pattern((int)sb + k);
                if (c == prev)
                    continue;
                prev = c;
                const float4 t = tab[c];
                const float2 un = units[c];
                float Ef;
                if constexpr (N == 6)
                    Ef = fp6_est16<WMSE>(v, b, t.y) * un.x;
                else
                    Ef = fpn_est16<N, WMSE>(v, b, t.y) * un.x;
                const float Ei = intn_est16<N, WMSE>(v, b, t.w) * un.y;
                // a NaN or infinite estimate (an infinite r_int, or |x| r
                // overflowing) leaves the block to the exact search
                defined = defined && Ef < __builtin_huge_valf() && Ei < __builtin_huge_valf();
                keep_best(Ef, c, e1, e2, cb);
                keep_best(Ei, c | 0x80, e1, e2, cb);
            }
            const int ctop = clamp_pattern((int)sb + hi);
            const float A = __builtin_fmaxf(a * invS * (1.0f + 4.0f * u),
                                            F::kFpMax * e4m3_value((uint32_t)ctop)) * (1.0f + 4.0f * u);
            const float t1 = est_bound(e1, A, W, 40.0f * u), t2 = est_bound(e2, A, W, 40.0f * u);
            const float4 tt = tab[ctop];
            const bool finite = F::kFpMax * tt.x < __builtin_huge_valf() &&
                                (float)F::kTop * tt.z < __builtin_huge_valf();
            const bool certain = defined && finite && e1 < __builtin_huge_valf() &&
                                 (e2 == __builtin_huge_valf() || e2 - t2 > e1 + t1);
            if (certain) {
                sbyte = (uint32_t)cb;
            } else { // exact binary64 search (rare)
                float w[16];
                if constexpr (WMSE)
                    load_weights16(imp, col0, w);
                double best = __builtin_huge_val();
                prev = -1;
                for (int k = lo; k <= hi; ++k) {
                    const int c = clamp_pattern((int)sb + k);
                    if (c == prev)
                        continue;
                    prev = c;
                    const float4 t = tab[c];
                    const double ef = fpn_error16<N, WMSE>(v, w, t.x, t.y, nullptr);
                    if (ef < best) {
                        best = ef;
                        sbyte = (uint32_t)c;
                    }
                    const double ei = intn_error16<N, WMSE>(v, w, t.z, t.w, nullptr);
                    if (ei < best) {
                        best = ei;
                        sbyte = (uint32_t)c | 0x80u;
                    }
                }
            }
            const float4 t = tab[sbyte & 0x7Fu];
            if constexpr (N == 6) {
                if (!(sbyte & 0x80u)) {
                    f32x16 pa, pb;
                    const u32x6 c6 = fp6_encode16(v, t.y, pa, pb);
                    words[0] = c6[0];
                    words[1] = c6[1];
                    words[2] = c6[2];
                    store_ifn<N>(codes, blk, words);
                    scales[blk] = (uint8_t)sbyte;
                    continue;
                }
            }
            if (sbyte & 0x80u)
                intn_codes16<N>(v, t.w, cds);
            else
                fpn_codes16<N>(v, t.y, cds);
        }
        pack_ifn<N>(cds, words);
        store_ifn<N>(codes, blk, words);
        scales[blk] = (uint8_t)sbyte;
    }
}

// ---------------------------------------------------------------------------
// dequantize and error
// ---------------------------------------------------------------------------

// decode one block's B values (before any un-rotation): FP4 nibbles through
// the hardware E2M1 decode (exact), times the block step D with one binary32
// rounding, x_hat = fl32(+-v * D); IF4 INT4 blocks as q * fl32(D * fl32(6/7))
// 32-bit words of one block's codes
template <int FMT, int B>
constexpr int code_words() { return FMT == kIF6 ? 3 : B / 8; }

// value of E2M(n-3) magnitude code m: E2M3 subnormals m/8, then
// 2^(e-1) (1 + f/8); E2M0 {0, 1, 2, 4}
template <int N>
__device__ __forceinline__ float fpn_value(uint32_t m)
{
    if constexpr (N == 6)
        return m < 8u ? (float)m * 0.125f : __uint_as_float(((m >> 3) + 126u) << 23 | (m & 7u) << 20);
    else
        return m == 3u ? 4.0f : (float)m;
}

template <int FMT, int B>
__device__ __forceinline__ void decode_block(const uint32_t* wds, uint32_t sb, float S, float* o)
{
    if constexpr (FMT == kIF3 || FMT == kIF6) {
        constexpr int N = FMT == kIF6 ? 6 : 3;
        const uint32_t mag = sb & 0x7Fu;
        const float D = ((mag == 0x7Fu) ? __builtin_nanf("") : e4m3_value(mag)) * S;
        const uint64_t lo = (uint64_t)wds[0] | ((uint64_t)wds[1] << 32);
        const uint64_t hi = N == 6 ? (uint64_t)wds[2] : 0u;
        const float Di = D * ifn_step<N>();
#pragma unroll
        for (int i = 0; i < B; ++i) {
            const int sh = N * i;
            uint32_t c = (uint32_t)(sh < 64 ? lo >> sh : hi >> (sh - 64));
            if (sh < 64 && sh + N > 64)
                c |= (uint32_t)(hi << (64 - sh));
            c &= (1u << N) - 1u;
            if (sb & 0x80u) { // INT: n-bit two's complement
                const int q = (c >> (N - 1)) ? (int)c - (1 << N) : (int)c;
                o[i] = (float)q * Di;
            } else {
                const float val = fpn_value<N>(c & ((1u << (N - 1)) - 1u)) * D;
                o[i] = (c >> (N - 1)) ? -val : val;
            }
        }
        return;
    }
    float D;
    if constexpr (FMT == kMXFP4) {
        D = (sb == 0xFFu) ? __builtin_nanf("")
            : (sb == 0u ? __uint_as_float(0x00400000u) : __uint_as_float(sb << 23));
    } else {
        const uint32_t mag = sb & 0x7Fu;
        float s = (mag == 0x7Fu) ? __builtin_nanf("") : e4m3_value(mag);
        if (FMT == kNVFP4 && (sb & 0x80u))
            s = -s;
        D = s * S;
        if (FMT == kIF4 && (sb & 0x80u)) {
            const float Di = D * kInt4Step;
#pragma unroll
            for (int i = 0; i < B; ++i) {
                const uint32_t nib = (wds[i >> 3] >> (4 * (i & 7))) & 0xFu;
                const int q = (nib & 8u) ? (int)nib - 16 : (int)nib;
                o[i] = (float)q * Di;
            }
            return;
        }
    }
#pragma unroll
    for (int w = 0; w < B / 8; ++w) {
        float q[8];
        fp4_unpack2<0>(wds[w], q[0], q[1]);
        fp4_unpack2<1>(wds[w], q[2], q[3]);
        fp4_unpack2<2>(wds[w], q[4], q[5]);
        fp4_unpack2<3>(wds[w], q[6], q[7]);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            o[8 * w + j] = q[j] * D;
    }
}

template <int FMT, int B>
__device__ __forceinline__ void load_codes(const uint8_t* __restrict__ codes, int64_t blk, uint32_t* wds)
{
    if constexpr (FMT == kIF6) {        // 12 bytes per block, 4-byte aligned
        const uint32_t* p = reinterpret_cast<const uint32_t*>(codes) + 3 * blk;
        wds[0] = p[0];
        wds[1] = p[1];
        wds[2] = p[2];
    } else if constexpr (FMT == kIF3) { // 6 bytes per block, 2-byte aligned
        const uint16_t* p = reinterpret_cast<const uint16_t*>(codes) + 3 * blk;
        wds[0] = (uint32_t)p[0] | ((uint32_t)p[1] << 16);
        wds[1] = (uint32_t)p[2];
    } else if constexpr (B == 16) {
        const uint2 c = reinterpret_cast<const uint2*>(codes)[blk];
        wds[0] = c.x;
        wds[1] = c.y;
    } else {
        const uint4 c = reinterpret_cast<const uint4*>(codes)[blk];
        wds[0] = c.x; wds[1] = c.y; wds[2] = c.z; wds[3] = c.w;
    }
}

// One lane decodes one block; each wave then writes its 64 consecutive
// blocks' output as whole 16-byte chunks in lane order (1 KiB contiguous per
// store instruction) after passing them through LDS, instead of every lane
// storing its own 32-128 bytes with a stride across the wave.
template <int FMT, int B, bool ROT, bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void dequant(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const float* __restrict__ Sp, int64_t nblocks, void* __restrict__ y)
{
    constexpr int NQ = B * (OUT_BF16 ? 2 : 4) / 16; // 16-byte output chunks per block
    __shared__ u32x4 stage[kThreads / 64][64 * NQ];
    const int lane = threadIdx.x & 63;
    u32x4* st = stage[threadIdx.x >> 6];
    const float S = (FMT == kMXFP4) ? 1.0f : *Sp;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    // wave-uniform loop: base is this wave's first block
    for (int64_t base = (int64_t)blockIdx.x * kThreads + (threadIdx.x & ~63); base < nblocks; base += stride) {
        const int64_t blk = base + lane;
        if (blk < nblocks) {
            uint32_t wds[code_words<FMT, B>()];
            load_codes<FMT, B>(codes, blk, wds);
            float o[B];
            decode_block<FMT, B>(wds, scales[blk], S, o);
            if constexpr (ROT)
                fwht<B>(o);
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                u32x4 t;
                if constexpr (OUT_BF16) {
                    t.x = bf16_pair(o[8 * q + 0], o[8 * q + 1]);
                    t.y = bf16_pair(o[8 * q + 2], o[8 * q + 3]);
                    t.z = bf16_pair(o[8 * q + 4], o[8 * q + 5]);
                    t.w = bf16_pair(o[8 * q + 6], o[8 * q + 7]);
                } else {
                    t.x = __float_as_uint(o[4 * q + 0]);
                    t.y = __float_as_uint(o[4 * q + 1]);
                    t.z = __float_as_uint(o[4 * q + 2]);
                    t.w = __float_as_uint(o[4 * q + 3]);
                }
                st[lane * NQ + q] = t;
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int64_t left = nblocks - base;
        const int nch = (left < 64 ? (int)left : 64) * NQ; // chunks of this wave's blocks
        u32x4* out = reinterpret_cast<u32x4*>(y) + base * NQ;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int ch = q * 64 + lane;
            if (ch < nch)
                __builtin_nontemporal_store(st[ch], out + ch);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
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
        uint32_t wds[code_words<FMT, B>()];
        load_codes<FMT, B>(codes, blk, wds);
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
// static scratch of the entry point that allocates nothing
// ---------------------------------------------------------------------------

// One workspace's worth of device memory at file scope.  Every GPU the
// library runs on holds its own copy, at its own address, until the process
// ends.  In host code `scratch` names a host-side stand-in, not device
// memory: kernels receive the address looked up below, never the name.
static __device__ __align__(256) unsigned char scratch[kWorkspaceBytes];

constexpr int kMaxScratchDevices = 256;
static std::mutex scratch_lock;
static void* scratch_addr[kMaxScratchDevices]; // per device, filled on first use

hipError_t static_scratch(hipStream_t stream, void** out)
{
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess)
        return e;
    int dev = cur;
    if (stream != nullptr && (e = hipStreamGetDevice(stream, &dev)) != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxScratchDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> guard(scratch_lock);
    if (scratch_addr[dev] == nullptr) {
        // the symbol's address on `dev` is looked up with `dev` current
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess)
            return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t r = hipSetDevice(cur);
            if (e == hipSuccess)
                e = r;
        }
        if (e != hipSuccess)
            return e;
        scratch_addr[dev] = p;
    }
    *out = scratch_addr[dev];
    return hipSuccess;
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

// one full round of resident workgroups of `kernel` (every compute unit
// filled once), so that grid-stride kernels amortize their prologue
template <typename K>
static int resident_groups(K kernel)
{
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, 0) != hipSuccess)
        return 2048;
    return per_cu > 0 && cus > 0 ? per_cu * cus : 2048;
}

template <typename K>
static int sweep_grid(K kernel, int64_t nb)
{
    const int64_t need = (nb + kThreads - 1) / kThreads;
    const int cap = resident_groups(kernel);
    return (int)(need < cap ? (need < 1 ? 1 : need) : cap);
}

template <bool BF16, bool ROT>
static void launch_nvfp4(const QuantArgs& a, int64_t nb, const float* part, int npart, int grid)
{
    const int64_t bpr = a.cols / 16;
    float* Sp = a.global_scale;
    uint2* codes = reinterpret_cast<uint2*>(a.codes);
    if (a.rule == kAbsMax) {
        hipLaunchKernelGGL((nvfp4_absmax<BF16, ROT>), grid, kThreads, 0, a.stream,
                           a.x, nb, part, npart, Sp, codes, a.scales);
    } else if (a.rule == kFourSix) {
        // one round of resident workgroups: each builds its LDS tables once
        if (a.objective == kWMSE) {
            auto k = nvfp4_foursix<BF16, ROT, true>;
            hipLaunchKernelGGL(k, sweep_grid(k, nb), kThreads, 0, a.stream,
                               a.x, nb, bpr, a.importance, part, npart, Sp, codes, a.scales);
        } else {
            auto k = nvfp4_foursix<BF16, ROT, false>;
            hipLaunchKernelGGL(k, sweep_grid(k, nb), kThreads, 0, a.stream,
                               a.x, nb, bpr, a.importance, part, npart, Sp, codes, a.scales);
        }
    } else {
        // the pages' two windows get a fully unrolled specialization
        const int win = (a.lo == -3 && a.hi == 7) ? 1 : ((a.lo == -8 && a.hi == 7) ? 2 : 0);
#define FP4Q_SWEEP(W, WI)                                                                      \
    {                                                                                         \
        auto k = nvfp4_sweep<BF16, ROT, W, WI>;                                               \
        hipLaunchKernelGGL(k, sweep_grid(k, nb), kThreads, 0, a.stream, a.x, nb, bpr,           \
                           a.importance, part, npart, Sp, a.lo, a.hi, codes, a.scales);       \
    }
        const bool wm = a.objective == kWMSE;
        if (win == 1) {
            if (wm) FP4Q_SWEEP(true, 1) else FP4Q_SWEEP(false, 1)
        } else if (win == 2) {
            if (wm) FP4Q_SWEEP(true, 2) else FP4Q_SWEEP(false, 2)
        } else {
            if (wm) FP4Q_SWEEP(true, 0) else FP4Q_SWEEP(false, 0)
        }
#undef FP4Q_SWEEP
    }
}

template <bool BF16, bool ROT>
static void launch_if4(const QuantArgs& a, int64_t nb, const float* part, int npart, int grid)
{
    const int64_t bpr = a.cols / 16;
    float* Sp = a.global_scale;
    uint2* codes = reinterpret_cast<uint2*>(a.codes);
    const bool wm = a.objective == kWMSE;
    // kernels that build LDS tables run one round of resident workgroups
    if (a.rule == kSweep) {
        if (wm) {
            auto k = if4_sweep<BF16, ROT, true>;
            hipLaunchKernelGGL(k, sweep_grid(k, nb), kThreads, 0, a.stream, a.x, nb,
                               bpr, a.importance, part, npart, Sp, a.lo, a.hi, codes, a.scales);
        } else {
            auto k = if4_sweep<BF16, ROT, false>;
            hipLaunchKernelGGL(k, sweep_grid(k, nb), kThreads, 0, a.stream, a.x, nb,
                               bpr, a.importance, part, npart, Sp, a.lo, a.hi, codes, a.scales);
        }
    } else if (wm) {
        auto k = if4_quant<BF16, ROT, true>;
        hipLaunchKernelGGL(k, sweep_grid(k, nb), kThreads, 0, a.stream,
                           a.x, nb, bpr, a.importance, part, npart, Sp, codes, a.scales);
    } else {
        hipLaunchKernelGGL((if4_quant<BF16, ROT, false>), grid, kThreads, 0, a.stream,
                           a.x, nb, bpr, a.importance, part, npart, Sp, codes, a.scales);
    }
}

template <int N, bool BF16, bool ROT>
static void launch_ifn(const QuantArgs& a, int64_t nb, const float* part, int npart)
{
    const int64_t bpr = a.cols / 16;
    const int lo = a.rule == kSweep ? a.lo : 0, hi = a.rule == kSweep ? a.hi : 0;
    // builds an LDS table of the patterns' steps: one round of resident workgroups
    if (a.objective == kWMSE) {
        auto k = ifn_quant<N, BF16, ROT, true>;
        hipLaunchKernelGGL(k, sweep_grid(k, nb), kThreads, 0, a.stream, a.x, nb, bpr, a.importance,
                           part, npart, a.global_scale, lo, hi, a.codes, a.scales);
    } else {
        auto k = ifn_quant<N, BF16, ROT, false>;
        hipLaunchKernelGGL(k, sweep_grid(k, nb), kThreads, 0, a.stream, a.x, nb, bpr, a.importance,
                           part, npart, a.global_scale, lo, hi, a.codes, a.scales);
    }
}

template <int N>
static void launch_ifn_dt(const QuantArgs& a, int64_t nb, const float* part, int npart)
{
    const bool rot = a.rotate != 0;
    if (a.bf16)
        rot ? launch_ifn<N, true, true>(a, nb, part, npart) : launch_ifn<N, true, false>(a, nb, part, npart);
    else
        rot ? launch_ifn<N, false, true>(a, nb, part, npart) : launch_ifn<N, false, false>(a, nb, part, npart);
}

template <bool BF16, bool ROT>
static void launch_mxfp4(const QuantArgs& a, int64_t nb, int grid)
{
    uint4* codes = reinterpret_cast<uint4*>(a.codes);
    if (a.rule == kSweep) {
        const int64_t bpr = a.cols / 32;
        if (a.objective == kWMSE) { // builds LDS tables: one round of resident workgroups
            auto k = mxfp4_sweep<BF16, ROT, true>;
            hipLaunchKernelGGL(k, sweep_grid(k, nb), kThreads, 0, a.stream, a.x, nb,
                               bpr, a.importance, a.lo, a.hi, codes, a.scales);
        } else {
            hipLaunchKernelGGL((mxfp4_sweep<BF16, ROT, false>), grid, kThreads, 0, a.stream, a.x, nb,
                               bpr, a.importance, a.lo, a.hi, codes, a.scales);
        }
    } else {
        if constexpr (BF16) // four lanes per block
            hipLaunchKernelGGL((mxfp4_quant_quad<ROT>), grid_for(nb * 4, kQuantGroupCap), kThreads, 0,
                               a.stream, a.x, nb, reinterpret_cast<uint32_t*>(a.codes), a.scales);
        else
            hipLaunchKernelGGL((mxfp4_quant<BF16, ROT>), grid, kThreads, 0, a.stream, a.x, nb, codes,
                               a.scales);
    }
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

// Launches the partial maxima of the global-scale rule when S is computed
// (NVFP4, IF4) and returns how many there are: 0 means that the quantize
// kernel reads S from a.global_scale (given by the caller, or written here
// for an empty tensor).
static int launch_scale_prologue(const QuantArgs& a)
{
    const int64_t n = a.rows * a.cols;
    float* partials = reinterpret_cast<float*>(a.workspace);
    if (a.format == kMXFP4 || a.global_scale_given)
        return 0;
    if (n == 0) {
        // nothing to reduce: S = 1 for an empty (all-zero) tensor
        hipLaunchKernelGGL(finalize_scale, 1, 1024, 0, a.stream, partials, 0, a.global_scale);
        return 0;
    }
    const int64_t items = (a.rotate == 0) ? n * (a.bf16 ? 2 : 4) / 16 : n / 16;
    const int npart = grid_for(items, kAmaxGroups);
    if (a.bf16)
        launch_amax<true>(a, partials, npart);
    else
        launch_amax<false>(a, partials, npart);
    return npart;
}

hipError_t launch_quantize(const QuantArgs& a)
{
    const int64_t n = a.rows * a.cols;
    const int B = (a.format == kMXFP4) ? 32 : 16;
    const int64_t nb = n / B;
    const float* partials = reinterpret_cast<const float*>(a.workspace);
    const int npart = launch_scale_prologue(a);
    if (nb > 0) {
        const int grid = grid_for(nb, kQuantGroupCap);
        const bool rot = a.rotate != 0;
        const float* part = partials;
        if (a.format == kNVFP4) {
            if (a.bf16)
                rot ? launch_nvfp4<true, true>(a, nb, part, npart, grid) : launch_nvfp4<true, false>(a, nb, part, npart, grid);
            else
                rot ? launch_nvfp4<false, true>(a, nb, part, npart, grid) : launch_nvfp4<false, false>(a, nb, part, npart, grid);
        } else if (a.format == kIF4) {
            if (a.bf16)
                rot ? launch_if4<true, true>(a, nb, part, npart, grid) : launch_if4<true, false>(a, nb, part, npart, grid);
            else
                rot ? launch_if4<false, true>(a, nb, part, npart, grid) : launch_if4<false, false>(a, nb, part, npart, grid);
        } else if (a.format == kIF6) {
            launch_ifn_dt<6>(a, nb, part, npart);
        } else if (a.format == kIF3) {
            launch_ifn_dt<3>(a, nb, part, npart);
        } else {
            if (a.bf16)
                rot ? launch_mxfp4<true, true>(a, nb, grid) : launch_mxfp4<true, false>(a, nb, grid);
            else
                rot ? launch_mxfp4<false, true>(a, nb, grid) : launch_mxfp4<false, false>(a, nb, grid);
        }
    }
    return hipGetLastError();
}

template <int FMT, bool BF16, int GROUP>
static void launch_relaxed_g(const RelaxArgs& a, int64_t nb, const float* part, int npart, int grid)
{
    if constexpr (BF16) { // B/8 lanes per block
        constexpr int L = (FMT == kMXFP4) ? 4 : 2;
        const int g = grid_for(nb * L, kQuantGroupCap);
        uint32_t* codes = reinterpret_cast<uint32_t*>(a.codes);
        if (a.scales_given)
            hipLaunchKernelGGL((relaxed_quant_lanes<FMT, GROUP, true>), g, kThreads, 0, a.stream,
                               a.x, nb, a.coef, part, npart, a.global_scale, codes, a.scales);
        else
            hipLaunchKernelGGL((relaxed_quant_lanes<FMT, GROUP, false>), g, kThreads, 0, a.stream,
                               a.x, nb, a.coef, part, npart, a.global_scale, codes, a.scales);
        return;
    }
    if (a.scales_given)
        hipLaunchKernelGGL((relaxed_quant<FMT, BF16, GROUP, true>), grid, kThreads, 0, a.stream,
                           a.x, nb, a.coef, part, npart, a.global_scale, a.codes, a.scales);
    else
        hipLaunchKernelGGL((relaxed_quant<FMT, BF16, GROUP, false>), grid, kThreads, 0, a.stream,
                           a.x, nb, a.coef, part, npart, a.global_scale, a.codes, a.scales);
}

template <int FMT, bool BF16>
static void launch_relaxed_f(const RelaxArgs& a, int64_t nb, const float* part, int npart, int grid)
{
    constexpr int B = (FMT == kMXFP4) ? 32 : 16;
    if (a.group == 8)
        launch_relaxed_g<FMT, BF16, 8>(a, nb, part, npart, grid);
    else
        launch_relaxed_g<FMT, BF16, B>(a, nb, part, npart, grid);
}

hipError_t launch_quantize_relaxed(const RelaxArgs& r)
{
    QuantArgs a{};
    a.format = r.format;
    a.global_scale_given = r.global_scale_given;
    a.bf16 = r.bf16;
    a.x = r.x;
    a.rows = r.rows;
    a.cols = r.cols;
    a.global_scale = r.global_scale;
    a.workspace = r.workspace;
    a.stream = r.stream;
    const int npart = launch_scale_prologue(a);
    const int B = (r.format == kMXFP4) ? 32 : 16;
    const int64_t nb = r.rows * r.cols / B;
    if (nb > 0) {
        const int grid = grid_for(nb, kQuantGroupCap);
        const float* part = reinterpret_cast<const float*>(r.workspace);
        if (r.format == kMXFP4)
            r.bf16 ? launch_relaxed_f<kMXFP4, true>(r, nb, part, npart, grid)
                   : launch_relaxed_f<kMXFP4, false>(r, nb, part, npart, grid);
        else
            r.bf16 ? launch_relaxed_f<kNVFP4, true>(r, nb, part, npart, grid)
                   : launch_relaxed_f<kNVFP4, false>(r, nb, part, npart, grid);
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
    else if (a.format == kIF6)
        launch_dequant_fmt<kIF6, 16>(a, nb, grid);
    else if (a.format == kIF3)
        launch_dequant_fmt<kIF3, 16>(a, nb, grid);
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
        else if (a.format == kIF6)
            a.bf16 ? launch_error_fmt<kIF6, 16, true>(a, nb, grid, partials)
                   : launch_error_fmt<kIF6, 16, false>(a, nb, grid, partials);
        else if (a.format == kIF3)
            a.bf16 ? launch_error_fmt<kIF3, 16, true>(a, nb, grid, partials)
                   : launch_error_fmt<kIF3, 16, false>(a, nb, grid, partials);
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
