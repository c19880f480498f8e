// sgqa_device.hpp -- device helpers shared by the gfx950 kernels of libsgqa.
//
// Wave64 primitives, bf16 packing with round-to-nearest-even, the CDNA4 bf16
// MFMA operand types, and the order-preserving float key used by the top-k.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sgqa {

constexpr int kWave = 64;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;  // MFMA A/B operand (8 x bf16)
typedef __attribute__((ext_vector_type(4))) float f32x4;    // 16x16 MFMA accumulator slice
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h)
{
    return __uint_as_float(h << 16);
}

// Round a finite fp32 to bf16 (nearest, ties to even).  NaN stays NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// Round an fp64 value to bf16 (nearest, ties to even) without double rounding:
// first to fp32 rounding to odd (truncate, then set the last bit if inexact),
// which keeps enough bits for the final round-to-nearest-even to be exact.
__device__ __forceinline__ uint32_t f64_to_bf16_bits(double x)
{
    float f = __double2float_rz(x);
    uint32_t u = __float_as_uint(f);
    if ((double)f != x && (u & 0x7f800000u) != 0x7f800000u)
        u |= 1u;
    return f32_to_bf16_bits(__uint_as_float(u));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v)
{
    return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ u32x4 load16(const void *p)
{
    return *reinterpret_cast<const u32x4 *>(p);
}

// The same load marked non-temporal, for data a kernel streams through once (a whole index
// scan): it reaches a higher share of the HBM read rate than cached loads (a 4 GiB streamed
// read measured 6.4 against 5.8 TB/s).
__device__ __forceinline__ u32x4 load16_stream(const void *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

__device__ __forceinline__ f32x4 mfma_16x16x32(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x)
{
    return __builtin_amdgcn_exp2f(x);
}

__device__ __forceinline__ float fast_log2(float x)
{
    return __builtin_amdgcn_logf(x);
}

// Order-preserving map fp32 -> u32: a > b as floats <=> key(a) > key(b).
// -0.0 is folded onto +0.0 so equal scores get equal keys.
__device__ __forceinline__ uint32_t score_key(float f)
{
    uint32_t u = __float_as_uint(f == 0.0f ? 0.0f : f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_score(uint32_t k)
{
    uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
    return __uint_as_float(u);
}

// Butterfly reductions across the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float max_across_rows(float v)
{
    v = fmaxf(v, __shfl_xor(v, 16));
    v = fmaxf(v, __shfl_xor(v, 32));
    return v;
}

// The larger of two non-NaN floats in one instruction: the median of (a, b, +inf).  fmaxf
// must first quiet signalling NaNs, an extra instruction per operand the compiler cannot
// prove canonical (matrix-core results).  `pinf` must come from opaque_pinf(): with a
// visible +inf constant the compiler turns the median back into fmaxf.
__device__ __forceinline__ float max_med3(float a, float b, float pinf)
{
    return __builtin_amdgcn_fmed3f(a, b, pinf);
}

__device__ __forceinline__ float opaque_pinf()
{
    float v;
    asm volatile("v_mov_b32 %0, 0x7f800000" : "=v"(v));
    return v;
}

// max_across_rows by the gfx950 lane swaps (v_permlane32_swap, v_permlane16_swap) instead of
// two LDS permutes: swapping a copy of v with itself puts the value of lane l ^ 32 (then
// l ^ 16) beside lane l's own, so two medians give every lane the maximum of its four rows.
__device__ __forceinline__ float max_across_rows_swap(float v, float pinf)
{
    const uint32_t u = __float_as_uint(v);
    const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const float m = max_med3(__uint_as_float(p[0]), __uint_as_float(p[1]), pinf);
    const uint32_t w = __float_as_uint(m);
    const auto q = __builtin_amdgcn_permlane16_swap(w, w, false, false);
    return max_med3(__uint_as_float(q[0]), __uint_as_float(q[1]), pinf);
}

__device__ __forceinline__ float sum_across_rows(float v)
{
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
}

// Orders the LDS accesses of one wave around a hand-off between its lanes (LDS operations of a
// wave execute in issue order; the fences keep the compiler from moving accesses across).
__device__ __forceinline__ void wave_lds_handoff()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Inclusive prefix sum of an int across a 64-lane wave.
__device__ __forceinline__ int wave_inclusive_scan(int v)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int n = __shfl_up(v, o);
        if (lane >= o)
            v += n;
    }
    return v;
}

// Exclusive prefix sum over a workgroup of NT threads; returns the prefix of
// this thread and writes the workgroup total.  `scratch` holds NT/64 ints.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int *scratch, int &total)
{
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int inc = wave_inclusive_scan(v);
    if (lane == 63)
        scratch[w] = inc;
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        int s = scratch[i];
        before += (i < w) ? s : 0;
        tot += s;
    }
    __syncthreads();
    total = tot;
    return before + inc - v;
}

// ---- OCP E4M3 (8-bit float: sign, 4 exponent bits with bias 7, 3 fraction bits) ----
// Four e4m3 codes (bytes of c, low byte first) -> four bf16 (two per word, low half first).
// Every e4m3 value is a bf16 value, so taking the top half of the fp32 conversion is exact.
__device__ __forceinline__ void e4m3x4_to_bf16(uint32_t c, uint32_t &w0, uint32_t &w1)
{
    const auto a = __builtin_amdgcn_cvt_pk_f32_fp8((int)c, false);  // bytes 0, 1
    const auto b = __builtin_amdgcn_cvt_pk_f32_fp8((int)c, true);   // bytes 2, 3
    w0 = (__float_as_uint(a[0]) >> 16) | (__float_as_uint(a[1]) & 0xffff0000u);
    w1 = (__float_as_uint(b[0]) >> 16) | (__float_as_uint(b[1]) & 0xffff0000u);
}

// Sixteen e4m3 codes -> two MFMA fragments of eight bf16 (codes 0-7, then 8-15).
__device__ __forceinline__ void e4m3x16_to_bf16x8x2(const u32x4 &c, bf16x8 &lo, bf16x8 &hi)
{
    uint32_t w[8];
    e4m3x4_to_bf16(c[0], w[0], w[1]);
    e4m3x4_to_bf16(c[1], w[2], w[3]);
    e4m3x4_to_bf16(c[2], w[4], w[5]);
    e4m3x4_to_bf16(c[3], w[6], w[7]);
    lo = as_bf16x8(u32x4{w[0], w[1], w[2], w[3]});
    hi = as_bf16x8(u32x4{w[4], w[5], w[6], w[7]});
}

// Nearest e4m3 code of y, ties to the even code, magnitudes >= 448 saturating to 448.
// In units of the spacing 2^(E-3) of y's binade (2^-9 below 2^-6) the value rounds to an
// integer r in [0, 16]; r = 16 is the next binade's first value.
__device__ __forceinline__ uint32_t e4m3_encode(float y)
{
    const uint32_t sgn = (__float_as_uint(y) >> 24) & 0x80u;
    const float a = fabsf(y);
    if (a >= 448.0f)
        return sgn | 0x7Eu;
    int E = (int)((__float_as_uint(a) >> 23) & 0xffu) - 127;
    if (E < -6)
        E = -6;
    const float r = rintf(ldexpf(a, 3 - E));
    if (r == 0.0f)
        return sgn;
    if (E == -6 && r < 8.0f)
        return sgn | (uint32_t)r;
    int Ev = E, mant = (int)r - 8;
    if (r == 16.0f) {
        Ev = E + 1;
        mant = 0;
    }
    return sgn | (uint32_t)(((Ev + 7) << 3) | mant);
}

} // namespace sgqa
