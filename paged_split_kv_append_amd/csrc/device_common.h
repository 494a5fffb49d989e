// Device-side helpers shared by the kernels of libnbx_paged (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nbx_paged.h"

namespace nbx {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- conversions

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h)
{
    return __uint_as_float(h << 16);
}

// fp32 -> bf16, round to nearest even; NaN -> quiet NaN with the sign kept.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x)
{
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return (uint16_t)(((u >> 16) & 0x8000u) | 0x7FC0u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// OCP E4M3FN code -> fp32 (exact).  Exponent field e (bias 7), mantissa m:
// e > 0 gives 2^(e-7) * (1 + m/8), built directly as an fp32 bit pattern;
// e == 0 gives m * 2^-9; 0x7F / 0xFF are NaN.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c)
{
    uint32_t em = c & 0x7Fu;
    uint32_t e = em >> 3;
    float v = e ? __uint_as_float(((e + 120u) << 23) | ((em & 7u) << 20))
                : (float)(em & 7u) * 0x1p-9f;
    v = (em == 0x7Fu) ? __builtin_nanf("") : v;
    return (c & 0x80u) ? -v : v;
}

// fp32 -> OCP E4M3FN code, round to nearest even, saturating at +-448,
// NaN -> 0x7F with the sign kept.  Works on the fp32 bit pattern: the value is
// rounded to 3 mantissa bits at its own binade (normal range, exponent >= -6)
// or to a multiple of 2^-9 (subnormal range).
__device__ __forceinline__ uint8_t f32_to_e4m3(float x)
{
    uint32_t u = __float_as_uint(x);
    uint32_t sign = (u >> 24) & 0x80u;
    uint32_t a = u & 0x7FFFFFFFu;
    if (a > 0x7F800000u)
        return (uint8_t)(sign | 0x7Fu);
    if (a >= 0x43E00000u)                      // |x| >= 448 (inf included)
        return (uint8_t)(sign | 0x7Eu);
    int exp = (int)(a >> 23) - 127;            // unbiased fp32 exponent
    uint32_t code;
    if (exp >= -6) {
        // keep 3 mantissa bits: drop 20, round half to even on the dropped part
        uint32_t mant = a & 0x7FFFFFu;
        uint32_t keep = mant >> 20, rest = mant & 0xFFFFFu;
        uint32_t up = (rest > 0x80000u) || (rest == 0x80000u && (keep & 1u));
        code = ((uint32_t)(exp + 7) << 3) + keep + up;   // carry rolls into the exponent
        if (code > 0x7Eu)
            code = 0x7Eu;
    } else {
        // subnormal target: q = round_half_even(|x| * 2^9), exact scaling by 2^9
        float s = __uint_as_float(a) * 512.0f;
        code = (uint32_t)__builtin_rintf(s);  // default rounding mode: nearest even
    }
    return (uint8_t)(sign | code);
}

template <int DT>
__device__ __forceinline__ float load_elem(const void *base, int64_t i);

template <>
__device__ __forceinline__ float load_elem<NBX_F32>(const void *base, int64_t i)
{
    return ((const float *)base)[i];
}
template <>
__device__ __forceinline__ float load_elem<NBX_BF16>(const void *base, int64_t i)
{
    return bf16_bits_to_f32(((const uint16_t *)base)[i]);
}
template <>
__device__ __forceinline__ float load_elem<NBX_FP8_E4M3>(const void *base, int64_t i)
{
    return e4m3_to_f32(((const uint8_t *)base)[i]);
}

// ---------------------------------------------------------------- wave reductions

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v += __shfl_xor(v, off, 64);
    return v;
}

// ---------------------------------------------------------------- pool bounds
//
// Bounds are non-negative floats or NaN ("unknown").  With the sign bit
// cleared, the bit patterns of non-negative floats order like their values and
// every NaN lies above +inf, so an unsigned maximum of the patterns keeps a
// NaN sticky.

__device__ __forceinline__ uint32_t bound_bits(float v) { return __float_as_uint(v) & 0x7FFFFFFFu; }

// raise bounds[i] to v
__device__ __forceinline__ void raise_bound(float *bounds, int64_t i, float v)
{
    atomicMax((unsigned int *)(bounds + i), bound_bits(v));
}

// NaN-sticky maximum of non-negative floats
__device__ __forceinline__ float bound_max(float a, float b)
{
    return __uint_as_float(max(bound_bits(a), bound_bits(b)));
}

// sum / NaN-sticky maximum over aligned groups of N lanes (N a power of two <= 64)
template <int N>
__device__ __forceinline__ float group_sum(float v)
{
#pragma unroll
    for (int off = N / 2; off >= 1; off >>= 1)
        v += __shfl_xor(v, off, 64);
    return v;
}

template <int N>
__device__ __forceinline__ float group_bound_max(float v)
{
#pragma unroll
    for (int off = N / 2; off >= 1; off >>= 1)
        v = bound_max(v, __shfl_xor(v, off, 64));
    return v;
}

__device__ __forceinline__ void flag_error(int32_t *dev_err, int32_t bit)
{
    if (dev_err)
        atomicOr(dev_err, bit);
}

}  // namespace nbx
