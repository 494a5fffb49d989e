// MFMA helpers for the 16-bit / 8-bit pool kernels (gfx950).
//
// Operand layout of v_mfma_f32_16x16x32_bf16 (lane l = 16 g + j, g = l / 16):
//   A (16 x 32): lane holds A[j][8 g + t], t = 0..7
//   B (32 x 16): lane holds B[8 g + t][j]
//   C (16 x 16): lane holds C[4 g + i][j], i = 0..3
// ds_read_tr16_b64: in each 16-lane group, lane j pointing at row 4 g' + j/4,
// column c0 + 4 (j % 4) of a row-major 16-bit tile receives the four elements
// of column c0 + j in rows 4 g' .. 4 g' + 3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"

namespace nbx {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// Raw buffer access (gfx9 buffer descriptors): base address and byte range in
// scalar registers, per-lane 32-bit offsets.  A lane whose access falls
// outside the range reads zeros and touches no memory.
__device__ u32x4 nbx_buffer_load_b128(i32x4 rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.v4i32");
__device__ u32x2 nbx_buffer_load_b64(i32x4 rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.v2i32");
__device__ int nbx_buffer_load_b32(i32x4 rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.i32");

// Cache policy of the K/V tile loads (the aux operand of the buffer loads;
// bit 1 is gfx950's nt): each K/V byte is read once per launch, so the loads
// are marked non-temporal and the lines are not kept in the L2 or the
// last-level cache for reuse.
constexpr int kStreamAux = 2;

// Descriptor for `bytes` bytes from `base` (uniform values; forced to SGPRs).
__device__ __forceinline__ i32x4 make_buffer_rsrc(const void *base, uint32_t bytes)
{
    const uint64_t a = (uint64_t)base;
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xFFFFu));
    r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
    r[3] = 0x00020000;
    return r;
}

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Instruction order for a block of `reads` LDS operand reads feeding `reads /
// per_read` groups of `mfma_per` products (group k using the reads k * per_read
// .. k * per_read + per_read - 1): the first `ahead` groups' reads, then for
// each further group one group of products and the next group's reads, then
// the last products.  Each product then finds its operand read `ahead` groups
// earlier, where the default schedule issued most reads just before their
// product and waited on each.  Placed after the reads and products it orders,
// in the same basic block; `id` keeps separate blocks apart.  (Masks of the
// scheduling builtin: 0x100 LDS read, 0x008 MFMA.)
template <int GROUPS, int PER_READ, int MFMA_PER, int AHEAD, int ID>
__device__ __forceinline__ void schedule_reads_ahead()
{
    constexpr int A = AHEAD < GROUPS ? AHEAD : GROUPS;
    __builtin_amdgcn_sched_group_barrier(0x100, A * PER_READ, ID);
#pragma unroll
    for (int i = 0; i < GROUPS - A; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, MFMA_PER, ID);
        __builtin_amdgcn_sched_group_barrier(0x100, PER_READ, ID);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, A * MFMA_PER, ID);
}

// 8 E4M3FN codes (two dwords) widened to 8 bf16 (four dwords), exactly: every
// E4M3FN value (subnormals included) is a bf16 value, so the hardware
// conversion with scale 1 is exact; NaN codes give NaN.  Byte 2 k + h of a
// dword lands in half h of result dword 2 k (bytes 0, 1) or 2 k + 1 (bytes 2, 3).
__device__ __forceinline__ u32x4 widen8_e4m3(u32x2 w)
{
    u32x4 r;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        r[2 * k] =
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[k], 1.0f, false));
        r[2 * k + 1] =
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[k], 1.0f, true));
    }
    return r;
}

// 8 consecutive pool elements as loaded (8 bf16 or 8 E4M3FN codes) and their
// bf16 form
template <int KVT>
struct KvRaw {
    using type = u32x4;
};
template <>
struct KvRaw<NBX_FP8_E4M3> {
    using type = u32x2;
};

template <int KVT>
__device__ __forceinline__ typename KvRaw<KVT>::type buffer_load8_raw(i32x4 rsrc, int voff)
{
    if constexpr (KVT == NBX_BF16)
        return nbx_buffer_load_b128(rsrc, voff, 0, kStreamAux);
    else
        return nbx_buffer_load_b64(rsrc, voff, 0, kStreamAux);
}

template <int KVT>
__device__ __forceinline__ u32x4 as_bf16x8(typename KvRaw<KVT>::type r)
{
    if constexpr (KVT == NBX_BF16)
        return r;
    else
        return widen8_e4m3(r);
}

// two floats rounded to bf16 (to nearest even), lo in the low half: one
// v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi)
{
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// {hi, lo} parts of a pair for the split P = hi + lo: lo holds the pair minus
// its bf16 rounding (the rounded values are the bits of hi)
__device__ __forceinline__ u32x2 pack_bf16_split(float x0, float x1)
{
    const uint32_t hi = pack_bf16(x0, x1);
    return u32x2{hi, pack_bf16(x0 - __uint_as_float(hi << 16), x1 - __uint_as_float(hi & 0xFFFF0000u))};
}

__device__ __forceinline__ float fast_exp2(float x)
{
    return __builtin_amdgcn_exp2f(x);
}

// Maximum / sum over the four lanes j, j + 16, j + 32, j + 48 (the four
// lanes holding one row of a 16 x 16 MFMA result), with the gfx950 lane swaps:
// v_permlane16_swap hands each lane its own value and the one 16 lanes away
// (lanes 0-15 <-> 16-31, 32-47 <-> 48-63), v_permlane32_swap its own and the
// one 32 lanes away, on the vector ALU rather than through LDS as a shuffle
// would.  Both operands of each step are the same pair of values in some order,
// and max and + are commutative, so the result is that of the xor-16 / xor-32
// butterfly bit for bit.  All 64 lanes must be active.
__device__ __forceinline__ float pair16_max(float v)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair32_max(float v)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair16_sum(float v)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float pair32_sum(float v)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float xor_max16_32(float v)
{
    return pair32_max(pair16_max(v));
}

__device__ __forceinline__ float xor_sum16_32(float v)
{
    return pair32_sum(pair16_sum(v));
}

// Hardware workgroup id -> logical id such that each of the 8 XCDs (which
// receive workgroups round-robin) gets one contiguous range of logical ids.
__device__ __forceinline__ uint32_t xcd_contiguous_id(uint32_t hw, uint32_t n)
{
    const uint32_t per = n / 8, rem = n % 8;
    const uint32_t xcd = hw % 8, slot = hw / 8;
    return xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
}

}  // namespace nbx
