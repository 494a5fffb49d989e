// Device helpers shared by the split-partial kernels on the matrix cores
// (the decode kernels of partial_mfma.hip and the multi-row kernel of
// partial_multirow.hip): sequence length and page lookups, the transposed
// read of a V operand from LDS, the online-softmax step and the fixed-shift
// softmax.
#pragma once

#include "kernels.h"
#include "mfma_common.h"

namespace nbx {

// A value every lane of the wave holds alike, moved to a scalar register.
__device__ __forceinline__ float wave_uniform(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

__device__ __forceinline__ int clamp_len(const PartialArgs &a, int b, bool flag_it)
{
    int L = a.seq_lens[b];
    const int cap = a.max_pages * a.page_tokens;
    if (L < 0 || L > cap) {
        if (flag_it)
            flag_error(a.dev_err, NBX_DEVERR_SEQ_RANGE);
        L = L < 0 ? 0 : cap;
    }
    return L;
}

// Page of the 16-position tile starting at position ts of sequence b, or -1
// if the tile is past `end` or the block table does not map it into the pool.
__device__ __forceinline__ int tile_page(const PartialArgs &a, int b, int ts, int end,
                                         bool flag_it)
{
    if (ts >= end)
        return -1;
    const int page = a.block_table[(int64_t)b * a.max_pages + ts / a.page_tokens];
    if (page < 0 || page >= a.num_pages) {
        if (flag_it)
            flag_error(a.dev_err, NBX_DEVERR_PAGE_RANGE);
        return -1;
    }
    return page;
}

// Buffer descriptor of tile rows [0, rows) starting at position ts in `page`
// (rows <= 0 or an unmapped page gives an empty range).
template <int ESZ>
__device__ __forceinline__ i32x4 tile_rsrc(const void *data, int64_t stride_page,
                                           int64_t head_off, int64_t stride_token, int page_tokens,
                                           int page, int ts, int rows)
{
    const int pg = page >= 0 ? page : 0;
    const int64_t off = (int64_t)(ts % page_tokens);
    const uint8_t *base =
        (const uint8_t *)data + ((int64_t)pg * stride_page + head_off + off * stride_token) * ESZ;
    const uint32_t bytes = page >= 0 && rows > 0 ? (uint32_t)(rows * stride_token * ESZ) : 0u;
    return make_buffer_rsrc(base, bytes);
}

// One new K or V row (D elements at src of a [.., D] array of src_dtype)
// stored at element offset dst of a bf16 or fp8 pool, with the append's
// conversions: bf16 -> bf16 bit copy, fp32 -> bf16 round to nearest even, to
// fp8 the correctly rounded quotient value / scale, rounded to nearest even
// and saturated.  Lane l stores elements l * D/64 .. (l + 1) * D/64 - 1.
// Returns the lane's share of the stored row's bound statistic (stored
// units): the sum of squares (K) or the largest magnitude (V).
template <int D, int KVT, bool V>
__device__ __forceinline__ float store_new_row(const void *src_base, int src_dtype, int64_t src,
                                               void *pool, int64_t dst, float scale, int lane)
{
    constexpr int E = D / 64;
    float stat = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int64_t i = lane * E + e;
        float stored;
        if constexpr (KVT == NBX_BF16) {
            const uint16_t bits = src_dtype == NBX_BF16
                                      ? ((const uint16_t *)src_base)[src + i]
                                      : f32_to_bf16_bits(((const float *)src_base)[src + i]);
            ((uint16_t *)pool)[dst + i] = bits;
            stored = bf16_bits_to_f32(bits);
        } else {
            const float x = src_dtype == NBX_BF16
                                ? bf16_bits_to_f32(((const uint16_t *)src_base)[src + i])
                                : ((const float *)src_base)[src + i];
            const uint8_t code = f32_to_e4m3(__fdiv_rn(x, scale));
            ((uint8_t *)pool)[dst + i] = code;
            stored = e4m3_to_f32(code);
        }
        stat = V ? bound_max(stat, fabsf(stored)) : fmaf(stored, stored, stat);
    }
    return stat;
}

// Whole-row loads of a 16-row bf16 tile of DW columns: load i of a wave
// (64 lanes x 16 bytes) takes the 16-byte units 64 i .. 64 i + 63 of the tile
// in row-major order, i.e. whole rows (4 of 256 bytes at DW = 128), so every
// load fetches complete 128-byte lines.  In LDS the tile is row-major with
// unit u of row r stored at unit (u + rot r) mod U of that row (U units per
// row, rot = 2 for U >= 16, else 1): the 16 lanes landing one row write 16
// different units, the 8 lanes of a K operand read (8 rows, one unit each)
// fall on different banks, and so do the 4-row pieces of a transposed V read.
template <int DW>
struct RowTile {
    static constexpr int U = DW / 8;           // 16-byte units per row
    static constexpr int ROT = U >= 16 ? 2 : 1;
    static constexpr int ROWB = DW * 2;        // bytes per row in LDS
    int lane, stride_b;                        // row stride of the pool in bytes
    __device__ RowTile(int lane_, int stride_b_) : lane(lane_), stride_b(stride_b_) {}
    // LDS offset of unit u of row r
    __device__ static int at(int r, int u) { return r * ROWB + ((u + ROT * r) % U) * 16; }
    // byte offset in the pool of this lane's piece of load i
    __device__ int global(int i) const
    {
        const int x = 64 * i + lane;
        return (x / U) * stride_b + (x % U) * 16;
    }
    // LDS offset of the same piece
    __device__ int lds(int i) const
    {
        const int x = 64 * i + lane;
        return at(x / U, x % U);
    }
    // A operand of S^T = K Q^T (lane 16 g + j: row j, unit u = 4 kk + g)
    __device__ int operand(int r, int u) const { return at(r, u); }
    // A operand of O^T += V^T P^T for 16-column slice dt from the two tiles
    // of a chunk (the second `half` bytes after the first): lane 16 g + j
    // reads row 4 g + j / 4, columns 16 dt + 4 (j % 4) .. + 3 of each, and the
    // transposing read hands it column 16 dt + j of rows 4 g .. 4 g + 3
    __device__ u32x4 transposed(const uint8_t *tile, int half, int g, int j, int dt) const
    {
        const uint8_t *p0 = tile + at(4 * g + (j >> 2), 2 * dt + ((j & 3) >> 1)) + (j & 1) * 8;
        const uint8_t *p1 = p0 + half;
        const bf16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_bf16x4 *)(__attribute__((address_space(3))) uint8_t *)p0);
        const bf16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_bf16x4 *)(__attribute__((address_space(3))) uint8_t *)p1);
        const u32x2 ux = __builtin_bit_cast(u32x2, x), uy = __builtin_bit_cast(u32x2, y);
        return u32x4{ux[0], ux[1], uy[0], uy[1]};
    }
};

// A operand of the P V product for 16-column slice dt from a column-blocked
// chunk tile (tile 0 blocks, then tile 1 blocks); `lane_base` is the lane's
// fixed address: block 0 of tile 0 + (4 g + j/4) * 32 + (j % 4) * 8.
template <int DT>
__device__ __forceinline__ u32x4 vt_operand(const uint8_t *lane_base, int dt)
{
    const uint8_t *p0 = lane_base + dt * 512;
    const uint8_t *p1 = p0 + DT * 512;
    const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4 *)(__attribute__((address_space(3))) uint8_t *)p0);
    const bf16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4 *)(__attribute__((address_space(3))) uint8_t *)p1);
    const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
    return u32x4{ua[0], ua[1], ub[0], ub[1]};
}

// Online-softmax step for one lane's row over NK k-steps of 32 positions (two
// 16-position tiles each): sc holds the scaled scores (log2 units, -inf where
// masked).  Updates m and l, returns the P operands of the k-steps (hi and
// residual lo parts) and the factor exp(m_old - m_new) by which the row's
// accumulator must be scaled before this step's P V is added.
template <bool PVS, int NK>
__device__ __forceinline__ float softmax_corr_n(float (&sc)[2 * NK][4], float &m_run, float &l_run,
                                                u32x4 (&ph)[NK], u32x4 (&pl)[NK])
{
    float mx = sc[0][0];
#pragma unroll
    for (int t = 0; t < 2 * NK; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            mx = fmaxf(mx, sc[t][i]);
    mx = xor_max16_32(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_safe = m_new == -INFINITY ? 0.0f : m_new;
    const float corr = fast_exp2(m_run - m_safe);
    float p[2 * NK][4], psum = 0.0f;
#pragma unroll
    for (int t = 0; t < 2 * NK; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p[t][i] = fast_exp2(sc[t][i] - m_safe);
            psum += p[t][i];
        }
    l_run = l_run * corr + psum;
    m_run = m_new;
#pragma unroll
    for (int k = 0; k < NK; ++k)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int t = 2 * k + u;
            if constexpr (PVS) {
                const u32x2 a = pack_bf16_split(p[t][0], p[t][1]);
                const u32x2 c = pack_bf16_split(p[t][2], p[t][3]);
                ph[k][2 * u] = a[0];
                pl[k][2 * u] = a[1];
                ph[k][2 * u + 1] = c[0];
                pl[k][2 * u + 1] = c[1];
            } else {
                ph[k][2 * u] = pack_bf16(p[t][0], p[t][1]);
                ph[k][2 * u + 1] = pack_bf16(p[t][2], p[t][3]);
            }
        }
    return corr;
}

// The same step with the row's accumulator o in this lane: it is rescaled when
// some row's running max moved (else every factor is 1 and o * 1 = o).
template <int DT, bool PVS, int NK>
__device__ __forceinline__ void softmax_step_n(float (&sc)[2 * NK][4], float &m_run, float &l_run,
                                               f32x4 (&o)[DT], u32x4 (&ph)[NK], u32x4 (&pl)[NK])
{
    const float corr = softmax_corr_n<PVS, NK>(sc, m_run, l_run, ph, pl);
    if (__any(corr != 1.0f)) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
            o[dt] *= corr;
    }
}

// Lazy variant for the multi-row kernel: the row's shift m_run moves only when
// the row's running maximum m_top has grown past it by more than kLazyShift
// (log2 units), so p = 2^(s - m_run) stays below 2^kLazyShift and the
// accumulator is rescaled on few chunks instead of on every chunk that raises
// some row's maximum.  lazy_finish puts the partial in the exact-maximum form.
constexpr float kLazyShift = 8.0f;

template <bool PVS, int NK>
__device__ __forceinline__ float softmax_lazy_n(float (&sc)[2 * NK][4], float &m_run, float &m_top,
                                                float &l_run, u32x4 (&ph)[NK], u32x4 (&pl)[NK])
{
    float mx = sc[0][0];
#pragma unroll
    for (int t = 0; t < 2 * NK; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            mx = fmaxf(mx, sc[t][i]);
    m_top = fmaxf(m_top, xor_max16_32(mx));
    // m_run = -inf (no key yet): the difference is +inf and the shift moves;
    // m_top = -inf too: NaN, and it stays
    const float m_new = m_top - m_run > kLazyShift ? m_top : m_run;
    const float m_safe = m_new == -INFINITY ? 0.0f : m_new;
    const float corr = fast_exp2(m_run - m_safe);      // exactly 1 when the shift stays
    float p[2 * NK][4], psum = 0.0f;
#pragma unroll
    for (int t = 0; t < 2 * NK; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p[t][i] = fast_exp2(sc[t][i] - m_safe);
            psum += p[t][i];
        }
    l_run = l_run * corr + psum;
    m_run = m_new;
#pragma unroll
    for (int k = 0; k < NK; ++k)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int t = 2 * k + u;
            if constexpr (PVS) {
                const u32x2 a = pack_bf16_split(p[t][0], p[t][1]);
                const u32x2 c = pack_bf16_split(p[t][2], p[t][3]);
                ph[k][2 * u] = a[0];
                pl[k][2 * u] = a[1];
                ph[k][2 * u + 1] = c[0];
                pl[k][2 * u + 1] = c[1];
            } else {
                ph[k][2 * u] = pack_bf16(p[t][0], p[t][1]);
                ph[k][2 * u + 1] = pack_bf16(p[t][2], p[t][3]);
            }
        }
    return corr;
}

// The lazy form's accumulator and sum rescaled from the shift m_run to the
// row's maximum m_top (m_run <= m_top), so that the stored partial holds
// m = the largest score, as the running-maximum form does.
template <int DT>
__device__ __forceinline__ void lazy_finish(float &m_run, float m_top, float &l_run,
                                            f32x4 (&o)[DT])
{
    const float fin = m_top == -INFINITY ? 1.0f : fast_exp2(m_run - m_top);
    l_run *= fin;
    if (__any(fin != 1.0f)) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
            o[dt] *= fin;
    }
    m_run = m_top;
}

// ------------------------------------------------------------------ fixed shift
//
// The fixed-shift softmax of the maxdiffusion PR #477 page (fixed-m splash
// attention with dynamic bounds), in log2 units: a split whose keys have
// norms <= kb, whose values (in the accumulator's units) are <= Vmax and
// whose sequence holds N keys gets C = 127 - ceil(log2 N) - ceil(log2 Vmax)
// and gate = floor((C + 125) / 2); a query row with norm |q| gets U = |scale|
// |q| kb (an upper bound of every |score|, here enlarged by 2^-12 to cover
// the rounding of the norms and of the fp32 dot product) and the shift
// m = ceil(U) - C.  When ceil(U) <= gate every exponent score - m lies in
// [-125, C]: no term leaves the normal fp32 range and N terms times Vmax
// stay below 2^127, so p = 2^(score - m) is summed with no running maximum
// and no rescaling.  Vmax = max(1, V bound * max(1, v_scale)) covers the
// accumulator both before and after the V scale is applied.

__device__ __forceinline__ int ceil_log2_count(int n)
{
    return n <= 1 ? 0 : 32 - __clz(n - 1);
}

// C and the gate for N keys and a V bound vb (false: the bound is not finite)
__device__ __forceinline__ bool fixed_shift_consts(int n, float vb, float v_scale, int &C,
                                                   int &gate)
{
    float vmax = vb * fmaxf(1.0f, v_scale);
    if (!(vmax <= 3.0e38f))                    // NaN (unknown) or infinite
        return false;
    vmax = fmaxf(vmax, 1.0f);
    int e;
    const float f = frexpf(vmax, &e);          // vmax = f 2^e, f in [0.5, 1)
    C = 127 - ceil_log2_count(n) - (f == 0.5f ? e - 1 : e);
    const int W = C + 125;
    gate = W >= 0 ? W / 2 : -((1 - W) / 2);    // floor(W / 2)
    return true;
}

// The row's shift m (log2 units); true when the row passes the gate
__device__ __forceinline__ bool fixed_shift_row(float q_norm, float kb, float scale_abs, int C,
                                                int gate, float &m)
{
    const float U = scale_abs * q_norm * kb * (1.0f + 0x1p-12f);
    const float cu = ceilf(U);
    m = cu - (float)C;
    return cu <= (float)gate;                  // false for NaN or infinite U
}

// Norm of this lane's query row from its bf16 operand registers (lane
// 16 g + j holds columns 8 g .. 8 g + 7 of every 32-column k-step of row j)
template <int KK>
__device__ __forceinline__ float q_row_norm(const u32x4 (&qb)[KK])
{
    float ss = 0.0f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float lo = __uint_as_float(qb[kk][w] << 16);
            const float hi = __uint_as_float(qb[kk][w] & 0xFFFF0000u);
            ss = fmaf(lo, lo, ss);
            ss = fmaf(hi, hi, ss);
        }
    return sqrtf(xor_sum16_32(ss));
}

// Softmax step with a fixed shift m: p = 2^(s - m), l += sum p, no rescaling
// (the P operands as softmax_step_n forms them)
template <bool PVS, int NK>
__device__ __forceinline__ void softmax_fixed_n(float (&sc)[2 * NK][4], float m, float &l_run,
                                                u32x4 (&ph)[NK], u32x4 (&pl)[NK])
{
    float p[2 * NK][4], psum = 0.0f;
#pragma unroll
    for (int t = 0; t < 2 * NK; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p[t][i] = fast_exp2(sc[t][i] - m);
            psum += p[t][i];
        }
    l_run += psum;
#pragma unroll
    for (int k = 0; k < NK; ++k)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int t = 2 * k + u;
            if constexpr (PVS) {
                const u32x2 a = pack_bf16_split(p[t][0], p[t][1]);
                const u32x2 c = pack_bf16_split(p[t][2], p[t][3]);
                ph[k][2 * u] = a[0];
                pl[k][2 * u] = a[1];
                ph[k][2 * u + 1] = c[0];
                pl[k][2 * u + 1] = c[1];
            } else {
                ph[k][2 * u] = pack_bf16(p[t][0], p[t][1]);
                ph[k][2 * u + 1] = pack_bf16(p[t][2], p[t][3]);
            }
        }
}

// m_part of a row: the fixed shift (no key: -inf) or the running maximum
__device__ __forceinline__ float stored_m(bool fixed, float m_fix, float m_run, float l_total)
{
    if (fixed)
        return l_total > 0.0f ? m_fix * kLn2 : -INFINITY;
    return m_run == -INFINITY ? -INFINITY : m_run * kLn2;
}

}  // namespace nbx
