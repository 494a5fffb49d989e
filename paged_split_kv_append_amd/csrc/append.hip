// Paged KV append: new positions written into the K and V pools through the
// slot mapping (nbxtensor paged_decode_attn.py, paged_kv_append_kernel: one
// slot per new token, slot = page * page_tokens + row, the values cast to the
// pool's dtype on store).
//
// Tail mode (no slot mapping): the n_new new tokens of sequence b go to its
// last n_new positions, the slot of each read from the block table.
//
// One thread moves 8 consecutive elements of one (token, KV head) row, so a
// row of D elements takes D/8 threads (of a group of 8, 16 or 32 lanes) and
// the K and V pools are written by the same launch (blockIdx.y selects K or
// V; V rows may be narrower).  A pool with bounds gets bounds[page, head]
// raised to the stored row's norm (K) or largest |element| (V).
#include "device_common.h"
#include "kernels.h"

namespace nbx {

template <int SRC>
__device__ __forceinline__ void load8(const void *src, int64_t i, float (&x)[8])
{
    if constexpr (SRC == NBX_F32) {
        const float4 *p = (const float4 *)((const float *)src + i);
        float4 a = p[0], b = p[1];
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    } else {
        uint4 w = *(const uint4 *)((const uint16_t *)src + i);
        uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            x[2 * k] = __uint_as_float(ws[k] << 16);
            x[2 * k + 1] = __uint_as_float(ws[k] & 0xFFFF0000u);
        }
    }
}

// Stores the 8 values x at element i of a DST pool (the conversions of the
// append) and returns in sv what was stored, in stored units.
template <int SRC, int DST>
__device__ __forceinline__ void store8(void *dst, int64_t i, const float (&x)[8], float scale,
                                       const void *src, int64_t si, float (&sv)[8])
{
    if constexpr (DST == NBX_F32) {
        float4 *p = (float4 *)((float *)dst + i);
        p[0] = make_float4(x[0], x[1], x[2], x[3]);
        p[1] = make_float4(x[4], x[5], x[6], x[7]);
#pragma unroll
        for (int k = 0; k < 8; ++k)
            sv[k] = x[k];
    } else if constexpr (DST == NBX_BF16) {
        if constexpr (SRC == NBX_BF16) {
            // same dtype: bit copy (x holds the same values exactly)
            *(uint4 *)((uint16_t *)dst + i) = *(const uint4 *)((const uint16_t *)src + si);
#pragma unroll
            for (int k = 0; k < 8; ++k)
                sv[k] = x[k];
        } else {
            uint32_t w[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t lo = f32_to_bf16_bits(x[2 * k]), hi = f32_to_bf16_bits(x[2 * k + 1]);
                w[k] = lo | (hi << 16);
                sv[2 * k] = bf16_bits_to_f32(lo);
                sv[2 * k + 1] = bf16_bits_to_f32(hi);
            }
            *(uint4 *)((uint16_t *)dst + i) = make_uint4(w[0], w[1], w[2], w[3]);
        }
    } else {
        // fp8: code of the correctly rounded fp32 quotient x / scale
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t a = f32_to_e4m3(__fdiv_rn(x[k], scale));
            const uint32_t b = f32_to_e4m3(__fdiv_rn(x[k + 4], scale));
            lo |= a << (8 * k);
            hi |= b << (8 * k);
            sv[k] = e4m3_to_f32(a);
            sv[k + 4] = e4m3_to_f32(b);
        }
        *(uint2 *)((uint8_t *)dst + i) = make_uint2(lo, hi);
    }
}

// 8-element pieces of a row are handled by a power-of-two group of lanes (8,
// 16 or 32), so that the lanes of one row share a wave for the bound's
// reduction
__host__ __device__ __forceinline__ int lanes_per_row(int pieces)
{
    return pieces <= 8 ? 8 : pieces <= 16 ? 16 : 32;
}

template <int SRC, int DST>
__global__ void __launch_bounds__(256)
paged_append_kernel(AppendArgs a)
{
    const bool is_v = blockIdx.y == 1;
    const int pieces = (is_v ? a.v_head_dim : a.head_dim) / 8;
    const int lpr = lanes_per_row(pieces);
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = a.n_tok * a.kv_heads * lpr;
    const void *src = is_v ? a.new_v : a.new_k;
    void *pool = is_v ? a.v_data : a.k_data;
    float *bounds = is_v ? a.v_bounds : a.k_bounds;
    const int64_t sp = is_v ? a.v_stride_page : a.k_stride_page;
    const int64_t sh = is_v ? a.v_stride_head : a.k_stride_head;
    const int64_t st = is_v ? a.v_stride_token : a.k_stride_token;
    const float scale = is_v ? a.v_scale : a.k_scale;

    const int64_t c = gid % lpr;
    const int64_t h = (gid / lpr) % a.kv_heads;
    const int64_t t = gid / (lpr * a.kv_heads);
    const bool lead = c == 0 && h == 0 && !is_v;
    // every lane stays to the end: the bound is reduced over the row's lanes
    bool row_ok = gid < total;
    int64_t slot = -1;
    if (row_ok) {
        if (a.slot_mapping) {
            slot = a.slot_mapping[t];
        } else {
            // tail mode: the slot of position L_b - n_new + i from the block table
            const int64_t b = t / a.n_new, i = t - b * a.n_new;
            const int64_t L = a.seq_lens[b];
            const int64_t pos = L - a.n_new + i;
            if (pos < 0 || L > (int64_t)a.max_pages * a.page_tokens) {
                if (lead)
                    flag_error(a.dev_err, NBX_DEVERR_SEQ_RANGE);
                row_ok = false;
            } else {
                const int32_t page = a.block_table[b * a.max_pages + pos / a.page_tokens];
                if (page < 0 || page >= a.num_pages) {
                    if (lead)
                        flag_error(a.dev_err, NBX_DEVERR_PAGE_RANGE);
                    row_ok = false;
                } else {
                    slot = (int64_t)page * a.page_tokens + pos % a.page_tokens;
                }
            }
        }
        if (row_ok && slot < 0)
            row_ok = false;                                // padding token
        if (row_ok && slot >= (int64_t)a.num_pages * a.page_tokens) {
            if (lead)
                flag_error(a.dev_err, NBX_DEVERR_SLOT_RANGE);
            row_ok = false;
        }
    }
    const int64_t page = row_ok ? slot / a.page_tokens : 0;
    float stat = 0.0f;             // K: sum of squares of the stored piece; V: largest |.|
    if (row_ok && c < pieces) {
        const int64_t row = slot - page * a.page_tokens;
        const int64_t si = t * (is_v ? a.v_new_stride_tok : a.new_stride_tok) +
                           h * (is_v ? a.v_new_stride_head : a.new_stride_head) + c * 8;
        const int64_t di = page * sp + h * sh + row * st + c * 8;
        float x[8], sv[8];
        load8<SRC>(src, si, x);
        store8<SRC, DST>(pool, di, x, scale, src, si, sv);
#pragma unroll
        for (int k = 0; k < 8; ++k)
            stat = is_v ? bound_max(stat, fabsf(sv[k])) : fmaf(sv[k], sv[k], stat);
    }
    if (bounds) {                  // uniform: one pool per launch row
        if (lpr == 8)
            stat = is_v ? group_bound_max<8>(stat) : group_sum<8>(stat);
        else if (lpr == 16)
            stat = is_v ? group_bound_max<16>(stat) : group_sum<16>(stat);
        else
            stat = is_v ? group_bound_max<32>(stat) : group_sum<32>(stat);
        if (row_ok && c == 0)
            raise_bound(bounds, page * a.kv_heads + h, is_v ? stat : sqrtf(stat));
    }
}

template <int SRC, int DST>
static hipError_t launch_append_t(const AppendArgs &a, hipStream_t stream)
{
    const int32_t widest = a.new_v && a.v_head_dim > a.head_dim ? a.v_head_dim : a.head_dim;
    const int64_t total = a.n_tok * a.kv_heads * lanes_per_row(widest / 8);
    if (!grid_fits((total + 255) / 256, 256))
        return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)((total + 255) / 256), a.new_v ? 2 : 1);
    hipLaunchKernelGGL((paged_append_kernel<SRC, DST>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------- bounds

__global__ void __launch_bounds__(256)
fill_zero_kernel(float *p, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        p[i] = 0.0f;
}

template <int DT>
__device__ __forceinline__ void load8_stored(const void *base, int64_t i, float (&x)[8])
{
    if constexpr (DT == NBX_FP8_E4M3) {
        const uint2 w = *(const uint2 *)((const uint8_t *)base + i);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            x[k] = e4m3_to_f32((w.x >> (8 * k)) & 0xFFu);
            x[k + 4] = e4m3_to_f32((w.y >> (8 * k)) & 0xFFu);
        }
    } else {
        load8<DT>(base, i, x);
    }
}

// Bounds of one pool over the rows the sequences hold: blockIdx.z = sequence,
// blockIdx.y = page of the sequence, x = (KV head, row of the page, piece)
// with a power-of-two lane group per row.
template <int DT>
__global__ void __launch_bounds__(256)
kv_bounds_kernel(BoundsArgs a, int is_v)
{
    const int D = is_v ? a.v_head_dim : a.head_dim;
    const int pieces = D / 8, lpr = lanes_per_row(pieces);
    const int T = a.page_tokens, H = a.kv_heads;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t total = (int64_t)H * T * lpr;
    const int b = blockIdx.z, pi = blockIdx.y;
    const int c = (int)(gid % lpr), r = (int)((gid / lpr) % T), h = (int)(gid / ((int64_t)lpr * T));
    const bool first = gid == 0 && pi == 0 && !is_v;
    int64_t L = a.seq_lens[b];
    const int64_t cap = (int64_t)a.max_pages * T;
    if (L < 0 || L > cap) {
        if (first)
            flag_error(a.dev_err, NBX_DEVERR_SEQ_RANGE);
        L = L < 0 ? 0 : cap;
    }
    const int64_t j = (int64_t)pi * T + r;
    bool ok = gid < total && j < L;
    int64_t page = 0;
    if (ok) {
        page = a.block_table[(int64_t)b * a.max_pages + pi];
        if (page < 0 || page >= a.num_pages) {
            if (!is_v && r == 0 && h == 0 && c == 0)
                flag_error(a.dev_err, NBX_DEVERR_PAGE_RANGE);
            ok = false;
        }
    }
    float stat = 0.0f;
    if (ok && c < pieces) {
        const void *base = is_v ? a.v_data : a.k_data;
        const int64_t i = is_v ? page * a.v_stride_page + h * a.v_stride_head + r * a.v_stride_token
                               : page * a.k_stride_page + h * a.k_stride_head + r * a.k_stride_token;
        float x[8];
        load8_stored<DT>(base, i + c * 8, x);
#pragma unroll
        for (int k = 0; k < 8; ++k)
            stat = is_v ? bound_max(stat, fabsf(x[k])) : fmaf(x[k], x[k], stat);
    }
    if (lpr == 8)
        stat = is_v ? group_bound_max<8>(stat) : group_sum<8>(stat);
    else if (lpr == 16)
        stat = is_v ? group_bound_max<16>(stat) : group_sum<16>(stat);
    else
        stat = is_v ? group_bound_max<32>(stat) : group_sum<32>(stat);
    if (ok && c == 0)
        raise_bound(is_v ? a.v_bounds : a.k_bounds, page * H + h, is_v ? stat : sqrtf(stat));
}

hipError_t launch_kv_bounds(const BoundsArgs &a, hipStream_t stream)
{
    const int64_t n = (int64_t)a.num_pages * a.kv_heads;
    for (int is_v = 0; is_v < 2; ++is_v) {
        const int D = is_v ? a.v_head_dim : a.head_dim;
        if (!grid_fits(((int64_t)a.kv_heads * a.page_tokens * lanes_per_row(D / 8) + 255) / 256, 256))
            return hipErrorInvalidConfiguration;
    }
    const unsigned zb = (unsigned)((n + 255) / 256 < 65535 ? (n + 255) / 256 : 65535);
    hipLaunchKernelGGL(fill_zero_kernel, dim3(zb), dim3(256), 0, stream, a.k_bounds, n);
    hipLaunchKernelGGL(fill_zero_kernel, dim3(zb), dim3(256), 0, stream, a.v_bounds, n);
    if (a.batch > 0) {
        for (int is_v = 0; is_v < 2; ++is_v) {
            const int D = is_v ? a.v_head_dim : a.head_dim;
            const int64_t per_page = (int64_t)a.kv_heads * a.page_tokens * lanes_per_row(D / 8);
            dim3 grid((unsigned)((per_page + 255) / 256), (unsigned)a.max_pages, (unsigned)a.batch);
            if (a.dtype == NBX_F32)
                hipLaunchKernelGGL(kv_bounds_kernel<NBX_F32>, grid, dim3(256), 0, stream, a, is_v);
            else if (a.dtype == NBX_BF16)
                hipLaunchKernelGGL(kv_bounds_kernel<NBX_BF16>, grid, dim3(256), 0, stream, a, is_v);
            else
                hipLaunchKernelGGL(kv_bounds_kernel<NBX_FP8_E4M3>, grid, dim3(256), 0, stream, a,
                                   is_v);
        }
    }
    return hipGetLastError();
}

// seq_lens[b] += n for every sequence (nbxtensor paged_decode_attn.py,
// paged_lens_advance_kernel: the length moves on the device after the step's
// append, so a recorded step replays with the same arguments)
__global__ void __launch_bounds__(256)
lens_advance_kernel(int32_t *seq_lens, int32_t batch, int32_t n)
{
    const int b = blockIdx.x * 256 + threadIdx.x;
    if (b < batch)
        seq_lens[b] += n;
}

hipError_t launch_lens_advance(int32_t *seq_lens, int32_t batch, int32_t n, hipStream_t stream)
{
    if (batch <= 0)
        return hipSuccess;
    hipLaunchKernelGGL(lens_advance_kernel, dim3((unsigned)((batch + 255) / 256)), dim3(256), 0,
                       stream, seq_lens, batch, n);
    return hipGetLastError();
}

hipError_t launch_append(const AppendArgs &a, hipStream_t stream)
{
    if (a.src_dtype == NBX_F32) {
        if (a.dst_dtype == NBX_F32) return launch_append_t<NBX_F32, NBX_F32>(a, stream);
        if (a.dst_dtype == NBX_BF16) return launch_append_t<NBX_F32, NBX_BF16>(a, stream);
        return launch_append_t<NBX_F32, NBX_FP8_E4M3>(a, stream);
    }
    if (a.dst_dtype == NBX_F32) return launch_append_t<NBX_BF16, NBX_F32>(a, stream);
    if (a.dst_dtype == NBX_BF16) return launch_append_t<NBX_BF16, NBX_BF16>(a, stream);
    return launch_append_t<NBX_BF16, NBX_FP8_E4M3>(a, stream);
}

}  // namespace nbx
