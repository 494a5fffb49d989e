// Paged KV append: new positions written into the K and V pools through the
// slot mapping (nbxtensor paged_decode_attn.py, paged_kv_append_kernel: one
// slot per new token, slot = page * page_tokens + row, the values cast to the
// pool's dtype on store).
//
// Tail mode (no slot mapping): the n_new new tokens of sequence b go to its
// last n_new positions, the slot of each read from the block table.
//
// One thread moves 8 consecutive elements of one (token, KV head) row, so a
// row of D elements takes D/8 threads and the K and V pools are written by
// the same launch (blockIdx.y selects K or V; V rows may be narrower).
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

template <int SRC, int DST>
__device__ __forceinline__ void store8(void *dst, int64_t i, const float (&x)[8], float inv_scale_div,
                                       const void *src, int64_t si)
{
    if constexpr (DST == NBX_F32) {
        float4 *p = (float4 *)((float *)dst + i);
        p[0] = make_float4(x[0], x[1], x[2], x[3]);
        p[1] = make_float4(x[4], x[5], x[6], x[7]);
    } else if constexpr (DST == NBX_BF16) {
        if constexpr (SRC == NBX_BF16) {
            // same dtype: bit copy
            *(uint4 *)((uint16_t *)dst + i) = *(const uint4 *)((const uint16_t *)src + si);
        } else {
            uint32_t w[4];
#pragma unroll
            for (int k = 0; k < 4; ++k)
                w[k] = (uint32_t)f32_to_bf16_bits(x[2 * k]) |
                       ((uint32_t)f32_to_bf16_bits(x[2 * k + 1]) << 16);
            *(uint4 *)((uint16_t *)dst + i) = make_uint4(w[0], w[1], w[2], w[3]);
        }
    } else {
        // fp8: code of the correctly rounded fp32 quotient x / scale
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            lo |= (uint32_t)f32_to_e4m3(__fdiv_rn(x[k], inv_scale_div)) << (8 * k);
            hi |= (uint32_t)f32_to_e4m3(__fdiv_rn(x[k + 4], inv_scale_div)) << (8 * k);
        }
        *(uint2 *)((uint8_t *)dst + i) = make_uint2(lo, hi);
    }
}

template <int SRC, int DST>
__global__ void __launch_bounds__(256)
paged_append_kernel(AppendArgs a)
{
    const bool is_v = blockIdx.y == 1;
    const int64_t chunks_per_row = (is_v ? a.v_head_dim : a.head_dim) / 8;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = a.n_tok * a.kv_heads * chunks_per_row;
    if (gid >= total)
        return;
    const void *src = is_v ? a.new_v : a.new_k;
    void *pool = is_v ? a.v_data : a.k_data;
    const int64_t sp = is_v ? a.v_stride_page : a.k_stride_page;
    const int64_t sh = is_v ? a.v_stride_head : a.k_stride_head;
    const int64_t st = is_v ? a.v_stride_token : a.k_stride_token;
    const float scale = is_v ? a.v_scale : a.k_scale;

    const int64_t c = gid % chunks_per_row;
    const int64_t h = (gid / chunks_per_row) % a.kv_heads;
    const int64_t t = gid / (chunks_per_row * a.kv_heads);
    const bool lead = c == 0 && h == 0 && !is_v;
    int64_t slot;
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
            return;
        }
        const int32_t page = a.block_table[b * a.max_pages + pos / a.page_tokens];
        if (page < 0 || page >= a.num_pages) {
            if (lead)
                flag_error(a.dev_err, NBX_DEVERR_PAGE_RANGE);
            return;
        }
        slot = (int64_t)page * a.page_tokens + pos % a.page_tokens;
    }
    if (slot < 0)
        return;                                            // padding token
    if (slot >= (int64_t)a.num_pages * a.page_tokens) {
        if (lead)
            flag_error(a.dev_err, NBX_DEVERR_SLOT_RANGE);
        return;
    }
    const int64_t page = slot / a.page_tokens;
    const int64_t row = slot - page * a.page_tokens;
    const int64_t si = t * (is_v ? a.v_new_stride_tok : a.new_stride_tok) +
                       h * (is_v ? a.v_new_stride_head : a.new_stride_head) + c * 8;
    const int64_t di = page * sp + h * sh + row * st + c * 8;
    float x[8];
    load8<SRC>(src, si, x);
    store8<SRC, DST>(pool, di, x, scale, src, si);
}

template <int SRC, int DST>
static hipError_t launch_append_t(const AppendArgs &a, hipStream_t stream)
{
    const int32_t widest = a.new_v && a.v_head_dim > a.head_dim ? a.v_head_dim : a.head_dim;
    const int64_t total = a.n_tok * a.kv_heads * (widest / 8);
    dim3 grid((unsigned)((total + 255) / 256), a.new_v ? 2 : 1);
    hipLaunchKernelGGL((paged_append_kernel<SRC, DST>), grid, dim3(256), 0, stream, a);
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
