// Fixed-order combine of split partials (nbxtensor attention_wrappers.py,
// decode_reduce: one program per query row, partials in split order).
//
// Per row: M = the largest m_s over non-empty splits (m_s = -inf marks an
// empty one), w_s = exp(m_s - M), out = sum_s w_s o_s / sum_s w_s l_s with s
// ascending.  One wave per row; each lane owns D/64 consecutive elements so
// the o_s rows are read with coalesced vector loads.
#include "device_common.h"
#include "kernels.h"

namespace nbx {

namespace {

template <int D, int OUT>
__global__ void __launch_bounds__(256)
merge_kernel(MergeArgs a)
{
    constexpr int E = D / 64;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= a.rows)
        return;
    const int ns = a.n_split;
    const float *m = a.m_part + row * ns;
    const float *l = a.l_part + row * ns;
    const float *o = a.o_part + row * (int64_t)ns * D + lane * E;

    float M = -INFINITY;
    bool has_nan = false;
    for (int s = 0; s < ns; ++s) {
        const float ms = m[s];
        has_nan |= ms != ms;
        M = fmaxf(M, ms);
    }
    float acc[E];
#pragma unroll
    for (int k = 0; k < E; ++k)
        acc[k] = 0.0f;
    float den = 0.0f;
    if (M != -INFINITY) {
        for (int s = 0; s < ns; ++s) {
            const float ms = m[s];
            if (ms == -INFINITY)
                continue;
            const float w = exp2f((ms - M) * kLog2e);
            den = fmaf(w, l[s], den);
            const float *os = o + (int64_t)s * D;
            if constexpr (E == 4) {
                const float4 v = *(const float4 *)os;
                acc[0] = fmaf(w, v.x, acc[0]);
                acc[1] = fmaf(w, v.y, acc[1]);
                acc[2] = fmaf(w, v.z, acc[2]);
                acc[3] = fmaf(w, v.w, acc[3]);
            } else if constexpr (E == 2) {
                const float2 v = *(const float2 *)os;
                acc[0] = fmaf(w, v.x, acc[0]);
                acc[1] = fmaf(w, v.y, acc[1]);
            } else {
                acc[0] = fmaf(w, os[0], acc[0]);
            }
        }
    }
    float res[E];
#pragma unroll
    for (int k = 0; k < E; ++k)
        res[k] = has_nan ? __builtin_nanf("") : (den > 0.0f ? acc[k] / den : 0.0f);

    if constexpr (OUT == NBX_F32) {
        float *dst = (float *)a.out + row * D + lane * E;
#pragma unroll
        for (int k = 0; k < E; ++k)
            dst[k] = res[k];
    } else {
        uint16_t *dst = (uint16_t *)a.out + row * D + lane * E;
#pragma unroll
        for (int k = 0; k < E; ++k)
            dst[k] = f32_to_bf16_bits(res[k]);
    }
}

template <int OUT>
hipError_t launch_out(const MergeArgs &a, hipStream_t stream)
{
    dim3 grid((unsigned)((a.rows + 3) / 4));
    switch (a.head_dim) {
    case 64: hipLaunchKernelGGL((merge_kernel<64, OUT>), grid, dim3(256), 0, stream, a); break;
    case 128: hipLaunchKernelGGL((merge_kernel<128, OUT>), grid, dim3(256), 0, stream, a); break;
    default: hipLaunchKernelGGL((merge_kernel<256, OUT>), grid, dim3(256), 0, stream, a); break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const MergeArgs &a, hipStream_t stream)
{
    if (a.rows == 0)
        return hipSuccess;
    return a.out_dtype == NBX_F32 ? launch_out<NBX_F32>(a, stream) : launch_out<NBX_BF16>(a, stream);
}

}  // namespace nbx
