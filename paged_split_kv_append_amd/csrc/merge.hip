// Fixed-order combine of split partials (nbxtensor attention_wrappers.py,
// decode_reduce: one program per query row, partials combined in a fixed
// order so the result does not depend on scheduling).
//
// Per row: M = the largest m_s over non-empty splits (m_s = -inf marks an
// empty one, whose o is not read), w_s = exp(m_s - M), out = sum_s w_s o_s /
// sum_s w_s l_s.
//
// One workgroup of 4 waves per row.  The lanes first take the splits 64 at a
// time to form M, the weights w_s (kept in LDS) and the denominator by a
// butterfly sum; then wave k accumulates w_s o_s over the splits s = k, k + 4,
// ... in ascending order, with 8 independent loads in flight, each lane owning
// D/64 consecutive elements; the four wave sums are added in order 0..3.  The
// order is fixed, so repeated runs give identical bits.
#include "device_common.h"
#include "kernels.h"

namespace nbx {

namespace {

constexpr int kMaxSplitsMerge = 4096;

template <int D, int OUT>
__global__ void __launch_bounds__(256)
merge_kernel(MergeArgs a)
{
    constexpr int E = D / 64;
    __shared__ float w_s[kMaxSplitsMerge];
    __shared__ float red[4][D];
    __shared__ float stat[2];                  // M, den
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t row = blockIdx.x;
    const int ns = a.n_split;
    const float *m = a.m_part + row * ns;
    const float *l = a.l_part + row * ns;

    if (wv == 0) {
        float M = -INFINITY;
        bool has_nan = false;
        for (int s = lane; s < ns; s += 64) {
            const float ms = m[s];
            has_nan |= ms != ms;
            M = fmaxf(M, ms);
        }
        M = wave_max(M);
        has_nan = __any(has_nan);
        float den = 0.0f;
        for (int s = lane; s < ns; s += 64) {
            const float ms = m[s];
            const float w = (ms == -INFINITY || M == -INFINITY) ? 0.0f
                                                                 : exp2f((ms - M) * kLog2e);
            w_s[s] = w;
            den = fmaf(w, l[s], den);
        }
        den = wave_sum(den);
        if (lane == 0) {
            stat[0] = has_nan ? __builtin_nanf("") : M;
            stat[1] = den;
        }
    }
    __syncthreads();

    float acc[E];
#pragma unroll
    for (int k = 0; k < E; ++k)
        acc[k] = 0.0f;
    const float *o = a.o_part + row * (int64_t)ns * D + lane * E;
    int s = wv;
    for (; s + 28 < ns; s += 32) {             // 8 splits of this wave per batch
        float v[8][E];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const float *os = o + (int64_t)(s + 4 * u) * D;
#pragma unroll
            for (int k = 0; k < E; ++k)
                v[u][k] = os[k];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const float w = w_s[s + 4 * u];
#pragma unroll
            for (int k = 0; k < E; ++k)   // an empty split's o is not defined: skip it
                acc[k] = w != 0.0f ? fmaf(w, v[u][k], acc[k]) : acc[k];
        }
    }
    for (; s < ns; s += 4) {
        const float w = w_s[s];
        if (w == 0.0f)
            continue;
        const float *os = o + (int64_t)s * D;
#pragma unroll
        for (int k = 0; k < E; ++k)
            acc[k] = fmaf(w, os[k], acc[k]);
    }
#pragma unroll
    for (int k = 0; k < E; ++k)
        red[wv][lane * E + k] = acc[k];
    __syncthreads();

    const float M = stat[0], den = stat[1];
    for (int e = threadIdx.x; e < D; e += 256) {
        float r = ((red[0][e] + red[1][e]) + red[2][e]) + red[3][e];
        r = M != M ? __builtin_nanf("") : (den > 0.0f ? r / den : 0.0f);
        if constexpr (OUT == NBX_F32)
            ((float *)a.out)[row * D + e] = r;
        else
            ((uint16_t *)a.out)[row * D + e] = f32_to_bf16_bits(r);
    }
}

template <int OUT>
hipError_t launch_out(const MergeArgs &a, hipStream_t stream)
{
    dim3 grid((unsigned)a.rows);
    switch (a.head_dim) {
    case 64: hipLaunchKernelGGL((merge_kernel<64, OUT>), grid, dim3(256), 0, stream, a); break;
    case 128: hipLaunchKernelGGL((merge_kernel<128, OUT>), grid, dim3(256), 0, stream, a); break;
    default: hipLaunchKernelGGL((merge_kernel<256, OUT>), grid, dim3(256), 0, stream, a); break;
    }
    return hipGetLastError();
}

}  // namespace

int merge_max_splits() { return kMaxSplitsMerge; }

hipError_t launch_merge(const MergeArgs &a, hipStream_t stream)
{
    if (a.rows == 0)
        return hipSuccess;
    return a.out_dtype == NBX_F32 ? launch_out<NBX_F32>(a, stream) : launch_out<NBX_BF16>(a, stream);
}

}  // namespace nbx
