// Fixed-order combine of split partials (nbxtensor attention_wrappers.py,
// decode_reduce: one program per query row, partials combined in a fixed
// order so the result does not depend on scheduling).
//
// Per row: M = the largest m_s over non-empty splits (m_s = -inf marks an
// empty one, whose o is not read), w_s = exp(m_s - M), out = sum_s w_s o_s /
// sum_s w_s l_s.
//
// One workgroup of 4 waves per row, wave k owning the columns [k D/4, (k+1)
// D/4).  A lane takes 4 consecutive columns of one split, so a wave covers
// 256 / (D/4) splits per pass; with up to 64 splits every load of the row
// (m, l and all o pieces) is issued at once and the row takes one memory
// round trip.  The number of passes is a template argument, the fewest that
// cover the launch's split count, so that no load is issued for splits that
// do not exist.  Each lane sums its splits in ascending order, then the lanes
// holding different splits of the same columns are added by a fixed butterfly
// (and the denominator by a wave butterfly), so the order is fixed and
// repeated runs give identical bits.  No LDS and no barrier: the four waves
// of a row compute M and the denominator alike and are otherwise independent.
#include "device_common.h"
#include "kernels.h"

namespace nbx {

namespace {

constexpr int kMaxSplitsMerge = 4096;

__device__ __forceinline__ float4 fma4(float w, float4 v, float4 acc)
{
    return make_float4(fmaf(w, v.x, acc.x), fmaf(w, v.y, acc.y), fmaf(w, v.z, acc.z),
                       fmaf(w, v.w, acc.w));
}

template <int D, int OUT, int NP>
__global__ void __launch_bounds__(256)
merge_kernel(MergeArgs a)
{
    constexpr int CW = D / 4;                  // columns per wave
    constexpr int LPS = CW / 4;                // lanes per split (4 columns each)
    constexpr int SPP = 64 / LPS;              // splits per pass
    static_assert(NP >= 1 && NP <= LPS, "at most 64 splits in flight");
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t row = blockIdx.x;
    const int ns = a.n_split;
    const float *m = a.m_part + row * ns;
    const float *l = a.l_part + row * ns;
    const int sub = lane / LPS;                // this lane's split within a pass
    const int col = wv * CW + (lane % LPS) * 4;
    const float *o = a.o_part + row * (int64_t)ns * D + col;
    const bool den_lane = lane % LPS == 0;     // one lane per split adds w_s l_s

    float M = -INFINITY;
    bool has_nan = false;
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    float den = 0.0f;
    auto weight = [&](float ms) {
        return (ms == -INFINITY || M == -INFINITY) ? 0.0f : exp2f((ms - M) * kLog2e);
    };
    if (ns <= SPP * NP) {
        // one round trip: every piece of the row in flight together
        float4 v[NP];
        float ms[NP], ls[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int s = p * SPP + sub;
            const bool in = s < ns;
            v[p] = in ? *(const float4 *)(o + (int64_t)s * D) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            ms[p] = in ? m[s] : -INFINITY;
            ls[p] = in ? l[s] : 0.0f;
        }
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            has_nan |= ms[p] != ms[p];
            M = fmaxf(M, ms[p]);
        }
        M = wave_max(M);
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const float w = weight(ms[p]);
            if (w != 0.0f)                     // an empty split's o is not defined: skip it
                acc = fma4(w, v[p], acc);
            if (den_lane)
                den = fmaf(w, ls[p], den);
        }
    } else {
        for (int s = lane; s < ns; s += 64) {
            const float ms = m[s];
            has_nan |= ms != ms;
            M = fmaxf(M, ms);
        }
        M = wave_max(M);
        for (int s0 = 0; s0 < ns; s0 += SPP * NP) {
            float4 v[NP];
            float ms[NP], ls[NP];
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                const int s = s0 + p * SPP + sub;
                const bool in = s < ns;
                v[p] = in ? *(const float4 *)(o + (int64_t)s * D)
                          : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                ms[p] = in ? m[s] : -INFINITY;
                ls[p] = in ? l[s] : 0.0f;
            }
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                const float w = weight(ms[p]);
                if (w != 0.0f)
                    acc = fma4(w, v[p], acc);
                if (den_lane)
                    den = fmaf(w, ls[p], den);
            }
        }
    }
    has_nan = __any(has_nan);
    den = wave_sum(den);
#pragma unroll
    for (int off = LPS; off < 64; off <<= 1) {
        acc.x += __shfl_xor(acc.x, off, 64);
        acc.y += __shfl_xor(acc.y, off, 64);
        acc.z += __shfl_xor(acc.z, off, 64);
        acc.w += __shfl_xor(acc.w, off, 64);
    }
    if (sub == 0) {
        float r[4] = {acc.x, acc.y, acc.z, acc.w};
#pragma unroll
        for (int k = 0; k < 4; ++k)
            r[k] = has_nan ? __builtin_nanf("") : (den > 0.0f ? r[k] / den : 0.0f);
        if constexpr (OUT == NBX_F32) {
            *(float4 *)((float *)a.out + row * D + col) = make_float4(r[0], r[1], r[2], r[3]);
        } else {
            const uint32_t lo = (uint32_t)f32_to_bf16_bits(r[0]) |
                                ((uint32_t)f32_to_bf16_bits(r[1]) << 16);
            const uint32_t hi = (uint32_t)f32_to_bf16_bits(r[2]) |
                                ((uint32_t)f32_to_bf16_bits(r[3]) << 16);
            *(uint2 *)((uint16_t *)a.out + row * D + col) = make_uint2(lo, hi);
        }
    }
}

// passes: the fewest powers of two that cover n_split splits at SPP splits per
// pass, at most the 64-split one-round-trip form (more splits loop over it)
template <int D, int OUT>
hipError_t launch_np(const MergeArgs &a, hipStream_t stream)
{
    constexpr int LPS = D / 16, SPP = 64 / LPS;
    dim3 grid((unsigned)a.rows);
    if (!grid_fits(a.rows, 256))
        return hipErrorInvalidConfiguration;
    const int need = (a.n_split + SPP - 1) / SPP;
    if (need <= 1)
        hipLaunchKernelGGL((merge_kernel<D, OUT, 1>), grid, dim3(256), 0, stream, a);
    else if (need <= 2)
        hipLaunchKernelGGL((merge_kernel<D, OUT, 2>), grid, dim3(256), 0, stream, a);
    else if (need <= 4 || LPS == 4)
        hipLaunchKernelGGL((merge_kernel<D, OUT, (LPS < 4 ? LPS : 4)>), grid, dim3(256), 0, stream,
                           a);
    else if (need <= 8 || LPS == 8)
        hipLaunchKernelGGL((merge_kernel<D, OUT, (LPS < 8 ? LPS : 8)>), grid, dim3(256), 0, stream,
                           a);
    else
        hipLaunchKernelGGL((merge_kernel<D, OUT, LPS>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <int OUT>
hipError_t launch_out(const MergeArgs &a, hipStream_t stream)
{
    switch (a.head_dim) {
    case 64: return launch_np<64, OUT>(a, stream);
    case 128: return launch_np<128, OUT>(a, stream);
    default: return launch_np<256, OUT>(a, stream);
    }
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
