// General split partial on the vector ALUs (any pool dtype, fp32 or bf16 Q).
//
// The split kernel of the nbxtensor paged_decode_attn.py page
// (paged_decode_attn_split_kernel): per split, scores q . k * scale for every
// position of the split, an online softmax (running max m, sum l, correction
// exp(m_old - m_new)), and an fp32 accumulator of p * v; the unnormalised
// (o, m, l) is stored.  Here one workgroup serves up to RB query rows of one KV
// head (GQA heads and window rows), so each K/V element of the split is read
// by one workgroup only.
//
// Workgroup (256 threads) per (row block, split, sequence * KV head); the row
// block is the fastest grid axis so the row blocks of one split run together.
// A split is walked in chunks of 64 positions:
//   A. 4 threads per position form q . k for every row (D/4 elements each,
//      combined by lane shuffles) and write the scaled score to LDS;
//   B. one wave per row takes the chunk max, rescales, forms p = 2^(s - m);
//   C. each thread owns one element e of the V head dim DV (which may differ
//      from the q/k head dim D) and a position phase, accumulating p * v[e];
//      phases are summed in a fixed order at the end.
// Scores are kept in log2 units (scale * log2 e folded in); m is stored back
// in natural-log units.
#include "device_common.h"
#include "kernels.h"

namespace nbx {

namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 64;

template <int QT>
__device__ __forceinline__ float load_q(const void *q, int64_t i)
{
    if constexpr (QT == NBX_F32)
        return ((const float *)q)[i];
    else
        return bf16_bits_to_f32(((const uint16_t *)q)[i]);
}

template <int KVT, int QT, int D, int DV, int RB>
__global__ void __launch_bounds__(kThreads)
partial_valu_kernel(PartialArgs a)
{
    constexpr int PG = kThreads / DV;         // position phases in step C
    __shared__ float q_s[RB][D];
    __shared__ float p_s[RB][kChunk];
    __shared__ int32_t page_s[kChunk];
    __shared__ float m_s[RB], l_s[RB], corr_s[RB];
    __shared__ int32_t n_s[RB];
    __shared__ float red_s[PG][RB][DV];

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int rb = blockIdx.x, s = blockIdx.y;
    const int b = blockIdx.z / a.kv_heads, g = blockIdx.z % a.kv_heads;
    const int row0 = rb * RB;
    const int rows_here = min(RB, a.rows_per_kv - row0);
    const int64_t row_base = ((int64_t)b * a.q_heads + (int64_t)g * a.group) * a.q_rows;

    const int S = device_split_size(a);
    int L = a.seq_lens[b];
    const int cap = a.max_pages * a.page_tokens;
    if (L < 0 || L > cap) {
        if (t == 0 && rb == 0 && s == 0)
            flag_error(a.dev_err, NBX_DEVERR_SEQ_RANGE);
        L = L < 0 ? 0 : cap;
    }
    if (s == a.n_split - 1 && L > a.n_split * S && t == 0 && rb == 0)
        flag_error(a.dev_err, NBX_DEVERR_SEQ_RANGE);

    for (int idx = t; idx < RB * D; idx += kThreads) {
        const int i = idx / D, e = idx % D;
        q_s[i][e] = i < rows_here ? load_q<QT>(a.q, (row_base + row0 + i) * D + e) : 0.0f;
    }
    const int wb = seq_window(a, b, t == 0 && rb == 0 && s == 0);
    if (t < RB) {
        const int n = t < rows_here ? row_keys(a, L, wb, (row0 + t) % a.q_rows) : 0;
        n_s[t] = n;
        m_s[t] = -INFINITY;
        l_s[t] = 0.0f;
    }
    __syncthreads();

    int n_max = 0;
#pragma unroll
    for (int i = 0; i < RB; ++i)
        n_max = max(n_max, n_s[i]);
    const int j_begin = s * S;
    const int j_end = min(j_begin + S, n_max);
    const float scale2 = a.scale * a.k_scale * kLog2e;

    const int e_c = t % DV, pg = t / DV;
    float acc[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i)
        acc[i] = 0.0f;

    for (int c0 = j_begin; c0 < j_end; c0 += kChunk) {
        // ---- A: scores
        {
            const int p = t >> 2, part = t & 3;
            const int j = c0 + p;
            bool valid = j < j_end;
            int64_t kbase = 0;
            if (valid) {
                const int page = a.block_table[(int64_t)b * a.max_pages + j / a.page_tokens];
                if (page < 0 || page >= a.num_pages) {
                    valid = false;
                    if (part == 0)
                        flag_error(a.dev_err, NBX_DEVERR_PAGE_RANGE);
                }
                if (part == 0)
                    page_s[p] = valid ? page : -1;
                kbase = (int64_t)page * a.k_stride_page + (int64_t)g * a.k_stride_head +
                        (int64_t)(j % a.page_tokens) * a.k_stride_token;
            } else if (part == 0) {
                page_s[p] = -1;
            }
            float dots[RB];
#pragma unroll
            for (int i = 0; i < RB; ++i)
                dots[i] = 0.0f;
            if (valid) {
                constexpr int Q4 = D / 4;
#pragma unroll 8
                for (int k = 0; k < Q4; ++k) {
                    const int e = part * Q4 + k;
                    const float kv = load_elem<KVT>(a.k_data, kbase + e);
#pragma unroll
                    for (int i = 0; i < RB; ++i)
                        dots[i] = fmaf(q_s[i][e], kv, dots[i]);
                }
            }
#pragma unroll
            for (int i = 0; i < RB; ++i) {
                dots[i] += __shfl_xor(dots[i], 1, 64);
                dots[i] += __shfl_xor(dots[i], 2, 64);
            }
            if (part == 0) {
#pragma unroll
                for (int i = 0; i < RB; ++i)
                    p_s[i][p] = (valid && j < n_s[i]) ? dots[i] * scale2 : -INFINITY;
            }
        }
        __syncthreads();
        // ---- B: online softmax, one wave per row
        for (int i = wave; i < RB; i += kThreads / 64) {
            const float sv = p_s[i][lane];
            const float m_old = m_s[i];
            const float m_new = fmaxf(m_old, wave_max(sv));
            const float m_safe = m_new == -INFINITY ? 0.0f : m_new;
            const float pv = exp2f(sv - m_safe);
            const float psum = wave_sum(pv);
            p_s[i][lane] = pv;
            if (lane == 0) {
                const float corr = exp2f(m_old - m_safe);
                corr_s[i] = corr;
                l_s[i] = l_s[i] * corr + psum;
                m_s[i] = m_new;
            }
        }
        __syncthreads();
        // ---- C: p * v
#pragma unroll
        for (int i = 0; i < RB; ++i)
            acc[i] *= corr_s[i];
        for (int p = pg; p < kChunk; p += PG) {
            const int page = page_s[p];
            if (page < 0)
                continue;
            const int j = c0 + p;
            const int64_t vi = (int64_t)page * a.v_stride_page + (int64_t)g * a.v_stride_head +
                               (int64_t)(j % a.page_tokens) * a.v_stride_token + e_c;
            const float v = load_elem<KVT>(a.v_data, vi) * a.v_scale;
#pragma unroll
            for (int i = 0; i < RB; ++i)
                acc[i] = fmaf(p_s[i][p], v, acc[i]);
        }
        __syncthreads();
    }

    // fixed-order sum of the position phases, then store the partial
#pragma unroll
    for (int i = 0; i < RB; ++i)
        red_s[pg][i][e_c] = acc[i];
    __syncthreads();
    for (int idx = t; idx < rows_here * DV; idx += kThreads) {
        const int i = idx / DV, e = idx % DV;
        float o = 0.0f;
#pragma unroll
        for (int k = 0; k < PG; ++k)
            o += red_s[k][i][e];
        const int64_t row = row_base + row0 + i;
        a.o_part[(row * a.n_split + s) * DV + e] = o;
        if (e == 0) {
            const float m = m_s[i];
            a.m_part[row * a.n_split + s] = m == -INFINITY ? -INFINITY : m * kLn2;
            a.l_part[row * a.n_split + s] = l_s[i];
        }
    }
}

template <int KVT, int QT, int D, int DV>
hipError_t launch_rb(const PartialArgs &a, hipStream_t stream)
{
    const int M = a.rows_per_kv;
    dim3 grid(0, a.n_split, a.batch * a.kv_heads);
#define NBX_LAUNCH(RB_)                                                                   \
    do {                                                                                  \
        grid.x = (M + (RB_)-1) / (RB_);                                                   \
        hipLaunchKernelGGL((partial_valu_kernel<KVT, QT, D, DV, RB_>), grid, dim3(kThreads), \
                           0, stream, a);                                                 \
    } while (0)
    if (M <= 1)
        NBX_LAUNCH(1);
    else if (M <= 2)
        NBX_LAUNCH(2);
    else if (M <= 4)
        NBX_LAUNCH(4);
    else
        NBX_LAUNCH(8);
#undef NBX_LAUNCH
    return hipGetLastError();
}

template <int KVT, int QT>
hipError_t launch_d(const PartialArgs &a, hipStream_t stream)
{
    switch (a.head_dim) {
    case 64: return launch_rb<KVT, QT, 64, 64>(a, stream);
    case 128: return launch_rb<KVT, QT, 128, 128>(a, stream);
    case 192: return launch_rb<KVT, QT, 192, 128>(a, stream);   // the only pair with 192
    default: return launch_rb<KVT, QT, 256, 256>(a, stream);
    }
}

}  // namespace

hipError_t launch_partial_valu(const PartialArgs &a, hipStream_t stream)
{
    const bool qf = a.q_dtype == NBX_F32;
    switch (a.kv_dtype) {
    case NBX_F32: return qf ? launch_d<NBX_F32, NBX_F32>(a, stream)
                            : launch_d<NBX_F32, NBX_BF16>(a, stream);
    case NBX_BF16: return qf ? launch_d<NBX_BF16, NBX_F32>(a, stream)
                             : launch_d<NBX_BF16, NBX_BF16>(a, stream);
    default: return qf ? launch_d<NBX_FP8_E4M3, NBX_F32>(a, stream)
                       : launch_d<NBX_FP8_E4M3, NBX_BF16>(a, stream);
    }
}

}  // namespace nbx
