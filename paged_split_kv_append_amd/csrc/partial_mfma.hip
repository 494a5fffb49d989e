// Split partials on the matrix cores for bf16 and fp8 (E4M3FN) pools with bf16 Q.
//
// The computation is that of the split kernel on the nbxtensor
// paged_decode_attn.py page (paged_decode_attn_split_kernel): per split, the
// scores q . k * scale over the split's positions, an online softmax (running
// max, running sum, correction factor) and an fp32 accumulator of p * v,
// stored unnormalised.  All query rows that share a KV head (GQA heads x
// window rows, the grouping of the nbxtensor attention_wrappers.py page,
// _math_attention) form the N side of the products, so each K/V byte is read
// from HBM once per split however many rows use it (TensorFold PR #1219).
//
// Products are v_mfma_f32_16x16x32_bf16 with fp32 accumulation:
//   S^T (16 positions x 16 rows) = K (16 x D) . Q^T (D x 16)
//   O^T (16 columns x 16 rows) += V^T (16 x 32 positions) . P^T (32 x 16)
// so that every lane owns one query row (its column) in both S^T and O^T and
// the softmax bookkeeping never leaves the lane's row.  K rows feed the A
// operand straight from 16-byte loads; V goes through LDS and is transposed
// by the LDS transpose read.  bf16 K/V products are exact; P is rounded to
// bf16 for the P V product, and for bf16 pools its rounding residual is
// multiplied in a second MFMA (P = hi + lo, relative error ~2^-17).  fp8 codes
// are widened to bf16 exactly; their per-tensor scales are applied to the
// scores (K) and to nothing else until the merge sees o (V scale folded into
// o here).  Scores are kept in log2 units.
//
// Two kernels:
//  - decode_mfma_kernel: at most 16 rows per KV head (decode, short windows).
//    One workgroup of 4 waves per (split, sequence x KV head); the waves take
//    interleaved 32-position chunks of the split, each with its own running
//    (m, l, O), and combine them in a fixed order at the end.  K goes from HBM
//    into MFMA operand registers; each wave stages its V chunk in private LDS.
//    The next chunk's loads are issued before the current one is computed.
//  - multirow_mfma_kernel: more rows per KV head (verify windows, prompt
//    chunks).  A workgroup takes RW x NT row tiles of 16 rows; its waves share
//    each K/V chunk through LDS (K XOR-swizzled for conflict-free operand
//    reads).  Workgroups are ordered row block fastest and mapped so that the
//    row blocks of one split land on the same XCD and share its L2.
#include "kernels.h"
#include "mfma_common.h"

namespace nbx {

namespace {

constexpr int kChunk = 32;   // positions per chunk: two 16-position S tiles, one PV k-step

template <int KVT, int UPT>
struct Loaded {
    u32x4 u[UPT];
};

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

// Online-softmax step for one lane's row over the 32 positions of a chunk:
// sc holds the scaled scores (log2 units, -inf where masked).  Updates m, l,
// rescales o and returns the P operand (hi and residual lo parts).
template <int DT, bool PVS>
__device__ __forceinline__ void softmax_step(float (&sc)[2][4], float &m_run, float &l_run,
                                             f32x4 (&o)[DT], u32x4 &ph, u32x4 &pl)
{
    float mx = sc[0][0];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            mx = fmaxf(mx, sc[t][i]);
    mx = xor_max16_32(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_safe = m_new == -INFINITY ? 0.0f : m_new;
    const float corr = fast_exp2(m_run - m_safe);
    float p[2][4], psum = 0.0f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p[t][i] = fast_exp2(sc[t][i] - m_safe);
            psum += p[t][i];
        }
    l_run = l_run * corr + psum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
        o[dt] *= corr;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        ph[2 * t] = pack_bf16(p[t][0], p[t][1]);
        ph[2 * t + 1] = pack_bf16(p[t][2], p[t][3]);
        if constexpr (PVS) {
            pl[2 * t] = pack_bf16(p[t][0] - bf16_round(p[t][0]), p[t][1] - bf16_round(p[t][1]));
            pl[2 * t + 1] =
                pack_bf16(p[t][2] - bf16_round(p[t][2]), p[t][3] - bf16_round(p[t][3]));
        }
    }
}

// ------------------------------------------------------------------ decode

// Swizzle of the 16-byte units of V tile row r: unit U of the row is stored at
// U ^ vswz(r), so that the 16 rows read by one transposed read spread over all
// LDS banks.
template <int UPR>
__device__ __forceinline__ int vswz(int r)
{
    return (2 * r) & (UPR - 2);
}

// Byte address in a swizzled [32 x D] bf16 V tile of the A operand of the P V
// product for column tile dt: lane 16 g + j reads 4 elements of rows
// 16 h + 4 g + j/4, columns 16 dt + 4 (j % 4) .. + 3.
template <int D>
__device__ __forceinline__ u32x4 lds_vt_operand_swz(const uint8_t *tile, int dt, int lane)
{
    constexpr int UPR = D / 8;
    const int g = lane >> 4, j = lane & 15;
    const int U = 2 * dt + ((j >> 1) & 1);
    const int r0 = 4 * g + (j >> 2), r1 = r0 + 16;
    const uint8_t *p0 = tile + r0 * (2 * D) + ((U ^ vswz<UPR>(r0)) * 16) + 8 * (j & 1);
    const uint8_t *p1 = tile + r1 * (2 * D) + ((U ^ vswz<UPR>(r1)) * 16) + 8 * (j & 1);
    const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4 *)(__attribute__((address_space(3))) uint8_t *)p0);
    const bf16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4 *)(__attribute__((address_space(3))) uint8_t *)p1);
    const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
    return u32x4{ua[0], ua[1], ub[0], ub[1]};
}

// PG waves per (split, sequence x KV head); wave w takes chunks w, w + PG, ...
template <int D, int KVT, bool PVS, int PG>
__global__ void __launch_bounds__(PG * 64)
decode_mfma_kernel(PartialArgs a)
{
    constexpr int KK = D / 32;                 // 32-wide k-steps of Q K^T
    constexpr int DT = D / 16;                 // 16-column tiles of O
    constexpr int UPR = D / 8;                 // 16-byte (8-element) units per V row
    constexpr int RPI = 64 / UPR;              // V rows per 64-lane load
    constexpr int VU = kChunk / RPI;           // V loads per lane per chunk
    constexpr int VBYTES = kChunk * 2 * D;     // one V tile (bf16)
    constexpr int CMB = PG > 1 ? PG * 16 * D * 4 : 0;
    constexpr int SMEM = (PG * VBYTES > CMB) ? PG * VBYTES : CMB;
    __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];
    __shared__ float cmb_m[PG][16], cmb_l[PG][16];

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int g = lane >> 4, j = lane & 15;
    const int s = blockIdx.x;
    const int b = blockIdx.y / a.kv_heads, gk = blockIdx.y % a.kv_heads;
    const int M = a.rows_per_kv;
    const int64_t row_base = ((int64_t)b * a.q_heads + (int64_t)gk * a.group) * a.q_rows;
    const bool lead = threadIdx.x == 0;

    const int L = clamp_len(a, b, lead && s == 0);
    if (lead && s == a.n_split - 1 && L > a.n_split * a.split_size)
        flag_error(a.dev_err, NBX_DEVERR_SEQ_RANGE);

    int n_j = 0;
    if (j < M) {
        n_j = a.causal ? L - a.q_rows + (j % a.q_rows) + 1 : L;
        n_j = n_j < 0 ? 0 : n_j;
    }
    int n_max = a.causal ? L - a.q_rows + min(M, a.q_rows) : L;
    n_max = n_max < 0 ? 0 : n_max;
    const int j0 = s * a.split_size;
    const int jend = min(j0 + a.split_size, n_max);
    const int e_j = min(jend, n_j);
    const int nchunk = jend > j0 ? (jend - j0 + kChunk - 1) / kChunk : 0;

    u32x4 qb[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
        qb[kk] = j < M ? *(const u32x4 *)((const uint16_t *)a.q + (row_base + j) * D + kk * 32 +
                                          g * 8)
                       : u32x4{0, 0, 0, 0};

    const float scale2 = a.scale * a.k_scale * kLog2e;
    float m_run = -INFINITY, l_run = 0.0f;
    f32x4 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
        o[dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    uint8_t *vt = smem + w * VBYTES;
    const int64_t k_head = (int64_t)gk * a.k_stride_head;
    const int64_t v_head = (int64_t)gk * a.v_stride_head;

    int pg_reg = -1;                           // lane i: page of tile (i & 1) of chunk q0 + i/2
    for (int q = 0, c = w; c < nchunk; ++q, c += PG) {
        if ((q & 31) == 0) {
            // page ids of this wave's next 32 chunks, one tile per lane
            const int cq = c + (lane >> 1) * PG;
            const int ts = j0 + cq * kChunk + 16 * (lane & 1);
            pg_reg = cq < nchunk ? tile_page(a, b, ts, jend, true) : -1;
        }
        const int p0 = j0 + c * kChunk;
        const int page0 = __builtin_amdgcn_readlane(pg_reg, 2 * (q & 31));
        const int page1 = __builtin_amdgcn_readlane(pg_reg, 2 * (q & 31) + 1);
        const int64_t off0 = (int64_t)(p0 % a.page_tokens);
        const int64_t off1 = (int64_t)((p0 + 16) % a.page_tokens);
        const int64_t kb0 = (int64_t)page0 * a.k_stride_page + k_head + off0 * a.k_stride_token;
        const int64_t kb1 = (int64_t)page1 * a.k_stride_page + k_head + off1 * a.k_stride_token;
        const int64_t vb0 = (int64_t)page0 * a.v_stride_page + v_head + off0 * a.v_stride_token;
        const int64_t vb1 = (int64_t)page1 * a.v_stride_page + v_head + off1 * a.v_stride_token;
        const int vrows = min(kChunk, jend - p0);          // V rows holding positions < jend

        // K rows straight into MFMA A operands (rows past jend are masked later)
        u32x4 kr[2][KK];
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            kr[0][kk] = page0 >= 0 ? load8_bf16<KVT>(a.k_data, kb0 + j * a.k_stride_token +
                                                                   kk * 32 + g * 8)
                                   : u32x4{0, 0, 0, 0};
            kr[1][kk] = page1 >= 0 ? load8_bf16<KVT>(a.k_data, kb1 + j * a.k_stride_token +
                                                                   kk * 32 + g * 8)
                                   : u32x4{0, 0, 0, 0};
        }
        // V rows into this wave's swizzled LDS tile; rows without data become 0
#pragma unroll
        for (int u = 0; u < VU; ++u) {
            const int r = u * RPI + lane / UPR, U = lane % UPR;
            const int t = r >> 4;
            const int page = t ? page1 : page0;
            const bool ok = page >= 0 && r < vrows;
            const int64_t src = (t ? vb1 : vb0) + (r & 15) * a.v_stride_token + (U ^ vswz<UPR>(r)) * 8;
            uint8_t *dst = vt + u * 1024;
            if constexpr (KVT == NBX_BF16) {
                if (ok)
                    __builtin_amdgcn_global_load_lds(
                        (const __attribute__((address_space(1))) void *)((const uint16_t *)a.v_data + src),
                        (__attribute__((address_space(3))) void *)dst, 16, 0, 0);
                else
                    *(u32x4 *)(dst + lane * 16) = u32x4{0, 0, 0, 0};
            } else {
                *(u32x4 *)(dst + lane * 16) =
                    ok ? load8_bf16<KVT>(a.v_data, src) : u32x4{0, 0, 0, 0};
            }
        }
        if constexpr (KVT == NBX_BF16)
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // V tile landed in LDS

        float sc[2][4];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
                acc = mfma_bf16(kr[t][kk], qb[kk], acc);
            const bool tv = (t ? page1 : page0) >= 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int pos = p0 + 16 * t + 4 * g + i;
                sc[t][i] = (tv && pos < e_j) ? acc[i] * scale2 : -INFINITY;
            }
        }
        u32x4 ph, pl;
        softmax_step<DT, PVS>(sc, m_run, l_run, o, ph, pl);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const u32x4 va = lds_vt_operand_swz<D>(vt, dt, lane);
            o[dt] = mfma_bf16(va, ph, o[dt]);
            if constexpr (PVS)
                o[dt] = mfma_bf16(va, pl, o[dt]);
        }
    }

    l_run = xor_sum16_32(l_run);
    const float vs = a.v_scale;
    if constexpr (PG == 1) {
        if (j < M) {
            const int64_t row = row_base + j;
            float *op = a.o_part + (row * a.n_split + s) * D;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                *(f32x4 *)(op + dt * 16 + 4 * g) = o[dt] * vs;
            if (g == 0) {
                a.m_part[row * a.n_split + s] = m_run == -INFINITY ? -INFINITY : m_run * kLn2;
                a.l_part[row * a.n_split + s] = l_run;
            }
        }
    } else {
        __syncthreads();                       // every wave is done with its V tile
        float *cmb_o = (float *)smem;
        if (g == 0) {
            cmb_m[w][j] = m_run;
            cmb_l[w][j] = l_run;
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
            *(f32x4 *)(cmb_o + (w * 16 + j) * D + dt * 16 + 4 * g) = o[dt] * vs;
        __syncthreads();
        for (int idx = threadIdx.x; idx < M * D; idx += PG * 64) {
            const int r = idx / D, e = idx % D;
            float mx = -INFINITY;
#pragma unroll
            for (int k = 0; k < PG; ++k)
                mx = fmaxf(mx, cmb_m[k][r]);
            float ov = 0.0f, lv = 0.0f;
            if (mx != -INFINITY) {
#pragma unroll
                for (int k = 0; k < PG; ++k) {
                    const float mk = cmb_m[k][r];
                    if (mk == -INFINITY)
                        continue;
                    const float f = fast_exp2(mk - mx);
                    ov = fmaf(f, cmb_o[(k * 16 + r) * D + e], ov);
                    lv = fmaf(f, cmb_l[k][r], lv);
                }
            }
            const int64_t row = row_base + r;
            a.o_part[(row * a.n_split + s) * D + e] = ov;
            if (e == 0) {
                a.m_part[row * a.n_split + s] = mx == -INFINITY ? -INFINITY : mx * kLn2;
                a.l_part[row * a.n_split + s] = lv;
            }
        }
    }
}

// ------------------------------------------------------------------ multi-row

template <int D, int KVT, bool PVS, int RW, int NT>
__global__ void __launch_bounds__(RW * 64)
multirow_mfma_kernel(PartialArgs a, int row_blocks)
{
    constexpr int KK = D / 32, DT = D / 16, UPR = D / 8;
    constexpr int NTHR = RW * 64;
    constexpr int UNITS = kChunk * UPR;                 // 8-element units per tile
    constexpr int UPT = (UNITS + NTHR - 1) / NTHR;      // units per thread
    constexpr int KRS = 2 * D;                          // K tile row stride (bytes)
    constexpr int VRS = 2 * D + 16;                     // V tile row stride (bytes)
    constexpr int SWZ = (UPR < 16 ? UPR : 16) - 1;      // XOR mask on the 16-byte unit
    constexpr int R = RW * NT * 16;                     // rows per workgroup
    __shared__ __attribute__((aligned(16))) uint8_t k_lds[kChunk * KRS];
    __shared__ __attribute__((aligned(16))) uint8_t v_lds[kChunk * VRS];

    const uint32_t id = xcd_contiguous_id(blockIdx.x, gridDim.x);
    const int rb = (int)(id % (uint32_t)row_blocks);
    const int rest = (int)(id / (uint32_t)row_blocks);
    const int s = rest % a.n_split;
    const int bg = rest / a.n_split;
    const int b = bg / a.kv_heads, gk = bg % a.kv_heads;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int g = lane >> 4, j = lane & 15;
    const int M = a.rows_per_kv;
    const int row_lo = rb * R, row_hi = min(M, row_lo + R);
    const int64_t row_base = ((int64_t)b * a.q_heads + (int64_t)gk * a.group) * a.q_rows;
    const bool lead = threadIdx.x == 0;

    const int L = clamp_len(a, b, lead && s == 0 && rb == 0);
    if (lead && rb == 0 && s == a.n_split - 1 && L > a.n_split * a.split_size)
        flag_error(a.dev_err, NBX_DEVERR_SEQ_RANGE);

    int n_row[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const int m = row_lo + (w * NT + n) * 16 + j;
        int nn = 0;
        if (m < row_hi) {
            nn = a.causal ? L - a.q_rows + (m % a.q_rows) + 1 : L;
            nn = nn < 0 ? 0 : nn;
        }
        n_row[n] = nn;
    }
    int n_max = L;
    if (a.causal) {
        n_max = 0;
        for (int m = row_lo; m < row_hi && m < row_lo + a.q_rows; ++m)
            n_max = max(n_max, L - a.q_rows + (m % a.q_rows) + 1);
    }
    const int j0 = s * a.split_size;
    const int jend = min(j0 + a.split_size, n_max);
    const int nchunk = jend > j0 ? (jend - j0 + kChunk - 1) / kChunk : 0;

    u32x4 qb[NT][KK];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const int m = row_lo + (w * NT + n) * 16 + j;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
            qb[n][kk] = m < row_hi ? *(const u32x4 *)((const uint16_t *)a.q + (row_base + m) * D +
                                                      kk * 32 + g * 8)
                                   : u32x4{0, 0, 0, 0};
    }
    const float scale2 = a.scale * a.k_scale * kLog2e;
    float m_run[NT], l_run[NT];
    f32x4 o[NT][DT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        m_run[n] = -INFINITY;
        l_run[n] = 0.0f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
            o[n][dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }

    u32x4 kr[UPT], vr[UPT];
    bool tv_next[2] = {false, false};
    auto gload = [&](int c) {
        const int p0 = j0 + c * kChunk;
        int64_t kb[2], vb[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int ts = p0 + 16 * t;
            const int page = tile_page(a, b, ts, jend, lead);
            tv_next[t] = page >= 0;
            const int64_t off = (int64_t)(ts % a.page_tokens);
            kb[t] = (int64_t)page * a.k_stride_page + (int64_t)gk * a.k_stride_head +
                    off * a.k_stride_token;
            vb[t] = (int64_t)page * a.v_stride_page + (int64_t)gk * a.v_stride_head +
                    off * a.v_stride_token;
        }
#pragma unroll
        for (int i = 0; i < UPT; ++i) {
            const int u = i * NTHR + (int)threadIdx.x;
            const int pr = u / UPR, c8 = u % UPR, t = (pr >> 4) & 1;
            const bool in = u < UNITS && tv_next[t];
            kr[i] = in ? load8_bf16<KVT>(a.k_data, kb[t] + (pr & 15) * a.k_stride_token + c8 * 8)
                       : u32x4{0, 0, 0, 0};
            vr[i] = (in && p0 + pr < jend)
                        ? load8_bf16<KVT>(a.v_data, vb[t] + (pr & 15) * a.v_stride_token + c8 * 8)
                        : u32x4{0, 0, 0, 0};
        }
    };

    if (nchunk > 0)
        gload(0);
    for (int c = 0; c < nchunk; ++c) {
        const bool tv[2] = {tv_next[0], tv_next[1]};
#pragma unroll
        for (int i = 0; i < UPT; ++i) {
            const int u = i * NTHR + (int)threadIdx.x;
            if (u < UNITS) {
                const int pr = u / UPR, c8 = u % UPR;
                *(u32x4 *)(k_lds + pr * KRS + ((c8 ^ (pr & SWZ)) * 16)) = kr[i];
                *(u32x4 *)(v_lds + pr * VRS + c8 * 16) = vr[i];
            }
        }
        __syncthreads();
        if (c + 1 < nchunk)
            gload(c + 1);                  // in flight while this chunk is computed
        const int p0 = j0 + c * kChunk;
        f32x4 acc[NT][2];
#pragma unroll
        for (int n = 0; n < NT; ++n)
            acc[n][0] = acc[n][1] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                const int pr = 16 * t + j;
                const u32x4 ka =
                    *(const u32x4 *)(k_lds + pr * KRS + (((kk * 4 + g) ^ (pr & SWZ)) * 16));
#pragma unroll
                for (int n = 0; n < NT; ++n)
                    acc[n][t] = mfma_bf16(ka, qb[n][kk], acc[n][t]);
            }
        u32x4 ph[NT], pl[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            const int e_n = min(jend, n_row[n]);
            float sc[2][4];
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int pos = p0 + 16 * t + 4 * g + i;
                    sc[t][i] = (tv[t] && pos < e_n) ? acc[n][t][i] * scale2 : -INFINITY;
                }
            softmax_step<DT, PVS>(sc, m_run[n], l_run[n], o[n], ph[n], pl[n]);
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const u32x4 va = lds_vt_operand(v_lds, VRS, dt * 16, lane);
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                o[n][dt] = mfma_bf16(va, ph[n], o[n][dt]);
                if constexpr (PVS)
                    o[n][dt] = mfma_bf16(va, pl[n], o[n][dt]);
            }
        }
        __syncthreads();                   // the tiles are rewritten next iteration
    }

    const float vs = a.v_scale;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const float lt = xor_sum16_32(l_run[n]);
        const int m = row_lo + (w * NT + n) * 16 + j;
        if (m < row_hi) {
            const int64_t row = row_base + m;
            float *op = a.o_part + (row * a.n_split + s) * D;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                *(f32x4 *)(op + dt * 16 + 4 * g) = o[n][dt] * vs;
            if (g == 0) {
                a.m_part[row * a.n_split + s] = m_run[n] == -INFINITY ? -INFINITY : m_run[n] * kLn2;
                a.l_part[row * a.n_split + s] = lt;
            }
        }
    }
}

// ------------------------------------------------------------------ dispatch

template <int D, int KVT, bool PVS>
hipError_t launch_kind(const PartialArgs &a, hipStream_t stream)
{
    const int M = a.rows_per_kv;
    if (M <= 16) {
        // waves per (split, head): enough to keep each wave's run of chunks short
        const int chunks = (a.split_size + kChunk - 1) / kChunk;
        dim3 grid(a.n_split, a.batch * a.kv_heads);
        if (chunks >= 16)
            hipLaunchKernelGGL((decode_mfma_kernel<D, KVT, PVS, 4>), grid, dim3(256), 0, stream, a);
        else if (chunks >= 4)
            hipLaunchKernelGGL((decode_mfma_kernel<D, KVT, PVS, 2>), grid, dim3(128), 0, stream, a);
        else
            hipLaunchKernelGGL((decode_mfma_kernel<D, KVT, PVS, 1>), grid, dim3(64), 0, stream, a);
        return hipGetLastError();
    }
    const int64_t heads = (int64_t)a.batch * a.kv_heads * a.n_split;
#define NBX_MULTIROW(RW_, NT_)                                                              \
    do {                                                                                    \
        const int rows_per_block = (RW_) * (NT_) * 16;                                      \
        const int row_blocks = (M + rows_per_block - 1) / rows_per_block;                   \
        const int64_t blocks = heads * row_blocks;                                          \
        if (blocks > 0x7FFFFFFF)                                                            \
            return hipErrorInvalidConfiguration;                                            \
        hipLaunchKernelGGL((multirow_mfma_kernel<D, KVT, PVS, RW_, NT_>), dim3((unsigned)blocks), \
                           dim3((RW_) * 64), 0, stream, a, row_blocks);                     \
    } while (0)
    if (M % 96 == 0)
        NBX_MULTIROW(6, 1);
    else if (M <= 64)
        NBX_MULTIROW(4, 1);
    else
        NBX_MULTIROW(4, 2);
#undef NBX_MULTIROW
    return hipGetLastError();
}

template <int KVT, bool PVS>
hipError_t launch_d(const PartialArgs &a, hipStream_t stream)
{
    switch (a.head_dim) {
    case 64: return launch_kind<64, KVT, PVS>(a, stream);
    case 128: return launch_kind<128, KVT, PVS>(a, stream);
    default: return launch_kind<256, KVT, PVS>(a, stream);
    }
}

}  // namespace

hipError_t launch_partial_mfma(const PartialArgs &a, hipStream_t stream)
{
    // bf16 pools carry P as hi + lo parts; fp8 pools (tolerance set by their
    // 3-bit mantissa) use the bf16-rounded P alone
    if (a.kv_dtype == NBX_BF16)
        return launch_d<NBX_BF16, true>(a, stream);
    return launch_d<NBX_FP8_E4M3, false>(a, stream);
}

}  // namespace nbx
