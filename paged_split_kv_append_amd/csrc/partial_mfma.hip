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
// the softmax bookkeeping never leaves the lane's row.  D is the q/k head dim
// and DV the V head dim (the width of o; they differ for latent-attention
// heads, e.g. 192 / 128).  bf16 K/V products are
// exact; P is rounded to bf16 for the P V product, and for bf16 pools the
// rounding residual is multiplied in a second MFMA (P = hi + lo, relative
// error about 2^-17).  fp8 codes are widened to bf16 exactly; the K scale is
// folded into the score scale and the V scale into the stored o.  Scores are
// kept in log2 units (scale * log2 e folded in); m is stored in natural units.
//
// Memory path.  A 32-position chunk is two 16-position tiles; a tile never
// straddles a page (page sizes are multiples of 16 and splits start on tile
// boundaries), so each tile is one buffer descriptor: base = the tile's first
// row, range = the rows that hold data (0 for an unmapped page).  Lanes carry
// fixed 32-bit offsets; out-of-range lanes read zeros and touch no memory.
// V tiles are staged in LDS column-blocked: for each 16-column slice, the 16
// rows x 32 bytes of a tile are one contiguous 512-byte block.  One 64-lane
// 16-byte load (one row slice per lane pair) fills two such blocks, and the
// LDS transpose read of a slice
// (lane 16 g + j: row 4 g + j/4, 8 bytes at column 4 (j % 4)) touches 512
// consecutive bytes, so it is free of bank conflicts and every slice is a
// constant offset from one per-lane address.  Page ids come from the block
// table once per 32 chunks (one per lane) and are broadcast with readlane.
//
// Three kernels:
//  - decode_persistent_kernel: at most 16 rows per KV head (decode, short
//    windows) and at most 256 sequences; one wave per (sequence, split, KV
//    head) item, as many waves as the device holds, items enumerated on the
//    device, the step's append fused in (described at the kernel).
//  - decode_mfma_kernel: the same rows for larger batches.  PG waves per
//    (split, sequence x KV head) take interleaved chunks of the split, each
//    with its own (m, l, O), combined in a fixed order at the end.
//    In both decode kernels K rows go from HBM straight into MFMA operand
//    registers; V rows are loaded into registers and written to the wave's
//    LDS tile once they land (fp8 codes widened on the way).  The wave's next
//    chunk is loaded while the current one is computed.
//  - multirow_mfma_kernel: more rows per KV head (verify windows, prompt
//    chunks).  A workgroup takes RW x NT row tiles of 16 rows; its waves share
//    the loads of each K and V chunk and stage it in LDS (K column-blocked by
//    64 bytes, which makes the operand reads conflict-free too); the next
//    chunk is in registers while the current one is computed.
//    Workgroups are ordered row block fastest and mapped so that the row
//    blocks of one split run on the same XCD and share its L2 (the rows-first
//    order of TensorFold PR #1219, made XCD-aware).
// The persistent and multi-row kernels also take the fixed-shift softmax
// when both pools carry per-page bounds (see "fixed shift" below).
#include <atomic>

#include "kernels.h"
#include "mfma_common.h"

namespace nbx {

namespace {

constexpr int kChunk = 32;   // positions per chunk: two 16-position tiles, one PV k-step

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

// Lane i of the result: page of tile (i & 1) of chunk c0 + (i / 2) * cstep,
// -1 past the split.  Refreshed once per 32 chunks of a wave.
__device__ __forceinline__ int chunk_pages(const PartialArgs &a, int b, int j0, int jend,
                                           int nchunk, int c0, int cstep, int lane, bool flag_it)
{
    const int cq = c0 + (lane >> 1) * cstep;
    const int ts = j0 + cq * kChunk + 16 * (lane & 1);
    return cq < nchunk ? tile_page(a, b, ts, jend, flag_it) : -1;
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
// masked).  Updates m, l, rescales o and returns the P operands of the k-steps
// (hi and residual lo parts).
template <int DT, bool PVS, int NK>
__device__ __forceinline__ void softmax_step_n(float (&sc)[2 * NK][4], float &m_run, float &l_run,
                                               f32x4 (&o)[DT], u32x4 (&ph)[NK], u32x4 (&pl)[NK])
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
    if (__any(corr != 1.0f)) {             // a row's max moved: rescale (else o * 1 = o)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
            o[dt] *= corr;
    }
#pragma unroll
    for (int k = 0; k < NK; ++k)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int t = 2 * k + u;
            ph[k][2 * u] = pack_bf16(p[t][0], p[t][1]);
            ph[k][2 * u + 1] = pack_bf16(p[t][2], p[t][3]);
            if constexpr (PVS) {
                pl[k][2 * u] =
                    pack_bf16(p[t][0] - bf16_round(p[t][0]), p[t][1] - bf16_round(p[t][1]));
                pl[k][2 * u + 1] =
                    pack_bf16(p[t][2] - bf16_round(p[t][2]), p[t][3] - bf16_round(p[t][3]));
            }
        }
}

// Online-softmax step for one lane's row over the 32 positions of a chunk
// (softmax_step_n with one k-step): returns the P operand (hi and residual lo).
template <int DT, bool PVS>
__device__ __forceinline__ void softmax_step(float (&sc)[2][4], float &m_run, float &l_run,
                                             f32x4 (&o)[DT], u32x4 &ph, u32x4 &pl)
{
    u32x4 ph1[1], pl1[1];
    softmax_step_n<DT, PVS, 1>(sc, m_run, l_run, o, ph1, pl1);
    ph = ph1[0];
    pl = pl1[0];
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
            ph[k][2 * u] = pack_bf16(p[t][0], p[t][1]);
            ph[k][2 * u + 1] = pack_bf16(p[t][2], p[t][3]);
            if constexpr (PVS) {
                pl[k][2 * u] =
                    pack_bf16(p[t][0] - bf16_round(p[t][0]), p[t][1] - bf16_round(p[t][1]));
                pl[k][2 * u + 1] =
                    pack_bf16(p[t][2] - bf16_round(p[t][2]), p[t][3] - bf16_round(p[t][3]));
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

// ------------------------------------------------------------------ decode

template <int D, int DV, int KVT, bool PVS, int PG>
__global__ void __launch_bounds__(PG * 64)
decode_mfma_kernel(PartialArgs a)
{
    constexpr int KK = D / 32;                 // 32-wide k-steps of Q K^T
    constexpr int DT = DV / 16;                // 16-column slices of V and O
    constexpr bool BF = KVT == NBX_BF16;
    constexpr int ESZ = BF ? 2 : 1;
    constexpr int VBYTES = kChunk * 2 * DV;    // one chunk of V as bf16
    constexpr int CMB = PG > 1 ? PG * 16 * DV * 4 : 0;
    constexpr int SMEM = (PG * VBYTES > CMB) ? PG * VBYTES : CMB;
    __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];
    __shared__ float cmb_m[PG][16], cmb_l[PG][16];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave index, uniform
    const int g = lane >> 4, j = lane & 15;
    // (sequence x KV head) is the fastest index: consecutive workgroups go to
    // different XCDs, so each XCD gets every split of an equal share of heads
    const int heads = a.batch * a.kv_heads;
    const int s = (int)(blockIdx.x / (uint32_t)heads);
    const int bg = (int)(blockIdx.x % (uint32_t)heads);
    const int b = bg / a.kv_heads, gk = bg % a.kv_heads;
    const int M = a.rows_per_kv;
    const int64_t row_base = ((int64_t)b * a.q_heads + (int64_t)gk * a.group) * a.q_rows;
    const bool lead = threadIdx.x == 0;

    const int S = device_split_size(a);
    const int L = clamp_len(a, b, lead && s == 0);
    if (lead && s == a.n_split - 1 && L > a.n_split * S)
        flag_error(a.dev_err, NBX_DEVERR_SEQ_RANGE);

    const int wb = seq_window(a, b, lead && s == 0);
    const int n_j = j < M ? row_keys(a, L, wb, j % a.q_rows) : 0;
    const int n_max = seq_keys(L, wb);
    const int j0 = s * S;
    const int jend = min(j0 + S, n_max);
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

    const int64_t k_head = (int64_t)gk * a.k_stride_head;
    const int64_t v_head = (int64_t)gk * a.v_stride_head;
    const int kst_b = (int)(a.k_stride_token * ESZ), vst_b = (int)(a.v_stride_token * ESZ);
    // fixed per-lane byte offsets inside a tile
    const int k_lane = j * kst_b + g * 8 * ESZ;                        // + kk * 32 * ESZ
    const int v_lane = ((lane & 31) >> 1) * vst_b + ((lane >> 5) * 16 + (lane & 1) * 8) * ESZ;
    uint8_t *const tile = smem + w * VBYTES;
    const uint8_t *vt_lane = tile + (4 * g + (j >> 2)) * 32 + (j & 3) * 8;

    // Software pipeline over this wave's chunks c = w, w + PG, ...:
    //   V(c) lands in LDS; V(c') is issued (c' the next chunk);
    //   S = K(c) Q^T from registers; K(c') is issued;
    //   softmax; O += P V(c) from LDS.
    // One register set each for K and V: a chunk's loads are in flight while
    // the previous chunk is computed.  The compiler places the waits.
    int pg_reg = -1;
    typename KvRaw<KVT>::type kr[2][KK];       // K as loaded; widened at its use
    u32x4 vr[BF ? DT : 1];
    u32x2 vraw[BF ? 1 : DT];                   // fp8: V codes awaiting widening
    auto pages_of = [&](int q, int &pg0, int &pg1) {
        pg0 = __builtin_amdgcn_readlane(pg_reg, 2 * (q & 31));
        pg1 = __builtin_amdgcn_readlane(pg_reg, 2 * (q & 31) + 1);
    };
    auto issue_v = [&](int c, int pg0, int pg1) {
        const int p0 = j0 + c * kChunk;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int ts = p0 + 16 * t;
            // rows past the data fall outside the range and read as 0
            const i32x4 rv = tile_rsrc<ESZ>(a.v_data, a.v_stride_page, v_head, a.v_stride_token,
                                            a.page_tokens, t ? pg1 : pg0, ts, min(16, jend - ts));
#pragma unroll
            for (int k = 0; k < DT / 2; ++k) {
                const int i = t * (DT / 2) + k;
                if constexpr (BF)
                    vr[i] = nbx_buffer_load_b128(rv, v_lane + k * 64, 0, 0);
                else
                    vraw[i] = nbx_buffer_load_b64(rv, v_lane + k * 32, 0, 0);
            }
        }
    };
    auto issue_k = [&](int c, int pg0, int pg1) {
        const int p0 = j0 + c * kChunk;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const i32x4 rk = tile_rsrc<ESZ>(a.k_data, a.k_stride_page, k_head, a.k_stride_token,
                                            a.page_tokens, t ? pg1 : pg0, p0 + 16 * t, 16);
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
                kr[t][kk] = buffer_load8_raw<KVT>(rk, k_lane + kk * 32 * ESZ);
        }
    };
    auto land_v = [&]() {
#pragma unroll
        for (int i = 0; i < DT; ++i) {
            const int t = i / (DT / 2), k = i % (DT / 2);
            u32x4 v;
            if constexpr (BF)
                v = vr[i];
            else
                v = widen8_e4m3(vraw[i]);
            *(u32x4 *)(tile + t * DT * 512 + k * 1024 + lane * 16) = v;
        }
    };

    int q = 0, c = w;
    if (c < nchunk) {
        pg_reg = chunk_pages(a, b, j0, jend, nchunk, c, PG, lane, true);
        int pg0, pg1;
        pages_of(0, pg0, pg1);
        issue_v(c, pg0, pg1);
        issue_k(c, pg0, pg1);
        for (;;) {
            const int cn = c + PG;
            const bool more = cn < nchunk;
            const int p0 = j0 + c * kChunk;
            const int cur0 = pg0, cur1 = pg1;
            land_v();                          // this wave's DS operations run in order
            if (more) {
                if (((q + 1) & 31) == 0)
                    pg_reg = chunk_pages(a, b, j0, jend, nchunk, cn, PG, lane, true);
                pages_of(q + 1, pg0, pg1);
                issue_v(cn, pg0, pg1);
            }
            float sc[2][4];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int kk = 0; kk < KK; ++kk)
                    acc = mfma_bf16(as_bf16x8<KVT>(kr[t][kk]), qb[kk], acc);
                const bool tv = (t ? cur1 : cur0) >= 0;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int pos = p0 + 16 * t + 4 * g + i;
                    sc[t][i] = (tv && pos < e_j) ? acc[i] * scale2 : -INFINITY;
                }
            }
            if (more)
                issue_k(cn, pg0, pg1);
            u32x4 ph, pl;
            softmax_step<DT, PVS>(sc, m_run, l_run, o, ph, pl);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const u32x4 va = vt_operand<DT>(vt_lane, dt);
                o[dt] = mfma_bf16(va, ph, o[dt]);
                if constexpr (PVS)
                    o[dt] = mfma_bf16(va, pl, o[dt]);
            }
            ++q;
            c = cn;
            if (!more)
                break;
        }
    }

    l_run = xor_sum16_32(l_run);
    const float vs = a.v_scale;
    if constexpr (PG == 1) {
        if (j < M) {
            const int64_t row = row_base + j;
            float *op = a.o_part + (row * a.n_split + s) * DV;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                *(f32x4 *)(op + dt * 16 + 4 * g) = o[dt] * vs;
            if (g == 0) {
                a.m_part[row * a.n_split + s] = m_run == -INFINITY ? -INFINITY : m_run * kLn2;
                a.l_part[row * a.n_split + s] = l_run;
            }
        }
    } else {
        __syncthreads();                       // every wave is done with its V tiles
        float *cmb_o = (float *)smem;
        if (g == 0) {
            cmb_m[w][j] = m_run;
            cmb_l[w][j] = l_run;
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
            *(f32x4 *)(cmb_o + (w * 16 + j) * DV + dt * 16 + 4 * g) = o[dt] * vs;
        __syncthreads();
        for (int idx = threadIdx.x; idx < M * DV; idx += PG * 64) {
            const int r = idx / DV, e = idx % DV;
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
                    ov = fmaf(f, cmb_o[(k * 16 + r) * DV + e], ov);
                    lv = fmaf(f, cmb_l[k][r], lv);
                }
            }
            const int64_t row = row_base + r;
            a.o_part[(row * a.n_split + s) * DV + e] = ov;
            if (e == 0) {
                a.m_part[row * a.n_split + s] = mx == -INFINITY ? -INFINITY : mx * kLn2;
                a.l_part[row * a.n_split + s] = lv;
            }
        }
    }
}

// ------------------------------------------------------------------ persistent decode

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

constexpr int kPersistMaxBatch = 256;      // sequences covered by the lane-register item table

// One wave per work item = (sequence b, split s, KV head g) with keys in the
// split.  The grid is sized to the waves the GPU can hold; items are numbered
// on the device from seq_lens (sequence-major, empty splits never numbered)
// and dealt out evenly: wave w takes items w, w + W', w + 2 W', ... where W'
// is the smallest wave count that gives every wave the same number of items.
// Each wave streams the chunks of its items back to back, with the next
// chunk's loads (and, one chunk ahead of an item boundary, the next item's Q
// and page ids) in flight while the current chunk is computed, so the cost of
// starting a wave is paid once, not once per split.  Splits without keys get
// m = -inf and l = 0; their o is not written.  BND: a pool carries bounds
// (raised by the fused append; with both, the fixed-shift softmax), a
// separate instantiation so that the plain kernel keeps its registers; at
// D = 128 it is held to 2 waves per SIMD like the plain one (it fits 256
// registers without spilling; left to itself the compiler takes one more
// AGPR block and halves the resident waves).
template <int D, int DV, int KVT, bool PVS, int NB, bool FA, bool BND>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu((BND && D == 128) ? 2 : 1)))
decode_persistent_kernel(PartialArgs a)
{
    constexpr int KK = D / 32, DT = DV / 16;
    constexpr bool BF = KVT == NBX_BF16;
    constexpr int ESZ = BF ? 2 : 1;
    constexpr int VBYTES = kChunk * 2 * DV;
    __shared__ __attribute__((aligned(16))) uint8_t tile[VBYTES];

    const int lane = threadIdx.x;
    const int g = lane >> 4, j = lane & 15;
    const int wv = blockIdx.x, W = gridDim.x;
    const int M = a.rows_per_kv, H = a.kv_heads, NS = a.n_split;
    const int cap = a.max_pages * a.page_tokens;

    // sequence table, lane l of block t describing b = 64 t + l: clamped
    // length, splits holding keys, inclusive prefix of item counts
    int Lr[NB], Wr[NB], nsr[NB], incl[NB];
    int longest = 1;
#pragma unroll
    for (int t = 0; t < NB; ++t) {
        const int b = 64 * t + lane;
        int L = 0;
        if (b < a.batch) {
            L = a.seq_lens[b];
            if (L < 0 || L > cap) {
                if (wv == 0)
                    flag_error(a.dev_err, NBX_DEVERR_SEQ_RANGE);
                L = L < 0 ? 0 : cap;
            }
        }
        Lr[t] = L;
        Wr[t] = b < a.batch ? seq_window(a, b, wv == 0) : 0;
        longest = max(longest, L);
    }
    // positions per split: the caller's, or (split_size == 0) derived from the
    // longest device length as device_split_size does
    int S = a.split_size;
    if (S == 0) {
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1)
            longest = max(longest, __shfl_xor(longest, off, 64));
        S = ((longest + NS - 1) / NS + 15) / 16 * 16;
    }
    int carry = 0;
#pragma unroll
    for (int t = 0; t < NB; ++t) {
        const int b = 64 * t + lane;
        const int L = Lr[t];
        if (wv == 0 && b < a.batch && (L > NS * S || (FA && L < a.n_new)))
            flag_error(a.dev_err, NBX_DEVERR_SEQ_RANGE);
        const int nmax = seq_keys(L, Wr[t]);
        const int ns = b < a.batch ? min((nmax + S - 1) / S, NS) : 0;
        int x = ns * H;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(x, off, 64);
            if (lane >= off)
                x += y;
        }
        nsr[t] = ns;
        incl[t] = carry + x;
        carry = __shfl(incl[t], 63, 64);
    }
    const int N = carry;
    auto lane_val = [&](const int (&arr)[NB], int b) {
        int v = arr[0];
#pragma unroll
        for (int t = 1; t < NB; ++t)
            v = (b >> 6) == t ? arr[t] : v;
        return __builtin_amdgcn_readlane(v, b & 63);
    };

    // splits without keys: m = -inf, l = 0 for their rows
    {
        const int per_b = NS * H, pairs = a.batch * per_b;
        for (int pi = wv; pi < pairs; pi += W) {
            const int b = pi / per_b, rem = pi - b * per_b, s = rem / H, gk = rem - s * H;
            if (s >= lane_val(nsr, b) && lane < M) {
                const int64_t row =
                    ((int64_t)b * a.q_heads + (int64_t)gk * a.group) * a.q_rows + lane;
                a.m_part[row * NS + s] = -INFINITY;
                a.l_part[row * NS + s] = 0.0f;
            }
        }
    }
    if (N == 0)
        return;
    const int k_per = (N + W - 1) / W;
    const int W_eff = (N + k_per - 1) / k_per;
    if (wv >= W_eff)
        return;

    struct Item {
        int b, gk, s, j0, jend, e_j, nchunk, L;
        int64_t row_base;
        float kb, vb;                          // K norm / V magnitude bounds of its pages
    };
    // fixed-shift softmax: both pools carry per-page bounds
    const bool use_bounds = BND && a.k_bounds != nullptr && a.v_bounds != nullptr;
    auto make_item = [&](int k) {
        Item it;
        int before = 0;                        // sequences whose items all precede k
#pragma unroll
        for (int t = 0; t < NB; ++t)
            before += __popcll(__ballot(incl[t] <= k));
        it.b = before;
        const int excl = lane_val(incl, it.b) - lane_val(nsr, it.b) * H;
        const int r = k - excl;
        it.s = r / H;
        it.gk = r - it.s * H;
        const int L = lane_val(Lr, it.b), wb = lane_val(Wr, it.b);
        it.j0 = it.s * S;
        it.jend = min(it.j0 + S, seq_keys(L, wb));
        it.nchunk = (it.jend - it.j0 + kChunk - 1) / kChunk;
        const int n_j = j < M ? row_keys(a, L, wb, j % a.q_rows) : 0;
        it.e_j = min(it.jend, n_j);
        it.row_base = ((int64_t)it.b * a.q_heads + (int64_t)it.gk * a.group) * a.q_rows;
        it.L = L;
        it.kb = it.vb = 0.0f;
        if (use_bounds) {                      // the bounds of the pages the item reads
            const int T = a.page_tokens;
            for (int pi = it.j0 / T + lane; pi <= (it.jend - 1) / T; pi += 64) {
                const int page = a.block_table[(int64_t)it.b * a.max_pages + pi];
                if (page >= 0 && page < a.num_pages) {
                    it.kb = bound_max(it.kb, a.k_bounds[(int64_t)page * H + it.gk]);
                    it.vb = bound_max(it.vb, a.v_bounds[(int64_t)page * H + it.gk]);
                }
            }
            it.kb = group_bound_max<64>(it.kb);
            it.vb = group_bound_max<64>(it.vb);
        }
        return it;
    };
    // Fused append: the new positions L - n_new .. L - 1 that fall in the item
    // are written to the pools (the conversions of the append kernel) before
    // any load of the item is issued.  Only this wave reads the item's tiles,
    // and a wave's memory operations are performed in order, so its later
    // tile loads see the new rows.
    // `pg` holds the page ids of the item's first 32 chunks (item_pages(it, 0)).
    // With bounds, each written row raises its page's bound and the item's.
    auto append_item = [&](Item &it, int pg) {
        if constexpr (FA) {
            const int first = it.L - a.n_new;
            const int lo = max(it.j0, max(first, 0)), hi = min(it.j0 + S, it.L);
            for (int p = lo; p < hi; ++p) {
                const int tl = (p - it.j0) >> 4;           // tile of p within the item
                const int page = tl < 64 ? __builtin_amdgcn_readlane(pg, tl)
                                         : tile_page(a, it.b, p, hi, lane == 0);
                if (page < 0)
                    continue;
                const int64_t src = ((int64_t)it.b * a.n_new + (p - first)) * H + it.gk;
                const int64_t r = p % a.page_tokens;
                const float ks = store_new_row<D, KVT, false>(
                    a.new_k, a.new_dtype, src * D, (void *)a.k_data,
                    (int64_t)page * a.k_stride_page + it.gk * a.k_stride_head + r * a.k_stride_token,
                    a.k_scale, lane);
                const float vs_ = store_new_row<DV, KVT, true>(
                    a.new_v, a.new_dtype, src * DV, (void *)a.v_data,
                    (int64_t)page * a.v_stride_page + it.gk * a.v_stride_head + r * a.v_stride_token,
                    a.v_scale, lane);
                if (BND && (a.k_bounds || a.v_bounds)) {
                    const float kn = sqrtf(group_sum<64>(ks)), vm = group_bound_max<64>(vs_);
                    const int64_t bi = (int64_t)page * H + it.gk;
                    if (a.k_bounds && lane == 0)
                        raise_bound(a.k_bounds, bi, kn);
                    if (a.v_bounds && lane == 0)
                        raise_bound(a.v_bounds, bi, vm);
                    it.kb = bound_max(it.kb, kn);
                    it.vb = bound_max(it.vb, vm);
                }
            }
            asm volatile("" ::: "memory");     // keep the tile loads after the stores
        }
    };
    auto load_q = [&](const Item &it, u32x4 (&qv)[KK]) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
            qv[kk] = j < M ? *(const u32x4 *)((const uint16_t *)a.q + (it.row_base + j) * D +
                                              kk * 32 + g * 8)
                           : u32x4{0, 0, 0, 0};
    };
    // lane i: page of tile (i & 1) of chunk c0 + i / 2 of the item
    auto item_pages = [&](const Item &it, int c0) {
        const int cq = c0 + (lane >> 1);
        const int ts = it.j0 + cq * kChunk + 16 * (lane & 1);
        return cq < it.nchunk ? tile_page(a, it.b, ts, it.jend, true) : -1;
    };

    const int kst_b = (int)(a.k_stride_token * ESZ), vst_b = (int)(a.v_stride_token * ESZ);
    const int k_lane = j * kst_b + g * 8 * ESZ;                        // + kk * 32 * ESZ
    const int v_lane = ((lane & 31) >> 1) * vst_b + ((lane >> 5) * 16 + (lane & 1) * 8) * ESZ;
    const uint8_t *vt_lane = tile + (4 * g + (j >> 2)) * 32 + (j & 3) * 8;
    const float scale2 = a.scale * a.k_scale * kLog2e;
    const float vs = a.v_scale;

    typename KvRaw<KVT>::type kr[2][KK];       // K as loaded; widened at its use
    u32x4 qb[KK];
    u32x4 vr[BF ? DT : 1];
    u32x2 vraw[BF ? 1 : DT];
    auto issue_v = [&](const Item &it, int c, int pg0, int pg1) {
        const int p0 = it.j0 + c * kChunk;
        const int64_t v_head = (int64_t)it.gk * a.v_stride_head;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int ts = p0 + 16 * t;
            const i32x4 rv = tile_rsrc<ESZ>(a.v_data, a.v_stride_page, v_head, a.v_stride_token,
                                            a.page_tokens, t ? pg1 : pg0, ts, min(16, it.jend - ts));
#pragma unroll
            for (int k = 0; k < DT / 2; ++k) {
                const int i = t * (DT / 2) + k;
                if constexpr (BF)
                    vr[i] = nbx_buffer_load_b128(rv, v_lane + k * 64, 0, 0);
                else
                    vraw[i] = nbx_buffer_load_b64(rv, v_lane + k * 32, 0, 0);
            }
        }
    };
    // K rows of the chunk and, with them, the item's Q rows (a few KB that stay
    // in L2): one register set each, refilled right after the scores are formed
    auto issue_k = [&](const Item &it, int c, int pg0, int pg1) {
        load_q(it, qb);
        const int p0 = it.j0 + c * kChunk;
        const int64_t k_head = (int64_t)it.gk * a.k_stride_head;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const i32x4 rk = tile_rsrc<ESZ>(a.k_data, a.k_stride_page, k_head, a.k_stride_token,
                                            a.page_tokens, t ? pg1 : pg0, p0 + 16 * t, 16);
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
                kr[t][kk] = buffer_load8_raw<KVT>(rk, k_lane + kk * 32 * ESZ);
        }
    };
    auto land_v = [&]() {
#pragma unroll
        for (int i = 0; i < DT; ++i) {
            const int t = i / (DT / 2), k = i % (DT / 2);
            u32x4 v;
            if constexpr (BF)
                v = vr[i];
            else
                v = widen8_e4m3(vraw[i]);
            *(u32x4 *)(tile + t * DT * 512 + k * 1024 + lane * 16) = v;
        }
    };

    float m_run = -INFINITY, l_run = 0.0f;
    bool fixed = false;                        // the item being computed uses a fixed shift
    float m_fix = 0.0f;                        // its shift for this lane's row (log2 units)
    f32x4 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
        o[dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    int i_item = 0;
    Item cur = make_item(wv);
    int pg_reg = item_pages(cur, 0), pg_next = -1;
    append_item(cur, pg_reg);
    Item nxt = cur;
    bool has_next = false;
    auto prepare_next = [&]() {
        const int kn = wv + (i_item + 1) * W_eff;
        has_next = i_item + 1 < k_per && kn < N;
        if (has_next) {
            nxt = make_item(kn);
            pg_next = item_pages(nxt, 0);
            append_item(nxt, pg_next);
        }
    };
    int c = 0;
    int pg0 = __builtin_amdgcn_readlane(pg_reg, 0), pg1 = __builtin_amdgcn_readlane(pg_reg, 1);
    issue_v(cur, 0, pg0, pg1);
    issue_k(cur, 0, pg0, pg1);
    if (cur.nchunk == 1)
        prepare_next();

    for (;;) {
        // the chunk to compute: (item `ci`, chunk `cc`) whose loads are in flight
        const Item ci = cur;
        const int cc = c, cpg0 = pg0, cpg1 = pg1;
        land_v();                              // DS operations of the wave run in order
        bool more = true, new_item = false;
        if (c + 1 < cur.nchunk) {
            ++c;
            if ((c & 31) == 0)
                pg_reg = item_pages(cur, c);
        } else if (has_next) {
            cur = nxt;
            ++i_item;
            c = 0;
            pg_reg = pg_next;
            new_item = true;
        } else {
            more = false;
        }
        if (more) {
            pg0 = __builtin_amdgcn_readlane(pg_reg, 2 * (c & 31));
            pg1 = __builtin_amdgcn_readlane(pg_reg, 2 * (c & 31) + 1);
            issue_v(cur, c, pg0, pg1);
        }
        const int p0 = ci.j0 + cc * kChunk;
        float sc[2][4];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
                acc = mfma_bf16(as_bf16x8<KVT>(kr[t][kk]), qb[kk], acc);
            const bool tv = (t ? cpg1 : cpg0) >= 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int pos = p0 + 16 * t + 4 * g + i;
                sc[t][i] = (tv && pos < ci.e_j) ? acc[i] * scale2 : -INFINITY;
            }
        }
        if (use_bounds && cc == 0) {           // the item's Q is still in qb
            int C, gate;
            bool ok = fixed_shift_consts(ci.L, ci.vb, vs, C, gate);
            ok = ok && fixed_shift_row(q_row_norm<KK>(qb), ci.kb, fabsf(scale2), C, gate, m_fix);
            fixed = __all(ok);
        }
        if (more) {
            issue_k(cur, c, pg0, pg1);
            if (c == cur.nchunk - 1)
                prepare_next();
        }
        u32x4 ph, pl;
        if (BND && fixed) {
            u32x4 ph1[1], pl1[1];
            softmax_fixed_n<PVS, 1>(sc, m_fix, l_run, ph1, pl1);
            ph = ph1[0];
            pl = pl1[0];
        } else {
            softmax_step<DT, PVS>(sc, m_run, l_run, o, ph, pl);
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const u32x4 va = vt_operand<DT>(vt_lane, dt);
            o[dt] = mfma_bf16(va, ph, o[dt]);
            if constexpr (PVS)
                o[dt] = mfma_bf16(va, pl, o[dt]);
        }
        if (cc == ci.nchunk - 1) {             // item done: store its partial, reset
            const float lt = xor_sum16_32(l_run);
            if (j < M) {
                const int64_t row = ci.row_base + j;
                float *op = a.o_part + (row * NS + ci.s) * DV;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
                    *(f32x4 *)(op + dt * 16 + 4 * g) = o[dt] * vs;
                if (g == 0) {
                    a.m_part[row * NS + ci.s] = stored_m(BND && fixed, m_fix, m_run, lt);
                    a.l_part[row * NS + ci.s] = lt;
                }
            }
            m_run = -INFINITY;
            l_run = 0.0f;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                o[dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
        if (!more)
            break;
    }
}

// ------------------------------------------------------------------ multi-row

// A workgroup of 8 waves takes 8 x NT row tiles of 16 rows of one (sequence,
// KV head, split).  The K and V tiles of a chunk are pieces of 1 KB (as bf16:
// 16 rows x 32 columns); waves 0-3 load the K pieces and waves 4-7 the V
// pieces, each wave all its pieces from one tile, so each of its loads has a
// fixed role (K or V, tile) and one descriptor per tile serves it.  Chunk c + 1
// waits in LDS and chunks c + 2 ... c + 1 + NSET in registers while chunk c is
// computed; one barrier per chunk.  K is stored in LDS with a 16-byte swizzle inside each 1 KB
// block (row r, piece p at unit 4 r + ((p + r / 4) & 3)), so that the 16
// lanes of a group reading one 16-byte operand piece each cover all banks.
template <int D, int DV, int KVT, bool PVS, int NT, int NK, int NSET>
__global__ void __launch_bounds__(512)
multirow_mfma_kernel(PartialArgs a, int row_blocks)
{
    constexpr int RW = 8;                      // waves per workgroup
    constexpr int CH = 32 * NK;                // positions per chunk (NK k-steps of P V)
    constexpr int TL = 2 * NK;                 // 16-position tiles per chunk
    constexpr int BATCH = 64 / TL;             // chunks whose tiles fill one lane register
    constexpr int KK = D / 32, DT = DV / 16;
    constexpr int KV = DV / 32;                // 32-column V pieces per tile
    constexpr bool BF = KVT == NBX_BF16;
    constexpr int ESZ = BF ? 2 : 1;
    constexpr int KBYTES = CH * 2 * D;         // K chunk as bf16: [tile][KK][16 rows][64 B]
    constexpr int VBYTES = CH * 2 * DV;        // V chunk as bf16: [tile][DT][16 rows][32 B]
    constexpr int BUF = KBYTES + VBYTES;
    // pieces per wave: TL x KK of K over waves 0-3, TL x KV of V over waves 4-7
    constexpr int PER_K = TL * KK / 4, PER_V = TL * KV / 4;
    constexpr int PMAX = PER_K > PER_V ? PER_K : PER_V;
    static_assert(PER_K <= KK && KK % PER_K == 0 && PER_V <= KV && KV % PER_V == 0,
                  "a wave's pieces lie in one tile");
    constexpr int R = RW * NT * 16;            // rows per workgroup
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * BUF];

    const uint32_t id = xcd_contiguous_id(blockIdx.x, gridDim.x);
    const int rb = (int)(id % (uint32_t)row_blocks);
    const int rest = (int)(id / (uint32_t)row_blocks);
    const int s = rest % a.n_split;
    const int bg = rest / a.n_split;
    const int b = bg / a.kv_heads, gk = bg % a.kv_heads;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave index, uniform
    const int g = lane >> 4, j = lane & 15;
    const int M = a.rows_per_kv;
    const int row_lo = rb * R, row_hi = min(M, row_lo + R);
    const int64_t row_base = ((int64_t)b * a.q_heads + (int64_t)gk * a.group) * a.q_rows;
    const bool lead = threadIdx.x == 0;
    // a wave whose row tiles are all past the last row loads its share only
    const bool has_rows = row_lo + w * NT * 16 < row_hi;

    const int S = device_split_size(a);
    const int L = clamp_len(a, b, lead && s == 0 && rb == 0);
    if (lead && rb == 0 && s == a.n_split - 1 && L > a.n_split * S)
        flag_error(a.dev_err, NBX_DEVERR_SEQ_RANGE);

    const int wb = seq_window(a, b, lead && s == 0 && rb == 0);
    int n_row[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const int m = row_lo + (w * NT + n) * 16 + j;
        n_row[n] = m < row_hi ? row_keys(a, L, wb, m % a.q_rows) : 0;
    }
    int n_max = 0;                             // the most keys a row of this block sees
    for (int m = row_lo; m < row_hi && m < row_lo + a.q_rows; ++m)
        n_max = max(n_max, row_keys(a, L, wb, m % a.q_rows));
    const int j0 = s * S;
    const int jend = min(j0 + S, n_max);
    const int nchunk = jend > j0 ? (jend - j0 + CH - 1) / CH : 0;

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
    // fixed-shift softmax where both pools carry bounds: per row tile, a shift
    // per row and one decision for the tile's 16 rows
    bool fixed[NT];
    float m_fix[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        fixed[n] = false;
        m_fix[n] = 0.0f;
    }
    if (a.k_bounds != nullptr && a.v_bounds != nullptr && nchunk > 0) {
        float kb = 0.0f, vb = 0.0f;
        const int T = a.page_tokens;
        for (int pi = j0 / T + lane; pi <= (jend - 1) / T; pi += 64) {
            const int page = a.block_table[(int64_t)b * a.max_pages + pi];
            if (page >= 0 && page < a.num_pages) {
                kb = bound_max(kb, a.k_bounds[(int64_t)page * a.kv_heads + gk]);
                vb = bound_max(vb, a.v_bounds[(int64_t)page * a.kv_heads + gk]);
            }
        }
        kb = group_bound_max<64>(kb);
        vb = group_bound_max<64>(vb);
        int C, gate;
        if (fixed_shift_consts(L, vb, a.v_scale, C, gate)) {
#pragma unroll
            for (int n = 0; n < NT; ++n)
                fixed[n] = __all(fixed_shift_row(q_row_norm<KK>(qb[n]), kb, fabsf(scale2), C, gate,
                                                 m_fix[n]));
        }
    }

    const int64_t k_head = (int64_t)gk * a.k_stride_head;
    const int64_t v_head = (int64_t)gk * a.v_stride_head;
    const int kst_b = (int)(a.k_stride_token * ESZ), vst_b = (int)(a.v_stride_token * ESZ);
    // fixed per-lane byte offsets of the 64-lane piece loads
    const int k_lane = (lane >> 2) * kst_b + (lane & 3) * 8 * ESZ;   // + kk * 32 * ESZ
    const int v_lane = ((lane & 31) >> 1) * vst_b + ((lane >> 5) * 16 + (lane & 1) * 8) * ESZ;
    // LDS: swizzled K store of this lane (row lane / 4, piece lane % 4) and
    // read of operand piece g of row j; transposed V read
    const int k_st = (4 * (lane >> 2) + (((lane & 3) + (lane >> 4)) & 3)) * 16;
    const uint8_t *k_rd = smem + (4 * j + ((g + (j >> 2)) & 3)) * 16;   // + (t*KK + kk) * 1024
    const uint8_t *vt_lane = smem + KBYTES + (4 * g + (j >> 2)) * 32 + (j & 3) * 8;

    // Wave roles: waves 0-3 load K, 4-7 load V; of the pieces of its pool
    // (tile-major: K 32-column groups kk, V 32-column pairs of 16-column
    // slices) wave w takes (w & 3) * per ... (w & 3) * per + per - 1, all in
    // tile t_w of every chunk.
    const bool is_k = w < 4;
    const int per = is_k ? PER_K : PER_V, pieces = is_k ? KK : KV;
    const int t_w = ((w & 3) * per) / pieces, pbase = ((w & 3) * per) % pieces;
    const uint8_t *role_base = is_k ? (const uint8_t *)a.k_data + k_head * ESZ
                                    : (const uint8_t *)a.v_data + v_head * ESZ;
    const int64_t role_sp = (is_k ? a.k_stride_page : a.v_stride_page) * ESZ;
    const int role_st = is_k ? kst_b : vst_b;
    const int role_lane = (is_k ? k_lane : v_lane) + pbase * 32 * ESZ;

    // Tiles of the chunks of even / odd batches of BATCH chunks, lane i holding
    // tile i % TL of chunk BATCH batch + i / TL: the byte offset of its first row from
    // this wave's pool and head (lo, hi), the bytes this wave may read from it
    // (0 for a tile outside the sequence or the pool) and whether it is mapped
    // (K bytes).  Two sets, so that refreshing the next batch keeps the tiles
    // of chunks still in flight; filled once per batch.
    uint32_t off_lo0 = 0, off_hi0 = 0, nbytes0 = 0, kvalid0 = 0;     // even batches
    uint32_t off_lo1 = 0, off_hi1 = 0, nbytes1 = 0, kvalid1 = 0;     // odd batches
    auto refresh = [&](int c) {
        const int cq = c + lane / TL;
        const int ts = j0 + cq * CH + 16 * (lane % TL);
        const int page = cq < nchunk ? tile_page(a, b, ts, jend, lead) : -1;
        const int row = ts % a.page_tokens;
        const bool ok = page >= 0;
        const int64_t off = ok ? (int64_t)page * role_sp + (int64_t)row * role_st : 0;
        const int vrows = min(16, max(jend - ts, 0));
        const uint32_t lo = (uint32_t)off, hi = (uint32_t)((uint64_t)off >> 32);
        const uint32_t nb = ok ? (uint32_t)((is_k ? 16 : vrows) * role_st) : 0u;
        if ((c / BATCH) & 1) {
            off_lo1 = lo;
            off_hi1 = hi;
            nbytes1 = nb;
            kvalid1 = ok;
        } else {
            off_lo0 = lo;
            off_hi0 = hi;
            nbytes0 = nb;
            kvalid0 = ok;
        }
    };
    auto tile_ok = [&](int c, int t) {
        const uint32_t r = ((c / BATCH) & 1) ? kvalid1 : kvalid0;
        return __builtin_amdgcn_readlane(r, TL * (c % BATCH) + t) != 0;
    };

    struct Regs {
        u32x4 r16[BF ? PMAX : 1];
        u32x2 r8[BF ? 1 : PMAX];
    };
    // this wave's pieces of chunk c into registers: one descriptor per chunk
    auto issue = [&](int c, Regs &rg) {
        const int q = (c / BATCH) & 1, li = TL * (c % BATCH) + t_w;
        const uint32_t lo = __builtin_amdgcn_readlane(q ? off_lo1 : off_lo0, li);
        const uint32_t hi = __builtin_amdgcn_readlane(q ? off_hi1 : off_hi0, li);
        const uint32_t nb = __builtin_amdgcn_readlane(q ? nbytes1 : nbytes0, li);
        const i32x4 rs = make_buffer_rsrc(role_base + (((uint64_t)hi << 32) | lo), nb);
#pragma unroll
        for (int x = 0; x < PMAX; ++x) {
            if (x >= per)                      // (never taken when K and V widths match)
                break;
            if constexpr (BF)
                rg.r16[x] = nbx_buffer_load_b128(rs, role_lane + x * 32 * ESZ, 0, 0);
            else
                rg.r8[x] = nbx_buffer_load_b64(rs, role_lane + x * 32 * ESZ, 0, 0);
        }
    };
    // this wave's pieces of a chunk, landed in registers, into an LDS buffer
    // (rows outside a descriptor range were read as zeros)
    auto land = [&](uint8_t *buf, const Regs &rg) {
        uint8_t *dst = is_k ? buf + (t_w * KK + pbase) * 1024 + k_st
                            : buf + KBYTES + t_w * DT * 512 + pbase * 1024 + lane * 16;
#pragma unroll
        for (int x = 0; x < PMAX; ++x) {
            if (x >= per)
                break;
            if constexpr (BF)
                *(u32x4 *)(dst + x * 1024) = rg.r16[x];
            else
                *(u32x4 *)(dst + x * 1024) = widen8_e4m3(rg.r8[x]);
        }
    };
    auto compute = [&](int c, int boff) {
        const int p0 = j0 + c * CH;
        bool ok[TL];
#pragma unroll
        for (int t = 0; t < TL; ++t)
            ok[t] = tile_ok(c, t);
        f32x4 acc[NT][TL];
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
            for (int t = 0; t < TL; ++t)
                acc[n][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
#pragma unroll
            for (int t = 0; t < TL; ++t) {
                const u32x4 ka = *(const u32x4 *)(k_rd + boff + (t * KK + kk) * 1024);
#pragma unroll
                for (int n = 0; n < NT; ++n)
                    acc[n][t] = mfma_bf16(ka, qb[n][kk], acc[n][t]);
            }
        u32x4 ph[NT][NK], pl[NT][NK];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            const int e_n = min(jend, n_row[n]);
            float sc[TL][4];
#pragma unroll
            for (int t = 0; t < TL; ++t) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int pos = p0 + 16 * t + 4 * g + i;
                    sc[t][i] = (ok[t] && pos < e_n) ? acc[n][t][i] * scale2 : -INFINITY;
                }
            }
            if (fixed[n])
                softmax_fixed_n<PVS, NK>(sc, m_fix[n], l_run[n], ph[n], pl[n]);
            else
                softmax_step_n<DT, PVS, NK>(sc, m_run[n], l_run[n], o[n], ph[n], pl[n]);
        }
#pragma unroll
        for (int kq = 0; kq < NK; ++kq)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const u32x4 va = vt_operand<DT>(vt_lane + boff + kq * 2 * DT * 512, dt);
#pragma unroll
                for (int n = 0; n < NT; ++n) {
                    o[n][dt] = mfma_bf16(va, ph[n][kq], o[n][dt]);
                    if constexpr (PVS)
                        o[n][dt] = mfma_bf16(va, pl[n][kq], o[n][dt]);
                }
            }
    };

    // Iteration c: barrier (chunk c is in LDS buffer c & 1, every wave is done
    // with chunk c - 1), compute chunk c, land chunk c + 1 from registers into
    // buffer (c + 1) & 1, issue chunk c + 1 + NSET into the registers just
    // freed (NSET register sets: NSET + 1 chunks ahead of the one computed).
    // Loads and landings past the last chunk are issued all the same (their
    // descriptors are empty, so they read zeros and touch no memory): with no
    // branch around them the waits for each register set stay exact and the
    // chunks behind it stay in flight.
    Regs rset[NSET];
    auto step = [&](int c, Regs &land_regs) {
        __syncthreads();
        if (has_rows && c < nchunk)
            compute(c, (c & 1) * BUF);
        land(smem + ((c + 1) & 1) * BUF, land_regs);
        if ((c + 1 + NSET) % BATCH == 0)
            refresh(c + 1 + NSET);
        issue(c + 1 + NSET, land_regs);
    };
    if (nchunk > 0) {
        refresh(0);
        issue(0, rset[0]);
        land(smem, rset[0]);
        issue(1, rset[0]);
        if constexpr (NSET == 2)
            issue(2, rset[1]);
        for (int c = 0; c < nchunk; c += NSET) {
            step(c, rset[0]);                  // lands c + 1, reissues c + 1 + NSET there
            if constexpr (NSET == 2)
                step(c + 1, rset[1]);          // lands c + 2, reissues c + 4 there
        }
    }

    const float vs = a.v_scale;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const float lt = xor_sum16_32(l_run[n]);
        const int m = row_lo + (w * NT + n) * 16 + j;
        if (m < row_hi) {
            const int64_t row = row_base + m;
            float *op = a.o_part + (row * a.n_split + s) * DV;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                *(f32x4 *)(op + dt * 16 + 4 * g) = o[n][dt] * vs;
            if (g == 0) {
                a.m_part[row * a.n_split + s] = stored_m(fixed[n], m_fix[n], m_run[n], lt);
                a.l_part[row * a.n_split + s] = lt;
            }
        }
    }
}

// ------------------------------------------------------------------ dispatch

// multi-row chunks: 2 k-steps (64 positions), one register set in flight
constexpr int kMrNK = 2, kMrNSet = 1;


// Waves the current device holds at once for the persistent decode kernel
// (resident workgroups per CU x CUs), cached per device.
template <int D, int DV, int KVT, bool PVS, int NB, bool FA, bool BND>
int persistent_waves()
{
    constexpr int kMaxDev = 64;
    static std::atomic<int> cache[kMaxDev];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return 0;
    if (dev < kMaxDev) {
        const int v = cache[dev].load(std::memory_order_relaxed);
        if (v > 0)
            return v;
    }
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu,
            reinterpret_cast<const void *>(&decode_persistent_kernel<D, DV, KVT, PVS, NB, FA, BND>),
            64,
            0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    const int v = per_cu * cus;
    if (dev < kMaxDev)
        cache[dev].store(v, std::memory_order_relaxed);
    return v;
}

template <int D, int DV, int KVT, bool PVS, int NB, bool FA, bool BND>
hipError_t launch_persistent(const PartialArgs &a, hipStream_t stream)
{
    const int64_t items = (int64_t)a.batch * a.kv_heads * a.n_split;
    const int waves = persistent_waves<D, DV, KVT, PVS, NB, FA, BND>();
    if (waves <= 0)
        return hipErrorInvalidConfiguration;
    const int grid = (int)(items < waves ? items : waves);
    hipLaunchKernelGGL((decode_persistent_kernel<D, DV, KVT, PVS, NB, FA, BND>), dim3(grid),
                       dim3(64), 0, stream, a);
    return hipGetLastError();
}

bool persistent_shape(const PartialArgs &a)
{
    return a.rows_per_kv <= 16 && a.batch <= kPersistMaxBatch;
}

template <int D, int DV, int KVT, bool PVS>
hipError_t launch_kind(const PartialArgs &a, hipStream_t stream)
{
    const int M = a.rows_per_kv;
    if (persistent_shape(a)) {
        const bool fa = a.new_k != nullptr && a.n_new > 0;
        // bounds matter to the fused append (any pool) and to the reads (both)
        const bool bnd = fa ? (a.k_bounds || a.v_bounds) : (a.k_bounds && a.v_bounds);
#define NBX_PERSIST(NB_)                                                                        \
    (fa ? (bnd ? launch_persistent<D, DV, KVT, PVS, NB_, true, true>(a, stream)                 \
               : launch_persistent<D, DV, KVT, PVS, NB_, true, false>(a, stream))               \
        : (bnd ? launch_persistent<D, DV, KVT, PVS, NB_, false, true>(a, stream)                \
               : launch_persistent<D, DV, KVT, PVS, NB_, false, false>(a, stream)))
        if (a.batch <= 64)
            return NBX_PERSIST(1);
        return NBX_PERSIST(4);
#undef NBX_PERSIST
    }
    if (a.new_k != nullptr && a.n_new > 0)
        return hipErrorInvalidValue;           // the caller appends first for these shapes
    if (M <= 16) {
        // waves per (split, head): enough that each wave's run of chunks is short
        const int split = a.split_size > 0 ? a.split_size
                                           : (a.max_pages * a.page_tokens + a.n_split - 1) / a.n_split;
        const int chunks = (split + kChunk - 1) / kChunk;
        const int64_t blocks = (int64_t)a.n_split * a.batch * a.kv_heads;
        if (blocks > 0x7FFFFFFF)
            return hipErrorInvalidConfiguration;
        dim3 grid((unsigned)blocks);
        if (chunks >= 16)
            hipLaunchKernelGGL((decode_mfma_kernel<D, DV, KVT, PVS, 4>), grid, dim3(256), 0, stream,
                               a);
        else if (chunks >= 4)
            hipLaunchKernelGGL((decode_mfma_kernel<D, DV, KVT, PVS, 2>), grid, dim3(128), 0, stream,
                               a);
        else
            hipLaunchKernelGGL((decode_mfma_kernel<D, DV, KVT, PVS, 1>), grid, dim3(64), 0, stream,
                               a);
        return hipGetLastError();
    }
    const int64_t heads = (int64_t)a.batch * a.kv_heads * a.n_split;
    const int nt = multirow_tiles(M, D);
    const int row_blocks = multirow_row_blocks(M, D);
    const int64_t blocks = heads * row_blocks;
    if (blocks > 0x7FFFFFFF)
        return hipErrorInvalidConfiguration;
    if (nt == 2)
        hipLaunchKernelGGL((multirow_mfma_kernel<D, DV, KVT, PVS, 2, kMrNK, kMrNSet>),
                           dim3((unsigned)blocks), dim3(512), 0, stream, a, row_blocks);
    else
        hipLaunchKernelGGL((multirow_mfma_kernel<D, DV, KVT, PVS, 1, kMrNK, kMrNSet>),
                           dim3((unsigned)blocks), dim3(512), 0, stream, a, row_blocks);
    return hipGetLastError();
}

template <int KVT, bool PVS>
hipError_t launch_d(const PartialArgs &a, hipStream_t stream)
{
    switch (a.head_dim) {
    case 64: return launch_kind<64, 64, KVT, PVS>(a, stream);
    case 128: return launch_kind<128, 128, KVT, PVS>(a, stream);
    case 192: return launch_kind<192, 128, KVT, PVS>(a, stream);   // the only pair with 192
    default: return launch_kind<256, 256, KVT, PVS>(a, stream);
    }
}

}  // namespace

bool partial_mfma_is_persistent(const PartialArgs &a) { return persistent_shape(a); }

// 8 waves x 16 rows per multi-row workgroup (8 x 32 where a KV head has more
// rows than that and D <= 128: D = 256 would spill at 32 rows per wave)
int multirow_tiles(int rows_per_kv, int head_dim)
{
    return rows_per_kv > 128 && head_dim <= 128 ? 2 : 1;
}

int multirow_row_blocks(int rows_per_kv, int head_dim)
{
    const int r = 128 * multirow_tiles(rows_per_kv, head_dim);
    return (rows_per_kv + r - 1) / r;
}

hipError_t launch_partial_mfma(const PartialArgs &a, hipStream_t stream)
{
    // bf16 pools carry P as hi + lo parts; fp8 pools (tolerance set by their
    // 3-bit mantissa) use the bf16-rounded P alone
    if (a.kv_dtype == NBX_BF16)
        return launch_d<NBX_BF16, true>(a, stream);
    return launch_d<NBX_FP8_E4M3, false>(a, stream);
}

}  // namespace nbx
