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
// Two kernels here (the multi-row kernel, which shares the products, operand
// layouts and softmax, is in partial_multirow.hip):
//  - decode_persistent_kernel: at most 16 rows per KV head (decode, short
//    windows) and at most 256 sequences; one wave per (sequence, split, KV
//    head) item, as many waves as the device holds, items enumerated on the
//    device, the step's append fused in (described at the kernel).
//  - decode_mfma_kernel: the same rows for larger batches.  PG waves per
//    (split, sequence x KV head) take interleaved chunks of the split, each
//    with its own (m, l, O), combined in a fixed order at the end.
// In decode_mfma_kernel, and in the persistent kernel for fp8 pools, K rows go
// from HBM straight into MFMA operand registers (16 rows x 64 bytes per load)
// and V rows are written to the wave's LDS tile once they land (fp8 codes
// widened on the way).  The persistent kernel loads bf16 K and V tiles as
// whole rows (64 consecutive 16-byte units per load, RowTile) into LDS and
// reads K back in the operand layout.  The wave's next chunk is loaded while
// the current one is computed.  The persistent kernel also takes the
// fixed-shift softmax (partial_common.h) when both pools carry per-page bounds.
#include <atomic>

#include "partial_common.h"

namespace nbx {

namespace {

constexpr int kChunk = 32;   // positions per chunk: two 16-position tiles, one PV k-step

// Lane i of the result: page of tile (i & 1) of chunk c0 + (i / 2) * cstep,
// -1 past the split.  Refreshed once per 32 chunks of a wave.
__device__ __forceinline__ int chunk_pages(const PartialArgs &a, int b, int j0, int jend,
                                           int nchunk, int c0, int cstep, int lane, bool flag_it)
{
    const int cq = c0 + (lane >> 1) * cstep;
    const int ts = j0 + cq * kChunk + 16 * (lane & 1);
    return cq < nchunk ? tile_page(a, b, ts, jend, flag_it) : -1;
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
                    vr[i] = nbx_buffer_load_b128(rv, v_lane + k * 64, 0, kStreamAux);
                else
                    vraw[i] = nbx_buffer_load_b64(rv, v_lane + k * 32, 0, kStreamAux);
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
// D = 128 it is held to 2 waves per SIMD like the plain one (256 registers,
// 12 bytes spilled outside the streaming path; left to itself the compiler
// takes one more AGPR block and halves the resident waves).
template <int D, int DV, int KVT, bool PVS, int NB, bool FA, bool BND>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(((BND || KVT == NBX_BF16) && D == 128) ? 2 : 1)))
decode_persistent_kernel(PartialArgs a)
{
    constexpr int KK = D / 32, DT = DV / 16;
    constexpr bool BF = KVT == NBX_BF16;
    constexpr int ESZ = BF ? 2 : 1;
    constexpr int VBYTES = kChunk * 2 * DV;
    // bf16 pools: K and V tiles are loaded as whole rows (rows_k / rows_v
    // below) and K is read back from LDS; fp8 pools load each operand's
    // 16 x 64-byte piece straight into registers
    constexpr bool RM = BF;
    constexpr int KBYTES = RM ? kChunk * 2 * D : 16;
    __shared__ __attribute__((aligned(16))) uint8_t tile[VBYTES];
    __shared__ __attribute__((aligned(16))) uint8_t ktile[KBYTES];

    const int lane = threadIdx.x;
    const int g = lane >> 4, j = lane & 15;
    const int wv = blockIdx.x, W = gridDim.x;
    const int M = a.rows_per_kv, H = a.kv_heads, NS = a.n_split;
    const int cap = a.max_pages * a.page_tokens;

    // sequence table, lane l of block t describing b = 64 t + l: clamped
    // length, splits holding keys, inclusive prefix of item counts
    // The block table into this XCD's L2 while the lengths are fetched: wave
    // wv reads 256 bytes of it, the slice wv / 8 (the waves of one XCD are
    // every eighth), so that the page lookups of the first items, which wait
    // on the lengths, find it in the cache.  A table larger than (waves / 8) x
    // 256 bytes is covered from its start; reads past its end return zeros
    // and touch no memory.
    const uint64_t bt_bytes = (uint64_t)a.batch * a.max_pages * 4;
    const int pf = nbx_buffer_load_b32(
        make_buffer_rsrc(a.block_table, (uint32_t)min(bt_bytes, (uint64_t)0x7FFFFFF0u)),
        (wv >> 3) * 256 + lane * 4, 0, 0);
    // (nsw holds a sequence's split count in its low 16 bits and its window
    // rows, at most 16, above them: one register per lane block for both)
    int Lr[NB], Wr[NB], nsw[NB], incl[NB];
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
    // S and N are wave-uniform.  With bounds at D <= 128 they are moved to
    // scalar registers: that instantiation then spills 16 bytes instead of 36.
    // Elsewhere the move buys nothing measurable (D <= 128) or makes the
    // D = 256 instantiations with bounds spill more, so it is not made.
    constexpr bool kScalarSN = BND && D <= 128;
    if constexpr (kScalarSN)
        S = __builtin_amdgcn_readfirstlane(S);
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
        nsw[t] = ns | (Wr[t] << 16);
        incl[t] = carry + x;
        carry = __shfl(incl[t], 63, 64);
    }
    const int N = kScalarSN ? __builtin_amdgcn_readfirstlane(carry) : carry;   // items
    // value of wave-uniform sequence b in a lane table (lane reads of the
    // table registers themselves, valid whatever lanes are active)
    auto lane_val = [&](const int (&arr)[NB], int b) {
        int v = __builtin_amdgcn_readlane(arr[0], b & 63);
#pragma unroll
        for (int t = 1; t < NB; ++t) {
            const int x = __builtin_amdgcn_readlane(arr[t], b & 63);
            v = (b >> 6) == t ? x : v;
        }
        return v;
    };

    // splits without keys: m = -inf, l = 0 for their rows
    {
        const int per_b = NS * H, pairs = a.batch * per_b;
        for (int pi = wv; pi < pairs; pi += W) {
            const int b = pi / per_b, rem = pi - b * per_b, s = rem / H, gk = rem - s * H;
            if (s >= (lane_val(nsw, b) & 0xFFFF) && lane < M) {
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
    // this lane's window row, j mod q_rows (j < 16), recomputed where it is
    // needed from a fresh lane id (an asm statement the compiler neither
    // merges nor keeps live, so that neither j nor the row takes a register
    // across the main loop)
    auto window_row = [&]() {
        int id;
        asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(id));
        int r = id & 15;
        while (r >= a.q_rows)
            r -= a.q_rows;
        return r;
    };
    auto make_item = [&](int k) {
        Item it;
        const int jrow = window_row();
        int before = 0;                        // sequences whose items all precede k
#pragma unroll
        for (int t = 0; t < NB; ++t)
            before += __popcll(__ballot(incl[t] <= k));
        it.b = before;
        const int nw = lane_val(nsw, it.b);
        const int excl = lane_val(incl, it.b) - (nw & 0xFFFF) * H;
        const int r = k - excl;
        it.s = r / H;
        it.gk = r - it.s * H;
        const int L = lane_val(Lr, it.b), wb = nw >> 16;
        it.j0 = it.s * S;
        it.jend = min(it.j0 + S, seq_keys(L, wb));
        it.nchunk = (it.jend - it.j0 + kChunk - 1) / kChunk;
        const int n_j = j < M ? row_keys(a, L, wb, jrow) : 0;
        it.e_j = min(it.jend, n_j);
        it.row_base = ((int64_t)it.b * a.q_heads + (int64_t)it.gk * a.group) * a.q_rows;
        it.L = L;
        it.kb = it.vb = 0.0f;                  // raised by the rows the append writes
        return it;
    };
    // Fused append: the new positions L - n_new .. L - 1 that fall in the item
    // are written to the pools (the conversions of the append kernel) before
    // any load of the item is issued.  The item of the last split also takes
    // the positions at or past NS * S that no item covers (a length the split
    // plan does not reach, flagged above); a sequence longer than its
    // block-table row gets none (the separate append skips it the same way).
    // Only this wave reads the item's tiles, and a wave's memory operations
    // are performed in order, so its later tile loads see the new rows.
    // `pg` holds the page ids of the item's first 32 chunks (item_pages(it, 0)).
    // With bounds, each written row raises its page's bound and the item's.
    auto append_item = [&](Item &it, int pg) {
        if constexpr (FA) {
            const int Lw = a.seq_lens[it.b];   // as given (it.L is clamped to the row)
            const int first = Lw - a.n_new;
            const int lo = max(it.j0, max(first, 0));
            const int hi = Lw > cap ? lo : it.s == NS - 1 ? Lw : min(it.j0 + S, Lw);
            for (int p = lo; p < hi; ++p) {
                const int tl = (p - it.j0) >> 4;           // tile of p within the item
                const int page = tl < 64 && p < it.jend ? __builtin_amdgcn_readlane(pg, tl)
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
                    it.kb = wave_uniform(bound_max(it.kb, kn));
                    it.vb = wave_uniform(bound_max(it.vb, vm));
                }
            }
            asm volatile("" ::: "memory");     // keep the tile loads after the stores
        }
    };
    // the item's Q rows through one descriptor over its M rows: lanes of rows
    // past M read zeros, and each lane's address is a 32-bit offset
    auto load_q = [&](const Item &it, u32x4 (&qv)[KK]) {
        const i32x4 rq = make_buffer_rsrc((const uint16_t *)a.q + it.row_base * D,
                                          (uint32_t)(M * D * 2));
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
            qv[kk] = nbx_buffer_load_b128(rq, j * (D * 2) + kk * 64 + g * 16, 0, 0);
    };
    // lane i: page of tile (i & 1) of chunk c0 + i / 2 of the item
    auto item_pages = [&](const Item &it, int c0) {
        const int cq = c0 + (lane >> 1);
        const int ts = it.j0 + cq * kChunk + 16 * (lane & 1);
        return cq < it.nchunk ? tile_page(a, it.b, ts, it.jend, true) : -1;
    };
    // Bounds of the pages an item reads (fixed shift), one lane per tile of its
    // first 32 chunks from its page ids `pg` (item_pages(it, 0)); past those,
    // the block table is walked.  The loads are issued with the item's first
    // tiles and reduced once those have landed, so that they wait on nothing
    // but the page ids.  Lane values; 0 where a lane has no page.
    float pkb = 0.0f, pvb = 0.0f;
    auto page_bounds = [&](const Item &it, int pg) {
        pkb = pvb = 0.0f;
        if (pg >= 0) {
            pkb = a.k_bounds[(int64_t)pg * H + it.gk];
            pvb = a.v_bounds[(int64_t)pg * H + it.gk];
        }
        if (it.nchunk > 32) {
            const int T = a.page_tokens;
            for (int pi = (it.j0 + 64 * 16) / T + lane; pi <= (it.jend - 1) / T; pi += 64) {
                const int page = a.block_table[(int64_t)it.b * a.max_pages + pi];
                if (page >= 0 && page < a.num_pages) {
                    pkb = bound_max(pkb, a.k_bounds[(int64_t)page * H + it.gk]);
                    pvb = bound_max(pvb, a.v_bounds[(int64_t)page * H + it.gk]);
                }
            }
        }
    };

    const int kst_b = (int)(a.k_stride_token * ESZ), vst_b = (int)(a.v_stride_token * ESZ);
    const int k_lane = j * kst_b + g * 8 * ESZ;                        // + kk * 32 * ESZ
    const int v_lane = ((lane & 31) >> 1) * vst_b + ((lane >> 5) * 16 + (lane & 1) * 8) * ESZ;
    const uint8_t *vt_lane = tile + (4 * g + (j >> 2)) * 32 + (j & 3) * 8;
    const RowTile<D> rows_k(lane, kst_b);
    const RowTile<DV> rows_v(lane, vst_b);
    const float scale2 = a.scale * a.k_scale * kLog2e;
    const float vs = a.v_scale;

    typename KvRaw<KVT>::type kr[2][KK];       // K as loaded; widened at its use
    u32x4 qb[KK];
    u32x4 qn[RM ? KK : 1];                     // bf16: the next chunk's Q, loaded with its K
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
                if constexpr (RM)
                    vr[i] = nbx_buffer_load_b128(rv, rows_v.global(k), 0, kStreamAux);
                else if constexpr (BF)
                    vr[i] = nbx_buffer_load_b128(rv, v_lane + k * 64, 0, kStreamAux);
                else
                    vraw[i] = nbx_buffer_load_b64(rv, v_lane + k * 32, 0, kStreamAux);
            }
        }
    };
    // K rows of the chunk and, with them, the item's Q rows (a few KB that stay
    // in L2): one register set each; for fp8 refilled right after the scores
    // are formed, for bf16 (K landed in LDS) with the V rows
    auto issue_k = [&](const Item &it, int c, int pg0, int pg1) {
        if constexpr (!RM)
            load_q(it, qb);
        else if (c == 0)                       // a new item: its Q, taken up at its first chunk
            load_q(it, qn);
        const int p0 = it.j0 + c * kChunk;
        const int64_t k_head = (int64_t)it.gk * a.k_stride_head;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const i32x4 rk = tile_rsrc<ESZ>(a.k_data, a.k_stride_page, k_head, a.k_stride_token,
                                            a.page_tokens, t ? pg1 : pg0, p0 + 16 * t, 16);
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                if constexpr (RM)
                    kr[t][kk] = nbx_buffer_load_b128(rk, rows_k.global(kk), 0, kStreamAux);
                else
                    kr[t][kk] = buffer_load8_raw<KVT>(rk, k_lane + kk * 32 * ESZ);
            }
        }
    };
    auto land_v = [&]() {
#pragma unroll
        for (int i = 0; i < DT; ++i) {
            const int t = i / (DT / 2), k = i % (DT / 2);
            if constexpr (RM) {
                *(u32x4 *)(tile + t * (VBYTES / 2) + rows_v.lds(k)) = vr[i];
            } else {
                u32x4 v;
                if constexpr (BF)
                    v = vr[i];
                else
                    v = widen8_e4m3(vraw[i]);
                *(u32x4 *)(tile + t * DT * 512 + k * 1024 + lane * 16) = v;
            }
        }
    };
    auto land_k = [&]() {
        if constexpr (RM) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int kk = 0; kk < KK; ++kk)
                    *(u32x4 *)(ktile + t * (KBYTES / 2) + rows_k.lds(kk)) = kr[t][kk];
        }
    };
    // A operand of S^T = K Q^T for k-step kk of tile t: lane (g, j) takes
    // row j, columns 32 kk + 8 g .. + 7 (from LDS for bf16)
    auto k_operand = [&](int t, int kk) {
        if constexpr (RM)
            return *(const u32x4 *)(ktile + t * (KBYTES / 2) + rows_k.operand(j, 4 * kk + g));
        else
            return as_bf16x8<KVT>(kr[t][kk]);
    };
    // A operand of O^T += V^T P^T for 16-column slice dt (both tiles)
    auto v_operand = [&](int dt) {
        if constexpr (RM)
            return rows_v.transposed(tile, VBYTES / 2, g, j, dt);
        else
            return vt_operand<DT>(vt_lane, dt);
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
    asm volatile("" ::"v"(pf));                // the prefetch has landed (its value is unused)
    int pg_reg = item_pages(cur, 0), pg_next = -1;
    append_item(cur, pg_reg);
    if (use_bounds)
        page_bounds(cur, pg_reg);
    Item nxt = cur;
    bool has_next = false;
    // the next item and its page ids, one chunk before its loads; its append
    // and page bounds wait for the switch to it, when the page ids are needed
    // anyway and no tile load is in flight
    auto prepare_next = [&]() {
        const int kn = wv + (i_item + 1) * W_eff;
        has_next = i_item + 1 < k_per && kn < N;
        if (has_next) {
            nxt = make_item(kn);
            pg_next = item_pages(nxt, 0);
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
        land_k();
        float kb_i = 0.0f, vb_i = 0.0f;        // the item's bounds (its page bounds have landed)
        if (use_bounds && cc == 0) {
            kb_i = wave_uniform(group_bound_max<64>(bound_max(pkb, ci.kb)));
            vb_i = wave_uniform(group_bound_max<64>(bound_max(pvb, ci.vb)));
        }
        if constexpr (RM) {
            if (cc == 0) {                     // the item's Q (loaded before its K)
#pragma unroll
                for (int kk = 0; kk < KK; ++kk)
                    qb[kk] = qn[kk];
            }
        }
        bool more = true;
        if (c + 1 < cur.nchunk) {
            ++c;
            if ((c & 31) == 0)
                pg_reg = item_pages(cur, c);
        } else if (has_next) {
            cur = nxt;
            ++i_item;
            c = 0;
            pg_reg = pg_next;
            append_item(cur, pg_reg);
            if (use_bounds)
                page_bounds(cur, pg_reg);
        } else {
            more = false;
        }
        if (more) {
            pg0 = __builtin_amdgcn_readlane(pg_reg, 2 * (c & 31));
            pg1 = __builtin_amdgcn_readlane(pg_reg, 2 * (c & 31) + 1);
            issue_v(cur, c, pg0, pg1);
            if constexpr (RM) {               // K(c) is in LDS: its registers are free
                issue_k(cur, c, pg0, pg1);
                if (c == cur.nchunk - 1)
                    prepare_next();
            }
        }
        const int p0 = ci.j0 + cc * kChunk;
        float sc[2][4];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
                acc = mfma_bf16(k_operand(t, kk), qb[kk], acc);
            const bool tv = (t ? cpg1 : cpg0) >= 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int pos = p0 + 16 * t + 4 * g + i;
                sc[t][i] = (tv && pos < ci.e_j) ? acc[i] * scale2 : -INFINITY;
            }
        }
        if (use_bounds && cc == 0) {           // the item's Q is still in qb
            int C, gate;
            bool ok = fixed_shift_consts(ci.L, vb_i, vs, C, gate);
            ok = ok && fixed_shift_row(q_row_norm<KK>(qb), kb_i, fabsf(scale2), C, gate, m_fix);
            fixed = __all(ok);
        }
        if (!RM && more) {
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
            const u32x4 va = v_operand(dt);
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
// ------------------------------------------------------------------ dispatch


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

// at most 16 rows per KV head: the persistent kernel, else (larger batches)
// the per-split workgroup kernel
template <int D, int DV, int KVT, bool PVS>
hipError_t launch_kind(const PartialArgs &a, hipStream_t stream)
{
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
    // waves per (split, head): enough that each wave's run of chunks is short
    const int split = a.split_size > 0 ? a.split_size
                                       : (a.max_pages * a.page_tokens + a.n_split - 1) / a.n_split;
    const int chunks = (split + kChunk - 1) / kChunk;
    const int64_t blocks = (int64_t)a.n_split * a.batch * a.kv_heads;
    if (!grid_fits(blocks, chunks >= 16 ? 256 : chunks >= 4 ? 128 : 64))
        return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)blocks);
    if (chunks >= 16)
        hipLaunchKernelGGL((decode_mfma_kernel<D, DV, KVT, PVS, 4>), grid, dim3(256), 0, stream, a);
    else if (chunks >= 4)
        hipLaunchKernelGGL((decode_mfma_kernel<D, DV, KVT, PVS, 2>), grid, dim3(128), 0, stream, a);
    else
        hipLaunchKernelGGL((decode_mfma_kernel<D, DV, KVT, PVS, 1>), grid, dim3(64), 0, stream, a);
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

hipError_t launch_partial_mfma(const PartialArgs &a, hipStream_t stream)
{
    if (a.rows_per_kv > 16)
        return launch_partial_multirow(a, stream);
    // bf16 pools carry P as hi + lo parts; fp8 pools (tolerance set by their
    // 3-bit mantissa) use the bf16-rounded P alone
    if (a.kv_dtype == NBX_BF16)
        return launch_d<NBX_BF16, true>(a, stream);
    return launch_d<NBX_FP8_E4M3, false>(a, stream);
}

}  // namespace nbx
