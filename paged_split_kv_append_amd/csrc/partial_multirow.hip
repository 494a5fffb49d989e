// Split partials for many query rows per KV head (verify windows, prompt
// chunks) on the matrix cores, bf16 and fp8 (E4M3FN) pools with bf16 Q.
//
// The computation is that of the split kernel on the nbxtensor
// paged_decode_attn.py page (paged_decode_attn_split_kernel) with all query
// rows of a KV head (GQA heads x window rows) as the N side of the products,
// so that each K/V byte is read from HBM once per split however many rows use
// it (TensorFold PR #1219).  The products, operand layouts and softmax are
// those of the decode kernels (partial_mfma.hip); what differs is that a
// workgroup's waves share the loads of each K and V chunk through LDS.
// Workgroups are ordered row block fastest and mapped so that the row blocks
// of one split run on the same XCD and share its L2 (the rows-first order of
// TensorFold PR #1219, made XCD-aware).  The fixed-shift softmax is taken
// when both pools carry per-page bounds; otherwise the online softmax moves a
// row's shift lazily (only when its maximum has grown by more than 2^8 in
// log2 units) and puts the partial in the exact-maximum form before the
// store.  Chunks that every stored row of a wave sees whole skip the mask.
#include "partial_common.h"

namespace nbx {

namespace {

// A workgroup of 8 waves takes 8 x NT row tiles of 16 rows of one (sequence,
// KV head, split).  The K and V tiles of a chunk are pieces of 1 KB (as bf16:
// 16 rows x 32 columns); waves 0-3 load the K pieces and waves 4-7 the V
// pieces, each wave all its pieces from one tile, so each of its loads has a
// fixed role (K or V, tile) and one descriptor per tile serves it.  Chunk c + 1
// waits in LDS and chunks c + 2 ... c + 1 + NSET in registers while chunk c is
// computed; one barrier per chunk.  K is stored in LDS with a 16-byte
// swizzle inside each 1 KB block (row r, piece p at unit 4 r + ((p + r / 2) &
// 3)): a 16-byte LDS read serves 8 lanes per cycle, and the 8 consecutive lanes
// of an operand read (8 rows, one piece each) then cover the 32 banks once.
// (With (p + r / 4) & 3 two of those rows shared banks: the bank-conflict
// counter read 28% of the LDS-active cycles, and the prompt chunk took 9% longer.)
// Within each phase the LDS operand reads run ahead of the products that use
// them (schedule_reads_ahead): K one k-step ahead, V four operands ahead.
// NTL: the K/V loads are marked non-temporal (one row block per split: no
// other workgroup reads the same tiles); with several row blocks they stay
// cacheable, since the row blocks of a split read its tiles from the L2.
// LW (at most 6 x 16 rows, e.g. a 16-row window over 6 query heads): waves
// 0-5 hold the rows and only compute, wave 6 loads and lands all K pieces and
// wave 7 all V pieces of each chunk, so that the waves that compute issue no
// load and no landing (with 8 waves of rows those two waves would hold none).
template <int D, int DV, int KVT, bool PVS, int NT, int NK, int NSET, bool NTL, bool LW>
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
    constexpr int ROWW = LW ? 6 : RW;          // waves holding rows
    constexpr int R = ROWW * NT * 16;          // rows per workgroup
    constexpr int PL = KK > KV ? KK : KV;      // LW: pieces per tile of a loader's pool
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
    const bool has_rows = w < ROWW && row_lo + w * NT * 16 < row_hi;
    const bool loader = LW && w >= ROWW;       // LW: wave 6 loads K, wave 7 V

    const int S = device_split_size(a);
    const int L = clamp_len(a, b, lead && s == 0 && rb == 0);
    if (lead && rb == 0 && s == a.n_split - 1 && L > a.n_split * S)
        flag_error(a.dev_err, NBX_DEVERR_SEQ_RANGE);

    const int wb = seq_window(a, b, lead && s == 0 && rb == 0);
    int n_row[NT];
    bool row_in[NT];                           // the lane's row of tile n is stored
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const int m = row_lo + (w * NT + n) * 16 + j;
        row_in[n] = m < row_hi;
        n_row[n] = row_in[n] ? row_keys(a, L, wb, m % a.q_rows) : 0;
    }
    int n_max = 0;                             // the most keys a row of this block sees
    for (int m = row_lo; m < row_hi && m < row_lo + a.q_rows; ++m)
        n_max = max(n_max, row_keys(a, L, wb, m % a.q_rows));
    const int j0 = s * S;
    const int jend = min(j0 + S, n_max);
    const int nchunk = jend > j0 ? (jend - j0 + CH - 1) / CH : 0;

    const int64_t k_head = (int64_t)gk * a.k_stride_head;
    const int64_t v_head = (int64_t)gk * a.v_stride_head;
    const int kst_b = (int)(a.k_stride_token * ESZ), vst_b = (int)(a.v_stride_token * ESZ);
    // fixed per-lane byte offsets of the 64-lane piece loads
    const int k_lane = (lane >> 2) * kst_b + (lane & 3) * 8 * ESZ;   // + kk * 32 * ESZ
    const int v_lane = ((lane & 31) >> 1) * vst_b + ((lane >> 5) * 16 + (lane & 1) * 8) * ESZ;
    // LDS: swizzled K store of this lane (row lane / 4, piece lane % 4) and
    // read of operand piece g of row j; transposed V read
    const int k_st = (4 * (lane >> 2) + (((lane & 3) + (lane >> 3)) & 3)) * 16;
    const uint8_t *k_rd = smem + (4 * j + ((g + (j >> 1)) & 3)) * 16;   // + (t*KK + kk) * 1024
    const uint8_t *vt_lane = smem + KBYTES + (4 * g + (j >> 2)) * 32 + (j & 3) * 8;

    // Wave roles: waves 0-3 load K, 4-7 load V; of the pieces of its pool
    // (tile-major: K 32-column groups kk, V 32-column pairs of 16-column
    // slices) wave w takes (w & 3) * per ... (w & 3) * per + per - 1, all in
    // tile t_w of every chunk.
    const bool is_k = LW ? w != 7 : w < 4;    // (LW: the row waves' role only sets kvalid)
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
                rg.r16[x] = nbx_buffer_load_b128(rs, role_lane + x * 32 * ESZ, 0, NTL ? kStreamAux : 0);
            else
                rg.r8[x] = nbx_buffer_load_b64(rs, role_lane + x * 32 * ESZ, 0, NTL ? kStreamAux : 0);
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
    // LW: a loader's pieces of all tiles of chunk c, one descriptor per tile
    struct RegsL {
        u32x4 r16[BF ? TL * PL : 1];
        u32x2 r8[BF ? 1 : TL * PL];
    };
    const int lw_pieces = is_k ? KK : KV;
    const int lw_lane = is_k ? k_lane : v_lane;
    // tile t of chunk c: its pieces into registers / from registers into LDS
    auto issue_tile = [&](int c, RegsL &rg, int t) {
        const int q = (c / BATCH) & 1, li = TL * (c % BATCH) + t;
        const uint32_t lo = __builtin_amdgcn_readlane(q ? off_lo1 : off_lo0, li);
        const uint32_t hi = __builtin_amdgcn_readlane(q ? off_hi1 : off_hi0, li);
        const uint32_t nb = __builtin_amdgcn_readlane(q ? nbytes1 : nbytes0, li);
        const i32x4 rs = make_buffer_rsrc(role_base + (((uint64_t)hi << 32) | lo), nb);
#pragma unroll
        for (int x = 0; x < PL; ++x) {
            if (x >= lw_pieces)
                break;
            if constexpr (BF)
                rg.r16[t * PL + x] = nbx_buffer_load_b128(rs, lw_lane + x * 32 * ESZ, 0,
                                                          NTL ? kStreamAux : 0);
            else
                rg.r8[t * PL + x] = nbx_buffer_load_b64(rs, lw_lane + x * 32 * ESZ, 0,
                                                        NTL ? kStreamAux : 0);
        }
    };
    auto land_tile = [&](uint8_t *buf, const RegsL &rg, int t) {
        uint8_t *dst = is_k ? buf + t * KK * 1024 + k_st : buf + KBYTES + t * DT * 512 + lane * 16;
#pragma unroll
        for (int x = 0; x < PL; ++x) {
            if (x >= lw_pieces)
                break;
            if constexpr (BF)
                *(u32x4 *)(dst + x * 1024) = rg.r16[t * PL + x];
            else
                *(u32x4 *)(dst + x * 1024) = widen8_e4m3(rg.r8[t * PL + x]);
        }
    };
    // LW: the loaders run their own loop and leave; the row state below is
    // never live in them.  Iteration c: barrier (every wave is done with chunk
    // c - 1), then for each tile land it for chunk c + 1 into buffer
    // (c + 1) & 1 and reload its registers with chunk c + 2 — one barrier per
    // chunk, as the row waves.
    if constexpr (LW) {
        if (loader) {
            RegsL lr;
            if (nchunk > 0) {
                refresh(0);
#pragma unroll
                for (int t = 0; t < TL; ++t)
                    issue_tile(0, lr, t);
#pragma unroll
                for (int t = 0; t < TL; ++t) {
                    land_tile(smem, lr, t);
                    issue_tile(1, lr, t);
                }
                for (int c = 0; c < nchunk; ++c) {
                    __syncthreads();
                    if ((c + 2) % BATCH == 0)
                        refresh(c + 2);
                    // (the first tiles of chunk c + 2 are in flight while the
                    // later ones of c + 1 land)
#pragma unroll
                    for (int t = 0; t < TL; ++t) {
                        land_tile(smem + ((c + 1) & 1) * BUF, lr, t);
                        issue_tile(c + 2, lr, t);
                    }
                }
            }
            return;
        }
    }

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
    float m_run[NT], m_top[NT], l_run[NT];     // shift (lazy), maximum, sum of each row
    f32x4 o[NT][DT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        m_run[n] = -INFINITY;
        m_top[n] = -INFINITY;
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
        // each K operand read one k-step (TL reads) ahead of its products
        schedule_reads_ahead<KK * TL, 1, NT, TL, 0>();
        // Every position of the chunk visible to every stored row of the wave
        // (all chunks of a split but its last ones and a causal window's
        // edge): the scores need no mask.  Rows past the workgroup's last
        // row are never stored and do not count.
        bool lane_full = p0 + CH <= jend;
#pragma unroll
        for (int n = 0; n < NT; ++n)
            lane_full = lane_full && (p0 + CH <= n_row[n] || !row_in[n]);
#pragma unroll
        for (int t = 0; t < TL; ++t)
            lane_full = lane_full && ok[t];
        const bool full = __all(lane_full);
        u32x4 ph[NT][NK], pl[NT][NK];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            const int e_n = min(jend, n_row[n]);
            float sc[TL][4];
            if (full) {
#pragma unroll
                for (int t = 0; t < TL; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        sc[t][i] = acc[n][t][i] * scale2;
            } else {
#pragma unroll
                for (int t = 0; t < TL; ++t) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int pos = p0 + 16 * t + 4 * g + i;
                        sc[t][i] = (ok[t] && pos < e_n) ? acc[n][t][i] * scale2 : -INFINITY;
                    }
                }
            }
            if (fixed[n]) {
                softmax_fixed_n<PVS, NK>(sc, m_fix[n], l_run[n], ph[n], pl[n]);
            } else {
                const float corr =
                    softmax_lazy_n<PVS, NK>(sc, m_run[n], m_top[n], l_run[n], ph[n], pl[n]);
                if (__any(corr != 1.0f)) {
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt)
                        o[n][dt] *= corr;
                }
            }
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
        // each V operand (two transposing reads) four operands ahead of its products
        schedule_reads_ahead<NK * DT, 2, NT * (PVS ? 2 : 1), 4, 1>();
    };

    // Iteration c: barrier (chunk c is in LDS buffer c & 1, every wave is done
    // with chunk c - 1), compute chunk c, land chunk c + 1 from registers into
    // buffer (c + 1) & 1, issue chunk c + 1 + NSET into the registers just
    // freed (NSET register sets: NSET + 1 chunks ahead of the one computed).
    // Loads and landings past the last chunk are issued all the same (their
    // descriptors are empty, so they read zeros and touch no memory): with no
    // branch around them the waits for each register set stay exact and the
    // chunks behind it stay in flight.
    if constexpr (LW) {
        // Iteration c: barrier, then the row waves compute chunk c (the
        // loaders, which returned above, land chunk c + 1 meanwhile).
        if (nchunk > 0) {
            refresh(0);
            for (int c = 0; c < nchunk; ++c) {
                __syncthreads();
                if (has_rows)
                    compute(c, (c & 1) * BUF);
                if ((c + 2) % BATCH == 0)
                    refresh(c + 2);
            }
        }
    } else {
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
#pragma unroll
        for (int r = 0; r < NSET; ++r)         // chunk k waits in set (k - 1) % NSET
            issue(1 + r, rset[r]);
        for (int c = 0; c < nchunk; c += NSET) {
#pragma unroll
            for (int r = 0; r < NSET; ++r)     // lands c + r + 1, reissues c + r + 1 + NSET there
                step(c + r, rset[r]);
        }
    }
    }

    const float vs = a.v_scale;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        if (!fixed[n])
            lazy_finish<DT>(m_run[n], m_top[n], l_run[n], o[n]);
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

// chunks of 2 k-steps (64 positions), one register set in flight
#ifndef NBX_MR_NK
#define NBX_MR_NK 2
#define NBX_MR_NSET 1
#endif
constexpr int kMrNK = NBX_MR_NK, kMrNSet = NBX_MR_NSET;

template <int D, int DV, int KVT, bool PVS>
hipError_t launch_mr(const PartialArgs &a, hipStream_t stream)
{
    const int M = a.rows_per_kv;
    const int64_t heads = (int64_t)a.batch * a.kv_heads * a.n_split;
    const int nt = multirow_tiles(M, D);
    const int row_blocks = multirow_row_blocks(M, D);
    const int64_t blocks = heads * row_blocks;
    if (!grid_fits(blocks, 512))
        return hipErrorInvalidConfiguration;
    if constexpr (D <= 128) {                 // two row tiles per wave only below D = 256
        if (nt == 2) {                         // (more than 128 rows: several row blocks)
            hipLaunchKernelGGL((multirow_mfma_kernel<D, DV, KVT, PVS, 2, kMrNK, kMrNSet, false, false>),
                               dim3((unsigned)blocks), dim3(512), 0, stream, a, row_blocks);
            return hipGetLastError();
        }
    }
    if (M <= 96)                               // rows fit 6 waves: two dedicated loaders
        hipLaunchKernelGGL((multirow_mfma_kernel<D, DV, KVT, PVS, 1, kMrNK, kMrNSet, true, true>),
                           dim3((unsigned)blocks), dim3(512), 0, stream, a, row_blocks);
    else if (row_blocks == 1)
        hipLaunchKernelGGL((multirow_mfma_kernel<D, DV, KVT, PVS, 1, kMrNK, kMrNSet, true, false>),
                           dim3((unsigned)blocks), dim3(512), 0, stream, a, row_blocks);
    else
        hipLaunchKernelGGL((multirow_mfma_kernel<D, DV, KVT, PVS, 1, kMrNK, kMrNSet, false, false>),
                           dim3((unsigned)blocks), dim3(512), 0, stream, a, row_blocks);
    return hipGetLastError();
}

template <int KVT, bool PVS>
hipError_t launch_mr_d(const PartialArgs &a, hipStream_t stream)
{
    switch (a.head_dim) {
    case 64: return launch_mr<64, 64, KVT, PVS>(a, stream);
    case 128: return launch_mr<128, 128, KVT, PVS>(a, stream);
    case 192: return launch_mr<192, 128, KVT, PVS>(a, stream);   // the only pair with 192
    default: return launch_mr<256, 256, KVT, PVS>(a, stream);
    }
}

}  // namespace

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

hipError_t launch_partial_multirow(const PartialArgs &a, hipStream_t stream)
{
    if (a.new_k != nullptr && a.n_new > 0)
        return hipErrorInvalidValue;           // the caller appends first for these shapes
    // bf16 pools carry P as hi + lo parts; fp8 pools (tolerance set by their
    // 3-bit mantissa) use the bf16-rounded P alone
    if (a.kv_dtype == NBX_BF16)
        return launch_mr_d<NBX_BF16, true>(a, stream);
    return launch_mr_d<NBX_FP8_E4M3, false>(a, stream);
}

}  // namespace nbx
