/*
 * nbx_paged.h - C ABI of the paged split-KV attention library for MI355X
 * (gfx950).  Library: libnbx_paged.so.
 *
 * The operation (pages: "nbxtensor attention_wrappers.py" and "nbxtensor
 * paged_decode_attn.py", the paged KV module description, paged_kv_append,
 * paged_decode_attention, decode_reduce; "TensorFold PR #1219" for several
 * query rows sharing the K/V of a KV head):
 *
 *   A per-layer pool per K and per V holds [num_pages, kv_heads, page_tokens,
 *   head_dim] elements; the positions of one KV head inside one page are
 *   consecutive rows.  Sequence b owns the pages block_table[b, 0..]; its
 *   logical position j lives in page block_table[b, j / page_tokens] at row
 *   j % page_tokens.  New positions are written through a slot mapping,
 *   slot = page * page_tokens + row.  A query row of head h attends KV head
 *   h / (q_heads / kv_heads).  The V rows may be narrower than the Q/K rows
 *   (value head dim Dv independent of the query/key head dim D: nbxtensor
 *   attention_wrappers.py, _math_attention's value head_dim, and the D_V of
 *   the split kernel on the nbxtensor paged_decode_attn.py page); outputs
 *   and partial outputs have Dv columns.  The keys are cut into splits of split_size
 *   positions; each split yields an unnormalised partial (o, m, l) with an
 *   fp32 accumulator, and the partials are merged in a fixed order.
 *
 * Conventions shared by every entry point:
 *
 *  - Pointers named in a nbx_kv_pool and every array argument are DEVICE
 *    pointers unless stated; structs themselves are passed by host pointer
 *    and read during the call only.
 *  - Strides are in elements.  The last (head_dim) dimension is contiguous.
 *  - The caller owns and allocates every buffer.  The library allocates and
 *    frees nothing, keeps no state between calls and is re-entrant.
 *  - All device work is enqueued on `stream` (0 = the null stream) without
 *    synchronising; inputs must stay alive until the stream passes the work.
 *  - Host-side validation never reads device memory.  It returns a negative
 *    nbx_status and enqueues nothing on failure; there is no fallback path.
 *  - Data errors that only the device can see (a slot beyond the pool, a
 *    block-table entry outside [0, num_pages) inside a sequence, a sequence
 *    longer than max_pages * page_tokens) are OR-ed into *dev_err when dev_err
 *    is non-null; the offending slot / position is skipped.
 */
#ifndef NBX_PAGED_H
#define NBX_PAGED_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types */
typedef enum {
    NBX_F32 = 0,      /* IEEE binary32 */
    NBX_BF16 = 1,     /* bfloat16: the upper 16 bits of a binary32 */
    NBX_FP8_E4M3 = 2  /* OCP E4M3FN: bias 7, no infinity, 0x7F/0xFF NaN, max 448 */
} nbx_dtype;

/* status codes (return values) */
typedef enum {
    NBX_OK = 0,
    NBX_ERR_NULL_PTR = -1,      /* a required pointer is null */
    NBX_ERR_BAD_DTYPE = -2,     /* dtype code unknown or combination not supported */
    NBX_ERR_BAD_SHAPE = -3,     /* sizes inconsistent (e.g. q_heads % kv_heads != 0,
                                   head_dim not in {64, 128, 256}, K/V pools differ) */
    NBX_ERR_BAD_ALIGN = -4,     /* page_tokens % 16, split_size % 16, split_size *
                                   n_split < the longest sequence, unit stride broken */
    NBX_ERR_WORKSPACE = -5,     /* workspace too small */
    NBX_ERR_UNSUPPORTED = -6,   /* valid request this build does not implement, or
                                   whose grid exceeds the 2^32 work-items of one
                                   dispatch */
    NBX_ERR_LAUNCH = -7,        /* the HIP runtime refused a kernel launch */
    NBX_ERR_SCRATCH_LIMIT = -8  /* the partials of the request need more than the
                                   library's static scratch holds
                                   (NBX_STEP_SCRATCH_BYTES) */
} nbx_status;

/* device-side data error bits OR-ed into *dev_err */
#define NBX_DEVERR_SLOT_RANGE 0x1   /* append: slot >= num_pages * page_tokens */
#define NBX_DEVERR_PAGE_RANGE 0x2   /* read: block-table entry outside [0, num_pages) */
#define NBX_DEVERR_SEQ_RANGE 0x4    /* read: seq_len > max_pages * page_tokens, or < 0 */

/* A paged K or V pool: data[page * stride_page + head * stride_head +
 * row * stride_token + e] for e in [0, head_dim).  `scale` multiplies every
 * stored element when read (fp8 per-tensor dequantisation factor; 1.0 for
 * fp32 / bf16 pools) and divides a value before it is stored by an append.
 *
 * `bounds` (device fp32 [num_pages, kv_heads], or null) carries, per page and
 * KV head, an upper bound of what the rows read from it hold, in stored units
 * (before `scale`): for a K pool the Euclidean norm of a row, for a V pool
 * the magnitude of an element.  NaN means unknown.  nbx_paged_kv_bounds
 * computes them from the rows the sequences hold; every append (slot
 * mapping or decode step) raises them for the rows it writes.  A caller that
 * writes a pool by other means, or hands a page to another sequence, must
 * recompute them.  When both pools of a read carry bounds, the split kernels
 * use the fixed-shift softmax of the maxdiffusion PR #477 page (fixed-m
 * splash attention, dynamic bounds): each query row i of a split subtracts
 * the precomputed shift m_i = ceil(U_i) - C(N) instead of a running maximum,
 * with U_i = |scale * k_scale| * log2(e) * |q_i| * (largest K bound of the
 * split's pages) (an upper bound of |q_i . k_j| in log2 units, enlarged by
 * 2^-12 for rounding), C(N) = 127 - ceil(log2 N) - ceil(log2 Vmax),
 * N = the sequence length, Vmax = max(1, largest V bound of the split's
 * pages * max(1, v_scale)).  A group of 16 rows uses the shift only if every
 * row passes the gate ceil(U_i) <= floor((C(N) + 125) / 2); otherwise (and
 * for NaN or infinite bounds) it keeps the running maximum.  Results agree
 * with the running-maximum form to rounding; a split's m_part then holds the
 * shift (natural-log units) instead of the split's largest score, which the
 * merge handles alike.  Kernels that use it: the single-launch decode kernel
 * (<= 16 rows per KV head, batch <= 256) and the multi-row kernel; the others
 * ignore the bounds. */
typedef struct {
    void *data;             /* device pointer */
    int32_t dtype;          /* nbx_dtype */
    int32_t num_pages;
    int32_t kv_heads;
    int32_t page_tokens;    /* a multiple of 16 */
    int32_t head_dim;       /* 64, 128, 192 or 256; a K / V pair of a read is
                               (64, 64), (128, 128), (256, 256) or (192, 128) */
    int64_t stride_page;    /* elements; head_dim <= stride_token <= 2^24 */
    int64_t stride_head;
    int64_t stride_token;
    float scale;
    float *bounds;          /* device [num_pages, kv_heads] or null (see above) */
} nbx_kv_pool;

/*
 * nbx_paged_kv_append - write new positions into the K and V pools through a
 * slot mapping (nbxtensor paged_decode_attn.py, paged_kv_append_kernel;
 * nbxtensor attention_wrappers.py, paged_kv_append).
 *
 *   new_k, new_v   device, [n_tok, kv_heads, head_dim] of new_dtype, element
 *                  (t, h, e) at t * new_stride_tok + h * new_stride_head + e.
 *                  new_v (and v_pool) may be null to write K only.  Both
 *                  pools of one call have the same head_dim (else
 *                  NBX_ERR_BAD_SHAPE): pools of different head dims are
 *                  written by two calls, each with one pool as k_pool.
 *   new_dtype      NBX_F32 or NBX_BF16.
 *   slot_mapping   device int32 [n_tok]; slot = page * page_tokens + row.
 *                  A negative slot is skipped (padding).  A slot at or beyond
 *                  num_pages * page_tokens is skipped and sets
 *                  NBX_DEVERR_SLOT_RANGE.  Two equal slots: unspecified winner.
 *
 * Stored value: same dtype -> bit copy; fp32 -> bf16 round-to-nearest-even
 * (NaN -> 0x7FC0 with the sign kept); bf16 -> fp32 exact; to fp8:
 * round-to-nearest-even of the fp32 quotient value / pool.scale, saturating at
 * +-448, NaN -> 0x7F with the sign kept.  n_tok == 0 is a no-op.  A pool with
 * bounds gets bounds[page, head] raised to the stored row's norm (K) or
 * largest |element| (V).
 */
int nbx_paged_kv_append(const void *new_k, const void *new_v, int32_t new_dtype, int64_t n_tok,
                        int64_t new_stride_tok, int64_t new_stride_head,
                        const nbx_kv_pool *k_pool, const nbx_kv_pool *v_pool,
                        const int32_t *slot_mapping, int32_t *dev_err, hipStream_t stream);

/*
 * nbx_paged_kv_bounds - recompute the bounds arrays of both pools (see
 * nbx_kv_pool) from the rows the sequences hold: bounds[page, h] = the
 * largest K row norm / |V element| over the rows (page, h, j % page_tokens)
 * with page = block_table[b, j / page_tokens], j < seq_lens[b]; 0 for pages
 * no sequence holds.  Both pools need bounds (else NBX_ERR_NULL_PTR) and the
 * layout rules of a read.  A block-table entry outside the pool sets
 * NBX_DEVERR_PAGE_RANGE and is skipped; a length outside [0, max_pages *
 * page_tokens] sets NBX_DEVERR_SEQ_RANGE and is clamped.  Reads every held
 * K and V element once.
 */
int nbx_paged_kv_bounds(const nbx_kv_pool *k_pool, const nbx_kv_pool *v_pool,
                        const int32_t *block_table, int32_t max_pages, const int32_t *seq_lens,
                        int32_t batch, int32_t *dev_err, hipStream_t stream);

/*
 * nbx_paged_decode_plan - host only.  The split rule of the nbxtensor
 * paged_decode_attn.py page (paged_decode_splits and the kernel's seg_len):
 *   n_split    = max(1, min(ceil(longest / split_positions), max_splits))
 *   split_size = ceil(ceil(longest / n_split) / 16) * 16
 * with longest = max(max_seq_len, 1).  The pages use split_positions = 256
 * and max_splits = 64.  split_positions, max_splits > 0 or NBX_ERR_BAD_SHAPE.
 */
int nbx_paged_decode_plan(int32_t max_seq_len, int32_t split_positions, int32_t max_splits,
                          int32_t *n_split, int32_t *split_size);

/*
 * nbx_paged_decode_plan_rows - host only.  A split plan that also looks at the
 * rows per KV head, rows_per_kv = (q_heads / kv_heads) * q_rows.  At most 16
 * (decode): nbx_paged_decode_plan(max_seq_len, 256, 64).  More (verify
 * windows, prompt chunks): each (sequence, KV head, split, block of 128 or
 * 256 rows) is one workgroup of the multi-row kernel, which holds a compute
 * unit alone, so
 *   n_split    = clamp(floor(CUs / (batch * kv_heads * row_blocks)), 1,
 *                      min(64, ceil(longest / 16)))
 *   split_size = ceil(ceil(longest / n_split) / 16) * 16
 * with CUs the current device's compute units: the workgroups fill the
 * device in one round, and the fewest splits that do so keep the partials
 * (rows * n_split * (Dv + 2) * 4 bytes, written and read back) small.
 * Reads the device attribute only.  NBX_ERR_BAD_SHAPE for sizes < 1,
 * q_heads % kv_heads != 0 or an unsupported head_dim (of q and k);
 * NBX_ERR_LAUNCH if the device cannot be queried.
 */
int nbx_paged_decode_plan_rows(int32_t batch, int32_t q_heads, int32_t kv_heads, int32_t q_rows,
                               int32_t head_dim, int32_t max_seq_len, int32_t *n_split,
                               int32_t *split_size);

/* nbx_paged_decode_workspace_bytes - host only.  Bytes of workspace that
 * nbx_paged_decode needs for `rows` query rows: the partials o [rows,
 * n_split, head_dim], m and l [rows, n_split], fp32, each 256-byte aligned.
 * head_dim is the V pool's (the width of o). */
size_t nbx_paged_decode_workspace_bytes(int64_t rows, int32_t n_split, int32_t head_dim);

/*
 * nbx_paged_decode_partial - the split partials (nbxtensor paged_decode_attn.py,
 * paged_decode_attn_split_kernel; several rows per KV head as in TensorFold
 * PR #1219).
 *
 *   q            device, [batch, q_heads, q_rows, head_dim] contiguous, NBX_F32
 *                or NBX_BF16 (read exactly, never rounded).  Query row index
 *                row = (b * q_heads + h) * q_rows + r.  At most 2^24 rows per
 *                KV head ((q_heads / kv_heads) * q_rows), else
 *                NBX_ERR_UNSUPPORTED.
 *   causal       0: every row of sequence b sees keys [0, seq_lens[b]).
 *                1: row r sees keys [0, seq_lens[b] - q_rows + r], i.e. the
 *                q_rows rows are the last q_rows positions of the sequence,
 *                already in the pool.
 *   k_pool/v_pool  same dtype, num_pages, kv_heads, page_tokens; head dims
 *                D (of q and K) and Dv (of V) one of the pairs listed at
 *                nbx_kv_pool.  q is [.., D]; o_part and the output [.., Dv].
 *   block_table  device int32 [batch, max_pages] (row stride max_pages), -1
 *                past each sequence.  Entries covering [0, seq_lens[b]) must
 *                lie in [0, num_pages); a violation sets NBX_DEVERR_PAGE_RANGE
 *                and that page's positions are skipped.
 *   seq_lens     device int32 [batch]; positions held by each sequence.
 *   scale        softmax scale applied to q . k (after pool.scale).
 *   split_size   positions per split, a multiple of 16; split s covers
 *                [s * split_size, min((s + 1) * split_size, n)) of the keys a
 *                row sees.  split_size * n_split must cover every sequence
 *                (not checkable on the host: longer sequences set
 *                NBX_DEVERR_SEQ_RANGE and their tail is not read).
 *                split_size == 0: derived on the device at every launch from
 *                the lengths, ceil(ceil(max(longest, 1) / n_split) / 16) * 16
 *                (the split kernel's rule on the nbxtensor paged_decode_attn.py
 *                page), so a launch recorded in a graph stays right as the
 *                lengths grow; n_split then only bounds the split count.
 *   o_part       device fp32 [rows, n_split, Dv]: sum_j exp(s_j - m) v_j
 *   m_part       device fp32 [rows, n_split]: max_j s_j (natural-log units)
 *   l_part       device fp32 [rows, n_split]: sum_j exp(s_j - m)
 *                where s_j = scale * pool.scale_k * (q . k_j) over the split.
 *                An empty split (no key of the row in it) stores m = -inf and
 *                l = 0; its o is left unwritten (the merge never reads it).
 *
 * Supported: pool dtype NBX_F32 with any q dtype; NBX_BF16 or NBX_FP8_E4M3
 * pools with NBX_BF16 or NBX_F32 q; n_split and batch * kv_heads each at
 * most 65535 and batch * kv_heads * n_split below 2^31 (else
 * NBX_ERR_BAD_SHAPE / NBX_ERR_UNSUPPORTED).
 */
int nbx_paged_decode_partial(const void *q, int32_t q_dtype, int32_t batch, int32_t q_heads,
                             int32_t q_rows, int32_t causal, const nbx_kv_pool *k_pool,
                             const nbx_kv_pool *v_pool, const int32_t *block_table,
                             int32_t max_pages, const int32_t *seq_lens, float scale,
                             int32_t split_size, int32_t n_split, float *o_part, float *m_part,
                             float *l_part, int32_t *dev_err, hipStream_t stream);

/*
 * nbx_paged_decode_partial_windows - split partials for a batch whose
 * sequences carry windows of different lengths (several streams' verify
 * windows in one launch, the ragged case of TensorFold PR #1219's contract).
 *
 *   q_rows        the longest window: q is [batch, q_heads, q_rows, head_dim]
 *                 with each sequence's window in its first rows.
 *   rows_per_seq  device int32 [batch]: window rows of sequence b, in
 *                 [0, q_rows] (an entry outside is clamped and sets
 *                 NBX_DEVERR_SEQ_RANGE).  Causal: row r < rows_per_seq[b] is
 *                 position seq_lens[b] - rows_per_seq[b] + r and sees keys up to
 *                 it; rows r >= rows_per_seq[b] are padding, every split of
 *                 theirs stores m = -inf, l = 0 (their merged output is 0).
 * Other arguments, layouts and errors as for nbx_paged_decode_partial.
 */
int nbx_paged_decode_partial_windows(const void *q, int32_t q_dtype, int32_t batch,
                                     int32_t q_heads, int32_t q_rows,
                                     const int32_t *rows_per_seq, int32_t causal,
                                     const nbx_kv_pool *k_pool, const nbx_kv_pool *v_pool,
                                     const int32_t *block_table, int32_t max_pages,
                                     const int32_t *seq_lens, float scale, int32_t split_size,
                                     int32_t n_split, float *o_part, float *m_part,
                                     float *l_part, int32_t *dev_err, hipStream_t stream);

/*
 * nbx_paged_decode_merge - fixed-order combine of split partials (nbxtensor
 * attention_wrappers.py, decode_reduce): per row, M = the largest m_s of the
 * non-empty splits (m_s != -inf; the o of an empty split is not read),
 * w_s = exp(m_s - M), and
 *   out = sum_s w_s o_s / sum_s w_s l_s,
 * summed in a fixed order that depends only on n_split (each group of splits
 * in ascending s, the groups then added pairwise in a fixed tree), so repeated
 * calls give identical bits.  A row with no non-empty split is 0.  NaN in a
 * partial propagates to the row.
 *
 *   o_part, m_part, l_part  as written by nbx_paged_decode_partial.
 *   out          device [rows, head_dim] of out_dtype (NBX_F32 or NBX_BF16,
 *                bf16 rounded to nearest even); head_dim is the partials'
 *                width Dv, 64, 128 or 256.
 *   n_split      at most 4096, else NBX_ERR_UNSUPPORTED.
 *   rows         below 2^24 (one 256-thread workgroup per row), else
 *                NBX_ERR_UNSUPPORTED.
 */
int nbx_paged_decode_merge(const float *o_part, const float *m_part, const float *l_part,
                           int64_t rows, int32_t n_split, int32_t head_dim, void *out,
                           int32_t out_dtype, hipStream_t stream);

/*
 * nbx_paged_decode - partial then merge on one stream (nbxtensor
 * attention_wrappers.py, paged_decode_attention).  Arguments as for the two
 * calls; `workspace` (device, at least nbx_paged_decode_workspace_bytes(rows,
 * n_split, Dv) bytes, 256-byte aligned) holds the partials; out is
 * [batch, q_heads, q_rows, Dv].
 */
int nbx_paged_decode(const void *q, int32_t q_dtype, int32_t batch, int32_t q_heads,
                     int32_t q_rows, int32_t causal, const nbx_kv_pool *k_pool,
                     const nbx_kv_pool *v_pool, const int32_t *block_table, int32_t max_pages,
                     const int32_t *seq_lens, float scale, int32_t split_size, int32_t n_split,
                     void *workspace, size_t workspace_bytes, void *out, int32_t out_dtype,
                     int32_t *dev_err, hipStream_t stream);

/*
 * nbx_paged_decode_step - one decode step: append the new tokens of every
 * sequence at its last positions, then partial and merge (nbxtensor
 * paged_decode_attn.py, paged_kv_append_step_kernel: the step's position is
 * found on the device from the sequence length and its page from the block
 * table, so the call's arguments do not change from step to step; then
 * paged_decode_attn_split_kernel and nbxtensor attention_wrappers.py,
 * decode_reduce).  Here seq_lens already count the new positions (the pages
 * advance the length in a separate launch after the append).
 *
 * Equivalent to nbx_paged_kv_append with slot_mapping[b * n_new + i] = the
 * slot of position seq_lens[b] - n_new + i of sequence b (read from the block
 * table on the device), followed by nbx_paged_decode with the same arguments.
 * seq_lens count the new positions.  Where the shape allows (bf16 Q, bf16 or
 * fp8 pool, at most 16 rows per KV head, batch <= 256) the whole step is one
 * kernel launch; otherwise the append, partial and merge kernels run in turn
 * on `stream`.
 *
 *   new_k, new_v   device, new_k [batch, n_new, kv_heads, D] and new_v
 *                  [batch, n_new, kv_heads, Dv], contiguous, of new_dtype
 *                  (NBX_F32 or NBX_BF16); stored with the conversions of
 *                  nbx_paged_kv_append.  Ignored if n_new == 0.
 *   n_new          new positions per sequence (>= 0).  A sequence shorter
 *                  than n_new sets NBX_DEVERR_SEQ_RANGE and its tokens that
 *                  would land before position 0 are skipped; a block-table
 *                  entry outside the pool sets NBX_DEVERR_PAGE_RANGE and that
 *                  token is skipped.  The slots of the new positions must not
 *                  be read by another sequence of the same call.
 *   workspace      as for nbx_paged_decode.  It holds the partials afterwards:
 *                  o at offset 0, m at round256(rows * n_split * Dv * 4),
 *                  l after m at round256(rows * n_split * 4), the layouts of
 *                  nbx_paged_decode_partial (round256 = next multiple of 256).
 *   out            may be null: the step then stops after the partials (for a
 *                  caller that merges later, e.g. after gathering the partials
 *                  of other position ranges) and out_dtype is ignored.
 * Other arguments, errors and results as for nbx_paged_decode.
 */
int nbx_paged_decode_step(const void *q, int32_t q_dtype, int32_t batch, int32_t q_heads,
                          int32_t q_rows, int32_t causal, const void *new_k, const void *new_v,
                          int32_t new_dtype, int32_t n_new, const nbx_kv_pool *k_pool,
                          const nbx_kv_pool *v_pool, const int32_t *block_table,
                          int32_t max_pages, const int32_t *seq_lens, float scale,
                          int32_t split_size, int32_t n_split, void *workspace,
                          size_t workspace_bytes, void *out, int32_t out_dtype, int32_t *dev_err,
                          hipStream_t stream);

/* Bytes of the device scratch of nbx_paged_decode_step_noalloc (32 MiB). */
#define NBX_STEP_SCRATCH_BYTES ((size_t)32 << 20)

/*
 * nbx_paged_decode_step_noalloc - nbx_paged_decode_step for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same append, partial and
 * merge, with the split partials kept in a static device array of the
 * library, NBX_STEP_SCRATCH_BYTES per GPU, instead of a caller workspace.
 * The call itself allocates nothing (no hipMalloc, hipFree or allocating
 * library routine); each GPU the library runs on holds the array from the
 * loading of the library's code on it until the process ends.
 *
 *   out    required (NBX_ERR_NULL_PTR if null): the partials are internal.
 * Other arguments, errors and results as for nbx_paged_decode_step.  A request
 * whose partials, nbx_paged_decode_workspace_bytes(batch * q_heads * q_rows,
 * n_split, Dv), exceed NBX_STEP_SCRATCH_BYTES returns NBX_ERR_SCRATCH_LIMIT
 * before any launch (1024 rows at Dv = 128 take up to 63 splits).  The first
 * call on a device looks the array's address up (hipGetSymbolAddress) with
 * that device current; NBX_ERR_LAUNCH if that fails.
 *
 * Every call on one GPU uses that GPU's one array, which keeps the last
 * call's partials: calls that overlap on one GPU (on different streams, or
 * from different threads without ordering) race and give wrong results.
 * Calls on one stream run in turn and are safe.
 */
int nbx_paged_decode_step_noalloc(const void *q, int32_t q_dtype, int32_t batch, int32_t q_heads,
                                  int32_t q_rows, int32_t causal, const void *new_k,
                                  const void *new_v, int32_t new_dtype, int32_t n_new,
                                  const nbx_kv_pool *k_pool, const nbx_kv_pool *v_pool,
                                  const int32_t *block_table, int32_t max_pages,
                                  const int32_t *seq_lens, float scale, int32_t split_size,
                                  int32_t n_split, void *out, int32_t out_dtype, int32_t *dev_err,
                                  hipStream_t stream);

/*
 * nbx_paged_lens_advance - seq_lens[b] += n for 0 <= b < batch, on the device
 * (nbxtensor paged_decode_attn.py, paged_lens_advance_kernel: the length of a
 * decode step moves on the device, so a recorded step replays unchanged).
 *   seq_lens  device int32 [batch].  batch == 0 is a no-op; batch < 0 gives
 *             NBX_ERR_BAD_SHAPE.  Overflow of an int32 length is the caller's.
 */
int nbx_paged_lens_advance(int32_t *seq_lens, int32_t batch, int32_t n, hipStream_t stream);

/* nbx_status_str - static message text for a status code (never null). */
const char *nbx_status_str(int status);

/* nbx_version - library version as major * 10000 + minor * 100 + patch. */
int nbx_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NBX_PAGED_H */
