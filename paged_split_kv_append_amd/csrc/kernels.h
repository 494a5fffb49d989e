// Internal launch interface between the C-ABI entry points and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nbx_paged.h"

namespace nbx {

struct AppendArgs {
    const void *new_k;
    const void *new_v;          // null: K only
    int32_t src_dtype, dst_dtype;
    int64_t n_tok, new_stride_tok, new_stride_head;
    int32_t kv_heads, head_dim, num_pages, page_tokens;
    // V rows: their own head dim and source strides (the same as K's unless the
    // V pool's head dim differs)
    int32_t v_head_dim;
    int64_t v_new_stride_tok, v_new_stride_head;
    void *k_data;
    int64_t k_stride_page, k_stride_head, k_stride_token;
    void *v_data;
    int64_t v_stride_page, v_stride_head, v_stride_token;
    float k_scale, v_scale;
    // per (page, KV head) bounds raised for every row written (null: none)
    float *k_bounds, *v_bounds;
    const int32_t *slot_mapping;    // null: tail mode (below)
    int32_t *dev_err;
    // tail mode: token t = b * n_new + i goes to position seq_lens[b] - n_new + i
    // of sequence b, its slot read from the block table
    const int32_t *seq_lens, *block_table;
    int32_t max_pages, n_new;
};

struct PartialArgs {
    const void *q;
    int32_t q_dtype, kv_dtype;
    int32_t batch, q_heads, q_rows, causal;
    int32_t kv_heads, group;        // group = q_heads / kv_heads
    int32_t rows_per_kv;            // group * q_rows: rows sharing one KV head
    int32_t head_dim, num_pages, page_tokens;
    int32_t v_head_dim;             // Dv: V rows, partial and output columns
    const void *k_data;
    int64_t k_stride_page, k_stride_head, k_stride_token;
    const void *v_data;
    int64_t v_stride_page, v_stride_head, v_stride_token;
    float k_scale, v_scale;
    // per (page, KV head) bounds: K row norms, V magnitudes (stored units).
    // Both set: fixed-shift softmax where the gate allows; the single-launch
    // step's append raises them for the rows it writes.
    float *k_bounds, *v_bounds;
    const int32_t *block_table;
    int32_t max_pages;
    const int32_t *seq_lens;
    float scale;                    // softmax scale
    int32_t split_size, n_split;
    float *o_part, *m_part, *l_part;
    int32_t *dev_err;
    // ragged windows: rows of sequence b (null: q_rows for every sequence)
    const int32_t *rows_per_seq;
    // single-launch step (persistent decode kernel): the n_new new positions
    // of each sequence, new_k [batch, n_new, kv_heads, head_dim] and new_v
    // [batch, n_new, kv_heads, v_head_dim] of new_dtype, are written by the
    // wave that owns the item holding them
    const void *new_k, *new_v;
    int32_t new_dtype, n_new;
};

// Positions per split: the caller's, or with split_size == 0 the rule of the
// nbxtensor paged_decode_attn.py split kernel evaluated on the device lengths,
// ceil(ceil(max(longest, 1) / n_split) / 16) * 16, so that a recorded launch
// stays right as the lengths grow (lengths clamped to the block-table row).
__device__ inline int device_split_size(const PartialArgs &a)
{
    if (a.split_size > 0)
        return a.split_size;
    const int cap = a.max_pages * a.page_tokens;
    int longest = 1;
    for (int b = 0; b < a.batch; ++b) {
        int L = a.seq_lens[b];
        L = L < 0 ? 0 : (L > cap ? cap : L);
        longest = L > longest ? L : longest;
    }
    const int per = (longest + a.n_split - 1) / a.n_split;
    return (per + 15) / 16 * 16;
}

// Window rows of sequence b: q_rows, or its rows_per_seq entry clamped to
// [0, q_rows] (an entry outside sets NBX_DEVERR_SEQ_RANGE when flag_it)
__device__ inline int seq_window(const PartialArgs &a, int b, bool flag_it)
{
    if (!a.rows_per_seq)
        return a.q_rows;
    int w = a.rows_per_seq[b];
    if (w < 0 || w > a.q_rows) {
        if (flag_it && a.dev_err)
            atomicOr(a.dev_err, NBX_DEVERR_SEQ_RANGE);
        w = w < 0 ? 0 : a.q_rows;
    }
    return w;
}

// Keys seen by window row r of a sequence of L keys whose window has wb rows:
// the window rows are its last wb positions (causal), rows past wb see none
__device__ inline int row_keys(const PartialArgs &a, int L, int wb, int r)
{
    if (r >= wb)
        return 0;
    const int n = a.causal ? L - wb + r + 1 : L;
    return n < 0 ? 0 : n;
}

// The most keys any window row of the sequence sees
__device__ inline int seq_keys(int L, int wb) { return wb > 0 ? L : 0; }

struct MergeArgs {
    const float *o_part, *m_part, *l_part;
    int64_t rows;
    int32_t n_split, head_dim;
    void *out;
    int32_t out_dtype;
};

hipError_t launch_append(const AppendArgs &a, hipStream_t stream);
hipError_t launch_lens_advance(int32_t *seq_lens, int32_t batch, int32_t n, hipStream_t stream);
// bounds of both pools from the rows the sequences hold (zeroed first)
struct BoundsArgs {
    const void *k_data, *v_data;
    int32_t dtype, num_pages, kv_heads, page_tokens, head_dim, v_head_dim;
    int64_t k_stride_page, k_stride_head, k_stride_token;
    int64_t v_stride_page, v_stride_head, v_stride_token;
    float *k_bounds, *v_bounds;
    const int32_t *block_table, *seq_lens;
    int32_t max_pages, batch;
    int32_t *dev_err;
};
// A 1-D launch of `blocks` workgroups of `threads` fits the 32-bit work-item
// count of a dispatch packet; launchers return hipErrorInvalidConfiguration
// (NBX_ERR_UNSUPPORTED at the boundary) when it does not.
inline bool grid_fits(int64_t blocks, int threads)
{
    return blocks >= 0 && blocks * threads <= (int64_t)0xFFFFFFFF;
}
hipError_t launch_kv_bounds(const BoundsArgs &a, hipStream_t stream);
hipError_t launch_partial_valu(const PartialArgs &a, hipStream_t stream);
// matrix-core partials (bf16 / fp8 pools, bf16 Q): more than 16 rows per KV
// head go to launch_partial_multirow
hipError_t launch_partial_mfma(const PartialArgs &a, hipStream_t stream);
hipError_t launch_partial_multirow(const PartialArgs &a, hipStream_t stream);
// true when launch_partial_mfma runs `a` as one persistent launch, so that it
// can also perform the append of a.new_k / a.new_v
bool partial_mfma_is_persistent(const PartialArgs &a);
// row tiles of 16 per wave, and workgroups per (sequence, KV head, split), of
// the multi-row kernel for a KV head serving rows_per_kv rows
int multirow_tiles(int rows_per_kv, int head_dim);
int multirow_row_blocks(int rows_per_kv, int head_dim);
hipError_t launch_merge(const MergeArgs &a, hipStream_t stream);

}  // namespace nbx
