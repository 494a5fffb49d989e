// C-ABI entry points of libnbx_paged: host validation, the split plan, the
// workspace layout and kernel dispatch.  Nothing here reads device memory or
// allocates; every launch goes to the caller's stream.
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

#include "kernels.h"
#include "nbx_paged.h"

namespace {

constexpr int kMaxGridYZ = 65535;
constexpr int kMaxMergeSplits = 4096;   // the most splits the merge takes (past 64 it loops)

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

bool dtype_ok(int32_t d) { return d == NBX_F32 || d == NBX_BF16 || d == NBX_FP8_E4M3; }

// head dims of one pool; a V pool's (the partial and output width) is one of
// 64, 128, 256
bool head_dim_ok(int32_t d) { return d == 64 || d == 128 || d == 192 || d == 256; }
bool value_dim_ok(int32_t d) { return d == 64 || d == 128 || d == 256; }

// (q/k head dim, v head dim) pairs the partial kernels are built for: equal
// dims, or the latent-attention pair 192 / 128
bool head_dims_ok(int32_t dk, int32_t dv)
{
    return (dk == dv && value_dim_ok(dk)) || (dk == 192 && dv == 128);
}

// geometry and alignment of one pool; returns NBX_OK or an error
int check_pool(const nbx_kv_pool *p)
{
    if (!p || !p->data)
        return NBX_ERR_NULL_PTR;
    if (!dtype_ok(p->dtype))
        return NBX_ERR_BAD_DTYPE;
    if (p->num_pages < 1 || p->kv_heads < 1 || !head_dim_ok(p->head_dim))
        return NBX_ERR_BAD_SHAPE;
    if (p->page_tokens < 16 || p->page_tokens % 16)
        return NBX_ERR_BAD_ALIGN;
    if (p->stride_token < p->head_dim || p->stride_head < 0 || p->stride_page < 0)
        return NBX_ERR_BAD_SHAPE;
    // the kernels address the rows of a 16-row tile with 32-bit byte offsets
    if (p->stride_token > ((int64_t)1 << 24))
        return NBX_ERR_BAD_SHAPE;
    // 16-element strides and 16-byte base: every K/V row starts 16-byte aligned
    if (p->stride_token % 16 || p->stride_head % 16 || p->stride_page % 16 || !aligned16(p->data))
        return NBX_ERR_BAD_ALIGN;
    if (!(p->scale > 0.0f) || p->scale == INFINITY)
        return NBX_ERR_BAD_SHAPE;
    if ((uintptr_t)p->bounds & 3u)
        return NBX_ERR_BAD_ALIGN;
    return NBX_OK;
}

// the same pages, heads, positions and element type (head dims checked apart)
bool same_layout(const nbx_kv_pool *a, const nbx_kv_pool *b)
{
    return a->dtype == b->dtype && a->num_pages == b->num_pages && a->kv_heads == b->kv_heads &&
           a->page_tokens == b->page_tokens;
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// a grid beyond the dispatch limit (see grid_fits) is a request this build
// does not serve; any other launch error is reported as such
int to_status(hipError_t e)
{
    if (e == hipSuccess)
        return NBX_OK;
    return e == hipErrorInvalidConfiguration ? NBX_ERR_UNSUPPORTED : NBX_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int nbx_version(void) { return 100; }

const char *nbx_status_str(int status)
{
    switch (status) {
    case NBX_OK: return "ok";
    case NBX_ERR_NULL_PTR: return "a required pointer is null";
    case NBX_ERR_BAD_DTYPE: return "unknown or unsupported element type";
    case NBX_ERR_BAD_SHAPE: return "inconsistent sizes";
    case NBX_ERR_BAD_ALIGN: return "alignment: page_tokens / split_size not a multiple of 16, "
                                   "strides not multiples of 16 elements, or a pointer not "
                                   "16-byte aligned";
    case NBX_ERR_WORKSPACE: return "workspace too small or misaligned";
    case NBX_ERR_UNSUPPORTED: return "request not supported by this build";
    case NBX_ERR_LAUNCH: return "kernel launch failed";
    case NBX_ERR_SCRATCH_LIMIT: return "request needs more than the static scratch holds";
    default: return "unknown status";
    }
}

int nbx_paged_decode_plan(int32_t max_seq_len, int32_t split_positions, int32_t max_splits,
                          int32_t *n_split, int32_t *split_size)
{
    if (!n_split || !split_size)
        return NBX_ERR_NULL_PTR;
    if (split_positions <= 0 || max_splits <= 0)
        return NBX_ERR_BAD_SHAPE;
    const int64_t longest = max_seq_len < 1 ? 1 : max_seq_len;
    int64_t n = (longest + split_positions - 1) / split_positions;
    if (n > max_splits)
        n = max_splits;
    if (n < 1)
        n = 1;
    const int64_t per = (longest + n - 1) / n;
    *n_split = (int32_t)n;
    *split_size = (int32_t)((per + 15) / 16 * 16);
    return NBX_OK;
}

int nbx_paged_decode_plan_rows(int32_t batch, int32_t q_heads, int32_t kv_heads, int32_t q_rows,
                               int32_t head_dim, int32_t max_seq_len, int32_t *n_split,
                               int32_t *split_size)
{
    if (!n_split || !split_size)
        return NBX_ERR_NULL_PTR;
    if (batch < 1 || q_heads < 1 || kv_heads < 1 || q_rows < 1 || q_heads % kv_heads ||
        !head_dim_ok(head_dim))
        return NBX_ERR_BAD_SHAPE;
    const int64_t rows_per_kv = (int64_t)(q_heads / kv_heads) * q_rows;
    if (rows_per_kv <= 16)
        return nbx_paged_decode_plan(max_seq_len, 256, 64, n_split, split_size);
    if (rows_per_kv > INT32_MAX)
        return NBX_ERR_BAD_SHAPE;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 1)
        return NBX_ERR_LAUNCH;
    const int64_t units = (int64_t)batch * kv_heads *
                          nbx::multirow_row_blocks((int)rows_per_kv, head_dim);
    const int64_t longest = max_seq_len < 1 ? 1 : max_seq_len;
    int64_t n = cus / units;                   // workgroups within one round of the CUs
    const int64_t tiles = (longest + 15) / 16;
    if (n > 64)
        n = 64;
    if (n > tiles)
        n = tiles;
    if (n < 1)
        n = 1;
    const int64_t per = (longest + n - 1) / n;
    *n_split = (int32_t)n;
    *split_size = (int32_t)((per + 15) / 16 * 16);
    return NBX_OK;
}

size_t nbx_paged_decode_workspace_bytes(int64_t rows, int32_t n_split, int32_t head_dim)
{
    if (rows <= 0 || n_split <= 0 || head_dim <= 0)
        return 0;
    const size_t o = (size_t)rows * n_split * head_dim * sizeof(float);
    const size_t ml = (size_t)rows * n_split * sizeof(float);
    return round256(o) + 2 * round256(ml);
}

int nbx_paged_kv_bounds(const nbx_kv_pool *k_pool, const nbx_kv_pool *v_pool,
                        const int32_t *block_table, int32_t max_pages, const int32_t *seq_lens,
                        int32_t batch, int32_t *dev_err, hipStream_t stream)
{
    if (!k_pool || !v_pool || !block_table || !seq_lens)
        return NBX_ERR_NULL_PTR;
    int st = check_pool(k_pool);
    if (st != NBX_OK)
        return st;
    if ((st = check_pool(v_pool)) != NBX_OK)
        return st;
    if (!k_pool->bounds || !v_pool->bounds)
        return NBX_ERR_NULL_PTR;
    if (!same_layout(k_pool, v_pool) || !head_dims_ok(k_pool->head_dim, v_pool->head_dim))
        return NBX_ERR_BAD_SHAPE;
    if (batch < 0 || max_pages < 1)
        return NBX_ERR_BAD_SHAPE;
    if (batch > kMaxGridYZ || max_pages > kMaxGridYZ ||
        (int64_t)max_pages * k_pool->page_tokens > INT32_MAX)
        return NBX_ERR_UNSUPPORTED;
    nbx::BoundsArgs a{};
    a.k_data = k_pool->data;
    a.v_data = v_pool->data;
    a.dtype = k_pool->dtype;
    a.num_pages = k_pool->num_pages;
    a.kv_heads = k_pool->kv_heads;
    a.page_tokens = k_pool->page_tokens;
    a.head_dim = k_pool->head_dim;
    a.v_head_dim = v_pool->head_dim;
    a.k_stride_page = k_pool->stride_page;
    a.k_stride_head = k_pool->stride_head;
    a.k_stride_token = k_pool->stride_token;
    a.v_stride_page = v_pool->stride_page;
    a.v_stride_head = v_pool->stride_head;
    a.v_stride_token = v_pool->stride_token;
    a.k_bounds = k_pool->bounds;
    a.v_bounds = v_pool->bounds;
    a.block_table = block_table;
    a.seq_lens = seq_lens;
    a.max_pages = max_pages;
    a.batch = batch;
    a.dev_err = dev_err;
    return to_status(nbx::launch_kv_bounds(a, stream));
}

int nbx_paged_lens_advance(int32_t *seq_lens, int32_t batch, int32_t n, hipStream_t stream)
{
    if (!seq_lens)
        return NBX_ERR_NULL_PTR;
    if (batch < 0)
        return NBX_ERR_BAD_SHAPE;
    return to_status(nbx::launch_lens_advance(seq_lens, batch, n, stream));
}

int nbx_paged_kv_append(const void *new_k, const void *new_v, int32_t new_dtype, int64_t n_tok,
                        int64_t new_stride_tok, int64_t new_stride_head,
                        const nbx_kv_pool *k_pool, const nbx_kv_pool *v_pool,
                        const int32_t *slot_mapping, int32_t *dev_err, hipStream_t stream)
{
    if (!new_k || !k_pool || !slot_mapping)
        return NBX_ERR_NULL_PTR;
    if ((new_v == nullptr) != (v_pool == nullptr))
        return NBX_ERR_NULL_PTR;
    if (new_dtype != NBX_F32 && new_dtype != NBX_BF16)
        return NBX_ERR_BAD_DTYPE;
    int st = check_pool(k_pool);
    if (st != NBX_OK)
        return st;
    if (v_pool) {
        if ((st = check_pool(v_pool)) != NBX_OK)
            return st;
        // one pair of source strides serves both: pools of different head
        // dims are appended in two calls
        if (!same_layout(k_pool, v_pool) || k_pool->head_dim != v_pool->head_dim)
            return NBX_ERR_BAD_SHAPE;
    }
    if (n_tok < 0 || new_stride_head < k_pool->head_dim || new_stride_tok < 0)
        return NBX_ERR_BAD_SHAPE;
    if (new_stride_tok % 8 || new_stride_head % 8 || !aligned16(new_k) ||
        (new_v && !aligned16(new_v)))
        return NBX_ERR_BAD_ALIGN;
    if (n_tok == 0)
        return NBX_OK;
    if (n_tok * k_pool->kv_heads * (k_pool->head_dim / 8) > (int64_t)INT32_MAX * 256)
        return NBX_ERR_BAD_SHAPE;

    nbx::AppendArgs a{};
    a.new_k = new_k;
    a.new_v = new_v;
    a.src_dtype = new_dtype;
    a.dst_dtype = k_pool->dtype;
    a.n_tok = n_tok;
    a.new_stride_tok = new_stride_tok;
    a.new_stride_head = new_stride_head;
    a.kv_heads = k_pool->kv_heads;
    a.head_dim = k_pool->head_dim;
    a.v_head_dim = k_pool->head_dim;
    a.v_new_stride_tok = new_stride_tok;
    a.v_new_stride_head = new_stride_head;
    a.num_pages = k_pool->num_pages;
    a.page_tokens = k_pool->page_tokens;
    a.k_data = k_pool->data;
    a.k_stride_page = k_pool->stride_page;
    a.k_stride_head = k_pool->stride_head;
    a.k_stride_token = k_pool->stride_token;
    a.k_scale = k_pool->scale;
    a.k_bounds = k_pool->bounds;
    if (v_pool) {
        a.v_data = v_pool->data;
        a.v_stride_page = v_pool->stride_page;
        a.v_stride_head = v_pool->stride_head;
        a.v_stride_token = v_pool->stride_token;
        a.v_scale = v_pool->scale;
        a.v_bounds = v_pool->bounds;
    }
    a.slot_mapping = slot_mapping;
    a.dev_err = dev_err;
    return to_status(nbx::launch_append(a, stream));
}

static int validate_partial(const void *q, int32_t q_dtype, int32_t batch, int32_t q_heads,
                            int32_t q_rows, int32_t causal, const nbx_kv_pool *k_pool,
                            const nbx_kv_pool *v_pool, const int32_t *block_table,
                            int32_t max_pages, const int32_t *seq_lens, float scale,
                            int32_t split_size, int32_t n_split)
{
    if (!q || !k_pool || !v_pool || !block_table || !seq_lens)
        return NBX_ERR_NULL_PTR;
    if (q_dtype != NBX_F32 && q_dtype != NBX_BF16)
        return NBX_ERR_BAD_DTYPE;
    int st = check_pool(k_pool);
    if (st != NBX_OK)
        return st;
    if ((st = check_pool(v_pool)) != NBX_OK)
        return st;
    if (!same_layout(k_pool, v_pool) || !head_dims_ok(k_pool->head_dim, v_pool->head_dim))
        return NBX_ERR_BAD_SHAPE;
    if (batch < 0 || q_heads < 1 || q_rows < 1 || max_pages < 1 || (causal != 0 && causal != 1))
        return NBX_ERR_BAD_SHAPE;
    if (q_heads % k_pool->kv_heads)
        return NBX_ERR_BAD_SHAPE;
    if ((int64_t)(q_heads / k_pool->kv_heads) * q_rows > ((int64_t)1 << 24))
        return NBX_ERR_UNSUPPORTED;            // rows per KV head are counted in 32 bits
    if (scale != scale || scale == INFINITY || scale == -INFINITY)
        return NBX_ERR_BAD_SHAPE;
    if (split_size < 0 || split_size % 16)   // 0: derived on the device from seq_lens
        return NBX_ERR_BAD_ALIGN;
    if (n_split < 1 || n_split > kMaxGridYZ)
        return NBX_ERR_BAD_SHAPE;
    if ((int64_t)batch * k_pool->kv_heads > kMaxGridYZ)
        return NBX_ERR_UNSUPPORTED;
    // (sequence, KV head, split) units are counted and enumerated in 32 bits
    if ((int64_t)batch * k_pool->kv_heads * n_split > INT32_MAX)
        return NBX_ERR_UNSUPPORTED;
    if ((int64_t)split_size * n_split > INT32_MAX || (int64_t)max_pages * k_pool->page_tokens > INT32_MAX)
        return NBX_ERR_BAD_SHAPE;
    if (!aligned16(q))
        return NBX_ERR_BAD_ALIGN;
    return NBX_OK;
}

static nbx::PartialArgs partial_args(const void *q, int32_t q_dtype, int32_t batch,
                                     int32_t q_heads, int32_t q_rows, int32_t causal,
                                     const nbx_kv_pool *k_pool, const nbx_kv_pool *v_pool,
                                     const int32_t *block_table, int32_t max_pages,
                                     const int32_t *seq_lens, float scale, int32_t split_size,
                                     int32_t n_split, float *o_part, float *m_part, float *l_part,
                                     int32_t *dev_err)
{
    nbx::PartialArgs a{};
    a.q = q;
    a.q_dtype = q_dtype;
    a.kv_dtype = k_pool->dtype;
    a.batch = batch;
    a.q_heads = q_heads;
    a.q_rows = q_rows;
    a.causal = causal;
    a.kv_heads = k_pool->kv_heads;
    a.group = q_heads / k_pool->kv_heads;
    a.rows_per_kv = a.group * q_rows;
    a.head_dim = k_pool->head_dim;
    a.v_head_dim = v_pool->head_dim;
    a.num_pages = k_pool->num_pages;
    a.page_tokens = k_pool->page_tokens;
    a.k_data = k_pool->data;
    a.k_stride_page = k_pool->stride_page;
    a.k_stride_head = k_pool->stride_head;
    a.k_stride_token = k_pool->stride_token;
    a.v_data = v_pool->data;
    a.v_stride_page = v_pool->stride_page;
    a.v_stride_head = v_pool->stride_head;
    a.v_stride_token = v_pool->stride_token;
    a.k_scale = k_pool->scale;
    a.v_scale = v_pool->scale;
    a.k_bounds = k_pool->bounds;
    a.v_bounds = v_pool->bounds;
    a.block_table = block_table;
    a.max_pages = max_pages;
    a.seq_lens = seq_lens;
    a.scale = scale;
    a.split_size = split_size;
    a.n_split = n_split;
    a.o_part = o_part;
    a.m_part = m_part;
    a.l_part = l_part;
    a.dev_err = dev_err;
    return a;
}

// matrix cores for 16/8-bit pools read with bf16 Q; the vector-ALU kernel for
// fp32 pools and fp32 Q
static bool uses_mfma(const nbx::PartialArgs &a)
{
    return a.q_dtype == NBX_BF16 && (a.kv_dtype == NBX_BF16 || a.kv_dtype == NBX_FP8_E4M3);
}

static hipError_t launch_partial(const nbx::PartialArgs &a, hipStream_t stream)
{
    return uses_mfma(a) ? nbx::launch_partial_mfma(a, stream) : nbx::launch_partial_valu(a, stream);
}

int nbx_paged_decode_partial(const void *q, int32_t q_dtype, int32_t batch, int32_t q_heads,
                             int32_t q_rows, int32_t causal, const nbx_kv_pool *k_pool,
                             const nbx_kv_pool *v_pool, const int32_t *block_table,
                             int32_t max_pages, const int32_t *seq_lens, float scale,
                             int32_t split_size, int32_t n_split, float *o_part, float *m_part,
                             float *l_part, int32_t *dev_err, hipStream_t stream)
{
    int st = validate_partial(q, q_dtype, batch, q_heads, q_rows, causal, k_pool, v_pool,
                              block_table, max_pages, seq_lens, scale, split_size, n_split);
    if (st != NBX_OK)
        return st;
    if (!o_part || !m_part || !l_part)
        return NBX_ERR_NULL_PTR;
    if (!aligned16(o_part) || ((uintptr_t)m_part & 3u) || ((uintptr_t)l_part & 3u))
        return NBX_ERR_BAD_ALIGN;
    if (batch == 0)
        return NBX_OK;

    const nbx::PartialArgs a =
        partial_args(q, q_dtype, batch, q_heads, q_rows, causal, k_pool, v_pool, block_table,
                     max_pages, seq_lens, scale, split_size, n_split, o_part, m_part, l_part,
                     dev_err);
    // matrix cores for 16/8-bit pools read with bf16 Q; the vector-ALU kernel
    // for fp32 pools and fp32 Q
    return to_status(launch_partial(a, stream));
}

int nbx_paged_decode_partial_windows(const void *q, int32_t q_dtype, int32_t batch,
                                     int32_t q_heads, int32_t q_rows,
                                     const int32_t *rows_per_seq, int32_t causal,
                                     const nbx_kv_pool *k_pool, const nbx_kv_pool *v_pool,
                                     const int32_t *block_table, int32_t max_pages,
                                     const int32_t *seq_lens, float scale, int32_t split_size,
                                     int32_t n_split, float *o_part, float *m_part,
                                     float *l_part, int32_t *dev_err, hipStream_t stream)
{
    if (!rows_per_seq)
        return NBX_ERR_NULL_PTR;
    int st = validate_partial(q, q_dtype, batch, q_heads, q_rows, causal, k_pool, v_pool,
                              block_table, max_pages, seq_lens, scale, split_size, n_split);
    if (st != NBX_OK)
        return st;
    if (!o_part || !m_part || !l_part)
        return NBX_ERR_NULL_PTR;
    if (!aligned16(o_part) || ((uintptr_t)m_part & 3u) || ((uintptr_t)l_part & 3u))
        return NBX_ERR_BAD_ALIGN;
    if (batch == 0)
        return NBX_OK;
    nbx::PartialArgs a =
        partial_args(q, q_dtype, batch, q_heads, q_rows, causal, k_pool, v_pool, block_table,
                     max_pages, seq_lens, scale, split_size, n_split, o_part, m_part, l_part,
                     dev_err);
    a.rows_per_seq = rows_per_seq;
    return to_status(launch_partial(a, stream));
}

int nbx_paged_decode_merge(const float *o_part, const float *m_part, const float *l_part,
                           int64_t rows, int32_t n_split, int32_t head_dim, void *out,
                           int32_t out_dtype, hipStream_t stream)
{
    if (!o_part || !m_part || !l_part || !out)
        return NBX_ERR_NULL_PTR;
    if (out_dtype != NBX_F32 && out_dtype != NBX_BF16)
        return NBX_ERR_BAD_DTYPE;
    if (rows < 0 || n_split < 1 || !value_dim_ok(head_dim))
        return NBX_ERR_BAD_SHAPE;
    if (n_split > kMaxMergeSplits)
        return NBX_ERR_UNSUPPORTED;
    if (!aligned16(o_part) || !aligned16(out) || ((uintptr_t)m_part & 3u) ||
        ((uintptr_t)l_part & 3u))
        return NBX_ERR_BAD_ALIGN;
    if (!nbx::grid_fits(rows, 256))              // one 256-thread workgroup per row
        return NBX_ERR_UNSUPPORTED;
    nbx::MergeArgs a{o_part, m_part, l_part, rows, n_split, head_dim, out, out_dtype};
    return to_status(nbx::launch_merge(a, stream));
}

int nbx_paged_decode(const void *q, int32_t q_dtype, int32_t batch, int32_t q_heads,
                     int32_t q_rows, int32_t causal, const nbx_kv_pool *k_pool,
                     const nbx_kv_pool *v_pool, const int32_t *block_table, int32_t max_pages,
                     const int32_t *seq_lens, float scale, int32_t split_size, int32_t n_split,
                     void *workspace, size_t workspace_bytes, void *out, int32_t out_dtype,
                     int32_t *dev_err, hipStream_t stream)
{
    int st = validate_partial(q, q_dtype, batch, q_heads, q_rows, causal, k_pool, v_pool,
                              block_table, max_pages, seq_lens, scale, split_size, n_split);
    if (st != NBX_OK)
        return st;
    if (!out)
        return NBX_ERR_NULL_PTR;
    if (out_dtype != NBX_F32 && out_dtype != NBX_BF16)
        return NBX_ERR_BAD_DTYPE;
    if (n_split > kMaxMergeSplits)
        return NBX_ERR_UNSUPPORTED;
    if (batch == 0)
        return NBX_OK;
    const int64_t rows = (int64_t)batch * q_heads * q_rows;
    const int32_t Dv = v_pool->head_dim;      // partial and output columns
    const size_t need = nbx_paged_decode_workspace_bytes(rows, n_split, Dv);
    if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u))
        return NBX_ERR_WORKSPACE;
    char *ws = (char *)workspace;
    float *o_part = (float *)ws;
    float *m_part = (float *)(ws + round256((size_t)rows * n_split * Dv * sizeof(float)));
    float *l_part = (float *)((char *)m_part + round256((size_t)rows * n_split * sizeof(float)));
    st = nbx_paged_decode_partial(q, q_dtype, batch, q_heads, q_rows, causal, k_pool, v_pool,
                                  block_table, max_pages, seq_lens, scale, split_size, n_split,
                                  o_part, m_part, l_part, dev_err, stream);
    if (st != NBX_OK)
        return st;
    return nbx_paged_decode_merge(o_part, m_part, l_part, rows, n_split, Dv, out, out_dtype,
                                  stream);
}

}  // extern "C"

namespace {

// The step with the partials in `workspace`; `small_ws` is the status of a
// workspace that is too small (the caller's, or the static scratch's limit).
int decode_step(const void *q, int32_t q_dtype, int32_t batch, int32_t q_heads, int32_t q_rows,
                int32_t causal, const void *new_k, const void *new_v, int32_t new_dtype,
                int32_t n_new, const nbx_kv_pool *k_pool, const nbx_kv_pool *v_pool,
                const int32_t *block_table, int32_t max_pages, const int32_t *seq_lens,
                float scale, int32_t split_size, int32_t n_split, void *workspace,
                size_t workspace_bytes, int small_ws, void *out, int32_t out_dtype,
                int32_t *dev_err, hipStream_t stream)
{
    int st = validate_partial(q, q_dtype, batch, q_heads, q_rows, causal, k_pool, v_pool,
                              block_table, max_pages, seq_lens, scale, split_size, n_split);
    if (st != NBX_OK)
        return st;
    if (out && out_dtype != NBX_F32 && out_dtype != NBX_BF16)
        return NBX_ERR_BAD_DTYPE;
    if (n_new < 0)
        return NBX_ERR_BAD_SHAPE;
    if (n_new > 0) {
        if (!new_k || !new_v)
            return NBX_ERR_NULL_PTR;
        if (new_dtype != NBX_F32 && new_dtype != NBX_BF16)
            return NBX_ERR_BAD_DTYPE;
        if (!aligned16(new_k) || !aligned16(new_v))
            return NBX_ERR_BAD_ALIGN;
        if ((int64_t)batch * n_new * k_pool->kv_heads * (k_pool->head_dim / 8) >
            (int64_t)INT32_MAX * 256)      // the wider of the K and V rows
            return NBX_ERR_BAD_SHAPE;
    }
    if (n_split > kMaxMergeSplits)
        return NBX_ERR_UNSUPPORTED;
    if (out && !aligned16(out))
        return NBX_ERR_BAD_ALIGN;
    if (batch == 0)
        return NBX_OK;
    const int64_t rows = (int64_t)batch * q_heads * q_rows;
    const int32_t D = k_pool->head_dim, Dv = v_pool->head_dim;
    const size_t need = nbx_paged_decode_workspace_bytes(rows, n_split, Dv);
    if (!workspace || ((uintptr_t)workspace & 255u))
        return NBX_ERR_WORKSPACE;
    if (workspace_bytes < need)
        return small_ws;
    char *ws = (char *)workspace;
    float *o_part = (float *)ws;
    float *m_part = (float *)(ws + round256((size_t)rows * n_split * Dv * sizeof(float)));
    float *l_part = (float *)((char *)m_part + round256((size_t)rows * n_split * sizeof(float)));
    nbx::PartialArgs a =
        partial_args(q, q_dtype, batch, q_heads, q_rows, causal, k_pool, v_pool, block_table,
                     max_pages, seq_lens, scale, split_size, n_split, o_part, m_part, l_part,
                     dev_err);
    hipError_t e = hipSuccess;
    if (n_new > 0 && uses_mfma(a) && nbx::partial_mfma_is_persistent(a)) {
        // one launch: the wave owning each new position writes it, then reads it
        a.new_k = new_k;
        a.new_v = new_v;
        a.new_dtype = new_dtype;
        a.n_new = n_new;
        e = nbx::launch_partial_mfma(a, stream);
    } else {
        if (n_new > 0) {
            nbx::AppendArgs ap{};
            ap.new_k = new_k;
            ap.new_v = new_v;
            ap.src_dtype = new_dtype;
            ap.dst_dtype = k_pool->dtype;
            ap.n_tok = (int64_t)batch * n_new;
            ap.new_stride_tok = (int64_t)k_pool->kv_heads * D;
            ap.new_stride_head = D;
            ap.kv_heads = k_pool->kv_heads;
            ap.head_dim = D;
            ap.v_head_dim = Dv;
            ap.v_new_stride_tok = (int64_t)k_pool->kv_heads * Dv;
            ap.v_new_stride_head = Dv;
            ap.num_pages = k_pool->num_pages;
            ap.page_tokens = k_pool->page_tokens;
            ap.k_data = k_pool->data;
            ap.k_stride_page = k_pool->stride_page;
            ap.k_stride_head = k_pool->stride_head;
            ap.k_stride_token = k_pool->stride_token;
            ap.v_data = v_pool->data;
            ap.v_stride_page = v_pool->stride_page;
            ap.v_stride_head = v_pool->stride_head;
            ap.v_stride_token = v_pool->stride_token;
            ap.k_scale = k_pool->scale;
            ap.v_scale = v_pool->scale;
            ap.k_bounds = k_pool->bounds;
            ap.v_bounds = v_pool->bounds;
            ap.slot_mapping = nullptr;
            ap.dev_err = dev_err;
            ap.seq_lens = seq_lens;
            ap.block_table = block_table;
            ap.max_pages = max_pages;
            ap.n_new = n_new;
            e = nbx::launch_append(ap, stream);
        }
        if (e == hipSuccess)
            e = launch_partial(a, stream);
    }
    if (e != hipSuccess)
        return to_status(e);
    if (!out)
        return NBX_OK;                         // partials only, left in the workspace
    nbx::MergeArgs m{o_part, m_part, l_part, rows, n_split, Dv, out, out_dtype};
    return to_status(nbx::launch_merge(m, stream));
}

// Partials of nbx_paged_decode_step_noalloc.  Host code uses the address that
// hipGetSymbolAddress gives for the current device (scratch_on_device), never
// the name, which on the host side is no device address.
static __device__ __align__(256) uint8_t scratch[NBX_STEP_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
std::atomic<uintptr_t> scratch_addr[kMaxScratchDevices];

// The current device's copy of `scratch`, looked up once per device (with that
// device current); null if the lookup fails.  Concurrent first calls may both
// look it up: they store the same address.
void *scratch_on_device()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices)
        return nullptr;
    uintptr_t p = scratch_addr[dev].load(std::memory_order_acquire);
    if (p == 0) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
            return nullptr;
        p = (uintptr_t)ptr;
        scratch_addr[dev].store(p, std::memory_order_release);
    }
    return (void *)p;
}

}  // namespace

extern "C" {

int nbx_paged_decode_step(const void *q, int32_t q_dtype, int32_t batch, int32_t q_heads,
                          int32_t q_rows, int32_t causal, const void *new_k, const void *new_v,
                          int32_t new_dtype, int32_t n_new, const nbx_kv_pool *k_pool,
                          const nbx_kv_pool *v_pool, const int32_t *block_table,
                          int32_t max_pages, const int32_t *seq_lens, float scale,
                          int32_t split_size, int32_t n_split, void *workspace,
                          size_t workspace_bytes, void *out, int32_t out_dtype, int32_t *dev_err,
                          hipStream_t stream)
{
    return decode_step(q, q_dtype, batch, q_heads, q_rows, causal, new_k, new_v, new_dtype, n_new,
                       k_pool, v_pool, block_table, max_pages, seq_lens, scale, split_size,
                       n_split, workspace, workspace_bytes, NBX_ERR_WORKSPACE, out, out_dtype,
                       dev_err, stream);
}

int nbx_paged_decode_step_noalloc(const void *q, int32_t q_dtype, int32_t batch, int32_t q_heads,
                                  int32_t q_rows, int32_t causal, const void *new_k,
                                  const void *new_v, int32_t new_dtype, int32_t n_new,
                                  const nbx_kv_pool *k_pool, const nbx_kv_pool *v_pool,
                                  const int32_t *block_table, int32_t max_pages,
                                  const int32_t *seq_lens, float scale, int32_t split_size,
                                  int32_t n_split, void *out, int32_t out_dtype, int32_t *dev_err,
                                  hipStream_t stream)
{
    if (!out)
        return NBX_ERR_NULL_PTR;
    // the size limit is checked on the validated shape, before the device is touched
    int st = validate_partial(q, q_dtype, batch, q_heads, q_rows, causal, k_pool, v_pool,
                              block_table, max_pages, seq_lens, scale, split_size, n_split);
    if (st != NBX_OK)
        return st;
    const int64_t rows = (int64_t)batch * q_heads * q_rows;
    if (rows > 0 &&
        nbx_paged_decode_workspace_bytes(rows, n_split, v_pool->head_dim) > NBX_STEP_SCRATCH_BYTES)
        return NBX_ERR_SCRATCH_LIMIT;
    void *ws = rows > 0 ? scratch_on_device() : nullptr;   // batch 0: nothing to do
    if (rows > 0 && !ws)
        return NBX_ERR_LAUNCH;
    return decode_step(q, q_dtype, batch, q_heads, q_rows, causal, new_k, new_v, new_dtype, n_new,
                       k_pool, v_pool, block_table, max_pages, seq_lens, scale, split_size,
                       n_split, ws, NBX_STEP_SCRATCH_BYTES, NBX_ERR_SCRATCH_LIMIT, out, out_dtype,
                       dev_err, stream);
}

}  // extern "C"
