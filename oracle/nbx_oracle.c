/*
 * Float64 CPU oracle for paged split-KV attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the GPU library links, includes or
 * calls this file; it shares no header, table or helper with it.  Only the
 * tests, the smoke check and the benchmark's CPU baseline use it.
 *
 * What it computes, each function citing the passage it follows (pages:
 * "nbxtensor attention_wrappers.py", "nbxtensor paged_decode_attn.py",
 * "TensorFold PR #1219", "maxdiffusion PR #477"):
 *
 *  - oracle_decode_value: the stored element as a real number.  bf16 is the
 *    upper half of an fp32; fp8 is OCP E4M3FN (bias 7, 3 mantissa bits,
 *    subnormals m*2^-9, S.1111.111 is NaN, no infinity, largest 448).  The
 *    pages only say "fp8 cache" (TensorFold PR #1219, the --kv-cache fp8 arm);
 *    E4M3FN with a per-tensor scale is the reading adopted.
 *  - oracle_encode_value: the append's cast to the pool dtype
 *    (nbxtensor paged_decode_attn.py, paged_kv_append_kernel: the new values
 *    are cast to the pool's element type on store): exact for the same dtype,
 *    round-to-nearest-even to bf16, and for fp8 round-to-nearest-even of the
 *    fp32 quotient x/scale, saturating at +-448.
 *  - oracle_append: slot -> (page, position) = (slot div T, slot mod T)
 *    (nbxtensor paged_decode_attn.py, module description of the slot mapping
 *    and paged_kv_append_kernel).
 *  - oracle_attention: the plain definition softmax(scale * q k^T) v over the
 *    positions a query row sees (nbxtensor attention_wrappers.py,
 *    _math_attention: scores, softmax, then P V), gathered through the block
 *    table (nbxtensor paged_decode_attn.py, module description).  GQA head map
 *    h_kv = h div G (paged_decode_attn_split_kernel).  A row that sees no key
 *    is 0 (attention_wrappers.py, the fully-masked-row guard).  The value
 *    head dimension Dv is its own size, independent of the D of q and k
 *    (_math_attention's value head_dim; the split kernel's D_V), so outputs
 *    and partial outputs have Dv columns.
 *  - oracle_partials: per split s over [s*S, min((s+1)*S, n)), the running max
 *    m, the sum of exp(s_j - m) and the unnormalised sum of exp(s_j - m) v_j
 *    (paged_decode_attn_split_kernel, the stored opart / mpart / lpart).  An
 *    empty split is (0, -inf, 0).
 *  - oracle_merge: fixed-order log-sum-exp combine of the partials in
 *    ascending split order (attention_wrappers.py, decode_reduce; its kernel
 *    body is not printed, the standard combine is the reading adopted).
 *  - oracle_split_plan: splits = max(1, min(ceil(longest/256), 64)) and the
 *    split length ceil(ceil(longest/splits)/A)*A (paged_decode_attn.py,
 *    paged_decode_splits and the kernel's seg_len).
 *  - oracle_fixed_shift_constants: the fixed-shift softmax constants of the
 *    maxdiffusion PR #477 page (dynamic bounds): C(N) = 127 - ceil(log2 N) -
 *    ceil(log2 Vmax), W(N) = C(N) + 125, gate = floor(W/2).
 *  - oracle_kv_bounds: the quantities those bounds are built from, per page
 *    and KV head: the largest Euclidean norm of a stored K row and the largest
 *    |element| of a stored V row over the positions the sequences hold
 *    (maxdiffusion PR #477: U_B is a product of the largest query norm and the
 *    largest key norm; the V magnitude bound enters C(N)).
 *
 * All arithmetic on values is in double.  Products of two stored values and a
 * scale are exact in double; sums round at 2^-53.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <omp.h>

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_E4M3 = 2 };

/* planted mistakes, used only by the checker-sanity tests */
enum {
    ORC_MUT_NONE = 0,
    ORC_MUT_DROP_LAST_SPLIT = 1,   /* merge ignores each row's last non-empty split */
    ORC_MUT_HEAD_MOD = 2,          /* KV head taken as h mod H_kv instead of h div G */
    ORC_MUT_CAUSAL_OFF_BY_ONE = 3, /* causal row r sees one key fewer */
    ORC_MUT_SWAP_KV = 4,           /* K and V pools exchanged */
    ORC_MUT_NO_MAX_SHIFT_SIGN = 5, /* exp(m - s) instead of exp(s - m) */
    ORC_MUT_PAGE_OFFSET = 6,       /* position in page taken as j mod T + 1 (wraps) */
    ORC_MUT_V_WIDTH = 7,           /* V rows addressed with the q/k head dim D, not Dv */
    ORC_MUT_NO_PAGE_CHECK = 8,     /* an unmapped (-1) page read as a page of the pool */
};
static int g_mutation = ORC_MUT_NONE;

void oracle_set_mutation(int m) { g_mutation = m; }
int oracle_get_mutation(void) { return g_mutation; }

/* ------------------------------------------------------------------ values */

static size_t elem_size(int dtype)
{
    return dtype == ORC_F32 ? 4 : dtype == ORC_BF16 ? 2 : 1;
}

double oracle_decode_value(int dtype, const void *base, int64_t index)
{
    if (dtype == ORC_F32) {
        float f;
        memcpy(&f, (const char *)base + 4 * index, 4);
        return (double)f;
    }
    if (dtype == ORC_BF16) {
        uint16_t h;
        uint32_t w;
        float f;
        memcpy(&h, (const char *)base + 2 * index, 2);
        w = (uint32_t)h << 16;
        memcpy(&f, &w, 4);
        return (double)f;
    }
    {
        uint8_t c = ((const uint8_t *)base)[index];
        int sign = c >> 7, e = (c >> 3) & 15, m = c & 7;
        double v;
        if (e == 15 && m == 7)
            return NAN;
        if (e == 0)
            v = ldexp((double)m, -9);             /* subnormal: m * 2^-9 */
        else
            v = ldexp(1.0 + m / 8.0, e - 7);      /* normal: 1.m * 2^(e-7) */
        return sign ? -v : v;
    }
}

/* Nearest bf16 to an fp32 value x (held exactly in a double), ties to even. */
static uint16_t encode_bf16(double x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x), q;
    int k, E;
    if (isnan(x))
        return (uint16_t)(sign | 0x7FC0);
    if (isinf(x))
        return (uint16_t)(sign | 0x7F80);
    if (a == 0.0)
        return sign;
    frexp(a, &k);                   /* a = f * 2^k, f in [0.5, 1) */
    E = k - 1;                      /* a = 1.xxx * 2^E */
    if (E < -126) {                 /* subnormal bf16: quantum 2^-133 */
        q = nearbyint(ldexp(a, 133));
        return (uint16_t)(sign | (uint16_t)q);   /* q == 128 is the least normal */
    }
    q = nearbyint(ldexp(a, 7 - E)); /* 8 significant bits: q in [128, 256] */
    if (q == 256.0) {
        q = 128.0;
        E += 1;
    }
    if (E + 127 >= 255)
        return (uint16_t)(sign | 0x7F80);
    return (uint16_t)(sign | ((E + 127) << 7) | ((int)q - 128));
}

/* Nearest E4M3FN code to v, ties to even, saturating at +-448, NaN kept. */
static uint8_t encode_e4m3(double v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0;
    double a = fabs(v), q;
    int k, E;
    if (isnan(v))
        return (uint8_t)(sign | 0x7F);
    if (a >= 448.0)
        return (uint8_t)(sign | 0x7E);
    if (a < ldexp(1.0, -6)) {       /* subnormal range: quantum 2^-9 */
        q = nearbyint(ldexp(a, 9)); /* q in [0, 8]; 8 is the least normal */
        return (uint8_t)(sign | (uint8_t)q);
    }
    frexp(a, &k);
    E = k - 1;                      /* E in [-6, 8] */
    q = nearbyint(ldexp(a, 3 - E)); /* 4 significant bits: q in [8, 16] */
    if (q == 16.0) {
        q = 8.0;
        E += 1;
    }
    {
        int code = ((E + 7) << 3) | ((int)q - 8);
        if (code > 0x7E)
            code = 0x7E;
        return (uint8_t)(sign | code);
    }
}

/* Store x (a value read from a source dtype, so exactly an fp32 value) into a
 * pool element of dtype dst.  For fp8 the code is that of fl32(x / scale). */
void oracle_encode_value(int dst, double x, double scale, void *base, int64_t index)
{
    if (dst == ORC_F32) {
        float f = (float)x;         /* x is an fp32 or bf16 value: exact */
        memcpy((char *)base + 4 * index, &f, 4);
    } else if (dst == ORC_BF16) {
        uint16_t h = encode_bf16(x);
        memcpy((char *)base + 2 * index, &h, 2);
    } else {
        /* x / scale correctly rounded to fp32: a double quotient of two fp32
         * values rounded once more to fp32 is the correctly rounded result */
        double quot = (double)(float)(x / scale);
        ((uint8_t *)base)[index] = encode_e4m3(quot);
    }
}

/* ------------------------------------------------------------------ append */

/* new: [n_tok, H_kv, D] of src dtype (contiguous).  pool: [P, H_kv, T, D] of
 * dst dtype (contiguous), updated in place.  Negative slot: skipped.  Slot at
 * or beyond P*T: skipped and counted.  Returns the number of such slots. */
int oracle_append(const void *new_vals, int src, int64_t n_tok, int h_kv, int d,
                  void *pool, int dst, double scale, int64_t num_pages, int page_tokens,
                  const int32_t *slot_mapping)
{
    int bad = 0;
    for (int64_t t = 0; t < n_tok; ++t) {
        int64_t slot = slot_mapping[t];
        int64_t page, pos;
        if (slot < 0)
            continue;
        if (slot >= num_pages * (int64_t)page_tokens) {
            ++bad;
            continue;
        }
        page = slot / page_tokens;
        pos = slot % page_tokens;
        for (int h = 0; h < h_kv; ++h)
            for (int e = 0; e < d; ++e) {
                int64_t src_i = (t * h_kv + h) * (int64_t)d + e;
                int64_t dst_i = ((page * h_kv + h) * (int64_t)page_tokens + pos) * d + e;
                if (src == dst && dst != ORC_E4M3) {
                    /* a cast to the element's own type leaves its bits alone,
                     * NaN payloads included */
                    size_t sz = elem_size(dst);
                    memcpy((char *)pool + dst_i * sz, (const char *)new_vals + src_i * sz, sz);
                    continue;
                }
                oracle_encode_value(dst, oracle_decode_value(src, new_vals, src_i), scale, pool,
                                    dst_i);
            }
    }
    return bad;
}

/* ------------------------------------------------------------------ plan */

/* splits = max(1, min(ceil(longest/positions), max_splits));
 * split length = ceil(ceil(longest/splits)/align)*align. */
void oracle_split_plan(int64_t longest, int64_t positions, int64_t max_splits, int64_t align,
                       int64_t *splits, int64_t *split_len)
{
    int64_t L = longest < 1 ? 1 : longest;
    int64_t n = (L + positions - 1) / positions;
    int64_t per;
    if (n > max_splits)
        n = max_splits;
    if (n < 1)
        n = 1;
    per = (L + n - 1) / n;
    *splits = n;
    *split_len = (per + align - 1) / align * align;
}

/* ------------------------------------------------------------------ attention */

typedef struct {
    const void *q; int q_dtype;
    int B, Hq, W, D, Dv, causal;
    const void *kpool, *vpool; int kv_dtype; double k_scale, v_scale;
    int64_t P; int Hkv, T;
    const int32_t *block_table; int max_pages;
    const int32_t *seq_lens;
    double scale;
} orc_problem;

/* keys row (b, h, r) sees: [0, n) */
static int64_t visible_keys(const orc_problem *pr, int b, int r)
{
    int64_t L = pr->seq_lens[b];
    int64_t n = L;
    if (pr->causal) {
        n = L - pr->W + r + 1;
        if (g_mutation == ORC_MUT_CAUSAL_OFF_BY_ONE)
            n -= 1;
    }
    return n < 0 ? 0 : n;
}

static int kv_head_of(const orc_problem *pr, int h)
{
    int G = pr->Hq / pr->Hkv;
    if (g_mutation == ORC_MUT_HEAD_MOD)
        return h % pr->Hkv;
    return h / G;
}

/* element offset of (logical position j, KV head g, element e) of sequence b
 * in a pool whose rows hold `width` elements, or -1 if the block table does
 * not map position j to a page of the pool */
static int64_t gather_offset(const orc_problem *pr, int b, int g, int64_t j, int e, int width)
{
    int64_t page = pr->block_table[(int64_t)b * pr->max_pages + j / pr->T];
    int64_t pos = j % pr->T;
    if (g_mutation == ORC_MUT_PAGE_OFFSET)
        pos = (pos + 1) % pr->T;
    if (g_mutation == ORC_MUT_NO_PAGE_CHECK)   /* wraps like a negative array index */
        page = ((page % pr->P) + pr->P) % pr->P;
    if (page < 0 || page >= pr->P)
        return -1;
    return ((page * pr->Hkv + g) * pr->T + pos) * width + e;
}

static const void *k_src(const orc_problem *pr)
{
    return g_mutation == ORC_MUT_SWAP_KV ? pr->vpool : pr->kpool;
}
static const void *v_src(const orc_problem *pr)
{
    return g_mutation == ORC_MUT_SWAP_KV ? pr->kpool : pr->vpool;
}

/* scores s_j = scale * sum_e q_e k_je for j in [j0, j1); returns -1 on a bad page */
static int row_scores(const orc_problem *pr, int b, int h, int r, int64_t j0, int64_t j1,
                      double *s)
{
    int g = kv_head_of(pr, h);
    int64_t qrow = ((int64_t)(b * pr->Hq + h) * pr->W + r) * pr->D;
    const void *kp = k_src(pr);
    double ks = g_mutation == ORC_MUT_SWAP_KV ? pr->v_scale : pr->k_scale;
    for (int64_t j = j0; j < j1; ++j) {
        double acc = 0.0;
        int64_t base = gather_offset(pr, b, g, j, 0, pr->D);
        if (base < 0)
            return -1;
        for (int e = 0; e < pr->D; ++e)
            acc += oracle_decode_value(pr->q_dtype, pr->q, qrow + e) *
                   (oracle_decode_value(pr->kv_dtype, kp, base + e) * ks);
        s[j - j0] = pr->scale * acc;
    }
    return 0;
}

/* weights w_j = exp(s_j - m) (or the planted wrong sign), m = max s_j */
static double shift_max(const double *s, int64_t n)
{
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j) {
        if (isnan(s[j]))
            return NAN;
        if (s[j] > m)
            m = s[j];
    }
    return m;
}

static double weight(double s, double m)
{
    if (g_mutation == ORC_MUT_NO_MAX_SHIFT_SIGN)
        return exp(m - s);
    return exp(s - m);
}

/* sum_j w_j v_j into o[Dv]; returns -1 on a bad page */
static int weighted_values(const orc_problem *pr, int b, int h, int64_t j0, int64_t j1,
                           const double *w, double *o)
{
    int g = kv_head_of(pr, h);
    const void *vp = v_src(pr);
    double vs = g_mutation == ORC_MUT_SWAP_KV ? pr->k_scale : pr->v_scale;
    int width = g_mutation == ORC_MUT_V_WIDTH ? pr->D : pr->Dv;
    for (int e = 0; e < pr->Dv; ++e)
        o[e] = 0.0;
    for (int64_t j = j0; j < j1; ++j) {
        int64_t base = gather_offset(pr, b, g, j, 0, width);
        if (base < 0)
            return -1;
        for (int e = 0; e < pr->Dv; ++e)
            o[e] += w[j - j0] * (oracle_decode_value(pr->kv_dtype, vp, base + e) * vs);
    }
    return 0;
}

static orc_problem make_problem(const void *q, int q_dtype, int B, int Hq, int W, int D,
                                int Dv, int causal, const void *kpool, const void *vpool,
                                int kv_dtype, double k_scale, double v_scale, int64_t P,
                                int Hkv, int T, const int32_t *block_table, int max_pages,
                                const int32_t *seq_lens, double scale)
{
    orc_problem pr;
    pr.q = q; pr.q_dtype = q_dtype; pr.B = B; pr.Hq = Hq; pr.W = W; pr.D = D; pr.Dv = Dv;
    pr.causal = causal; pr.kpool = kpool; pr.vpool = vpool; pr.kv_dtype = kv_dtype;
    pr.k_scale = k_scale; pr.v_scale = v_scale; pr.P = P; pr.Hkv = Hkv; pr.T = T;
    pr.block_table = block_table; pr.max_pages = max_pages; pr.seq_lens = seq_lens;
    pr.scale = scale;
    return pr;
}

/* out: [B*Hq*W, Dv] doubles, rows ordered (b, h, r).  Only rows
 * [row_begin, row_end) are computed (a bounded sample); others untouched.
 * Returns 0, or -1 if some visible position has no page in the pool. */
int oracle_attention_rows(const void *q, int q_dtype, int B, int Hq, int W, int D, int Dv,
                          int causal,
                          const void *kpool, const void *vpool, int kv_dtype,
                          double k_scale, double v_scale, int64_t P, int Hkv, int T,
                          const int32_t *block_table, int max_pages, const int32_t *seq_lens,
                          double scale, int64_t row_begin, int64_t row_end, double *out)
{
    orc_problem pr = make_problem(q, q_dtype, B, Hq, W, D, Dv, causal, kpool, vpool, kv_dtype,
                                  k_scale, v_scale, P, Hkv, T, block_table, max_pages,
                                  seq_lens, scale);
    int status = 0;
    if (Hkv <= 0 || Hq % Hkv != 0)
        return -2;
    if ((g_mutation == ORC_MUT_SWAP_KV && D != Dv) || (g_mutation == ORC_MUT_V_WIDTH && D > Dv))
        return -2;                                /* would read past a pool */
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t row = row_begin; row < row_end; ++row) {
        int r = (int)(row % W);
        int h = (int)((row / W) % Hq);
        int b = (int)(row / ((int64_t)W * Hq));
        int64_t n = visible_keys(&pr, b, r);
        double *o = out + row * Dv;
        double *s, m, den = 0.0;
        if (n == 0) {
            for (int e = 0; e < Dv; ++e)
                o[e] = 0.0;
            continue;
        }
        s = (double *)malloc(sizeof(double) * (size_t)n);
        if (row_scores(&pr, b, h, r, 0, n, s) != 0) {
#pragma omp atomic write
            status = -1;
            free(s);
            continue;
        }
        m = shift_max(s, n);
        for (int64_t j = 0; j < n; ++j) {
            s[j] = weight(s[j], m);
            den += s[j];
        }
        if (weighted_values(&pr, b, h, 0, n, s, o) != 0) {
#pragma omp atomic write
            status = -1;
        }
        for (int e = 0; e < Dv; ++e)
            o[e] /= den;
        free(s);
    }
    return status;
}

int oracle_attention(const void *q, int q_dtype, int B, int Hq, int W, int D, int Dv,
                     int causal,
                     const void *kpool, const void *vpool, int kv_dtype, double k_scale,
                     double v_scale, int64_t P, int Hkv, int T, const int32_t *block_table,
                     int max_pages, const int32_t *seq_lens, double scale, double *out)
{
    return oracle_attention_rows(q, q_dtype, B, Hq, W, D, Dv, causal, kpool, vpool, kv_dtype,
                                 k_scale, v_scale, P, Hkv, T, block_table, max_pages, seq_lens,
                                 scale, 0, (int64_t)B * Hq * W, out);
}

/* o: [rows, n_split, Dv], m, l: [rows, n_split]. */
int oracle_partials(const void *q, int q_dtype, int B, int Hq, int W, int D, int Dv,
                    int causal,
                    const void *kpool, const void *vpool, int kv_dtype, double k_scale,
                    double v_scale, int64_t P, int Hkv, int T, const int32_t *block_table,
                    int max_pages, const int32_t *seq_lens, double scale,
                    int64_t split_len, int n_split, double *o, double *m, double *l)
{
    orc_problem pr = make_problem(q, q_dtype, B, Hq, W, D, Dv, causal, kpool, vpool, kv_dtype,
                                  k_scale, v_scale, P, Hkv, T, block_table, max_pages,
                                  seq_lens, scale);
    int64_t rows = (int64_t)B * Hq * W;
    int status = 0;
    if (Hkv <= 0 || Hq % Hkv != 0)
        return -2;
    if ((g_mutation == ORC_MUT_SWAP_KV && D != Dv) || (g_mutation == ORC_MUT_V_WIDTH && D > Dv))
        return -2;                                /* would read past a pool */
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t row = 0; row < rows; ++row) {
        int r = (int)(row % W);
        int h = (int)((row / W) % Hq);
        int b = (int)(row / ((int64_t)W * Hq));
        int64_t n = visible_keys(&pr, b, r);
        double *s = (double *)malloc(sizeof(double) * (size_t)(split_len > 0 ? split_len : 1));
        for (int sp = 0; sp < n_split; ++sp) {
            int64_t j0 = (int64_t)sp * split_len, j1 = j0 + split_len;
            double *os = o + (row * n_split + sp) * Dv;
            double mm, ll = 0.0;
            if (j1 > n)
                j1 = n;
            if (j0 >= j1) {                       /* empty split */
                for (int e = 0; e < Dv; ++e)
                    os[e] = 0.0;
                m[row * n_split + sp] = -INFINITY;
                l[row * n_split + sp] = 0.0;
                continue;
            }
            if (row_scores(&pr, b, h, r, j0, j1, s) != 0) {
#pragma omp atomic write
                status = -1;
                continue;
            }
            mm = shift_max(s, j1 - j0);
            for (int64_t j = 0; j < j1 - j0; ++j) {
                s[j] = weight(s[j], mm);
                ll += s[j];
            }
            if (weighted_values(&pr, b, h, j0, j1, s, os) != 0) {
#pragma omp atomic write
                status = -1;
            }
            m[row * n_split + sp] = mm;
            l[row * n_split + sp] = ll;
        }
        free(s);
    }
    return status;
}

/* out[row] = sum_s w_s o_s / sum_s w_s l_s, w_s = exp(m_s - M), M the largest
 * m_s of the non-empty splits (m_s = -inf marks an empty split), taken in
 * ascending split order.  A row with no non-empty split is 0. */
void oracle_merge(const double *o, const double *m, const double *l, int64_t rows,
                  int n_split, int D, double *out)
{
    for (int64_t row = 0; row < rows; ++row) {
        double M = -INFINITY, den = 0.0;
        int last = -1, has_nan = 0;
        double *dst = out + row * D;
        for (int s = 0; s < n_split; ++s) {
            double ms = m[row * n_split + s];
            if (isnan(ms))
                has_nan = 1;
            else if (ms != -INFINITY) {
                if (ms > M)
                    M = ms;
                last = s;
            }
        }
        for (int e = 0; e < D; ++e)
            dst[e] = 0.0;
        if (has_nan) {
            for (int e = 0; e < D; ++e)
                dst[e] = NAN;
            continue;
        }
        if (last < 0)
            continue;
        for (int s = 0; s < n_split; ++s) {
            double ms = m[row * n_split + s], w;
            if (ms == -INFINITY)
                continue;
            if (g_mutation == ORC_MUT_DROP_LAST_SPLIT && s == last)
                continue;
            w = exp(ms - M);
            den += w * l[row * n_split + s];
            for (int e = 0; e < D; ++e)
                dst[e] += w * o[(row * n_split + s) * D + e];
        }
        for (int e = 0; e < D; ++e)
            dst[e] = den > 0.0 ? dst[e] / den : 0.0;
    }
}

/* ------------------------------------------------------------------ fixed shift */

/* smallest integer k with 2^k >= x, for x >= 1 (exact: frexp) */
static int64_t ceil_log2(double x)
{
    int e;
    double f = frexp(x, &e);          /* x = f * 2^e, f in [0.5, 1) */
    return f == 0.5 ? e - 1 : e;
}

/* C(N) = 127 - ceil(log2 N) - ceil(log2 v_max), W = C + 125, gate = floor(W / 2).
 * n >= 1 and v_max >= 1, else -1. */
int oracle_fixed_shift_constants(int64_t n, double v_max, int64_t *c, int64_t *w, int64_t *gate)
{
    int64_t cc, ww;
    if (n < 1 || !(v_max >= 1.0) || isinf(v_max))
        return -1;
    cc = 127 - ceil_log2((double)n) - ceil_log2(v_max);
    ww = cc + 125;
    *c = cc;
    *w = ww;
    *gate = ww >= 0 ? ww / 2 : -((-ww + 1) / 2);     /* floor division */
    return 0;
}

/* bounds[page * Hkv + h]: over the rows (page, h, row) holding a position
 * j < L_b of some sequence b (page = block_table[b, j / T], row = j mod T),
 * the largest Euclidean norm of the stored row (is_value == 0) or the largest
 * |stored element| (is_value != 0), in stored units (pool scale not applied).
 * A NaN element makes its bound NaN; rows no sequence holds leave 0.
 * Returns -1 if a held position has no page in the pool. */
int oracle_kv_bounds(const void *pool, int dtype, int64_t P, int Hkv, int T, int D, int is_value,
                     const int32_t *block_table, int max_pages, const int32_t *seq_lens, int B,
                     double *bounds)
{
    for (int64_t i = 0; i < P * Hkv; ++i)
        bounds[i] = 0.0;
    for (int b = 0; b < B; ++b) {
        int64_t L = seq_lens[b];
        for (int64_t j = 0; j < L; ++j) {
            int64_t page = block_table[(int64_t)b * max_pages + j / T];
            if (page < 0 || page >= P)
                return -1;
            for (int h = 0; h < Hkv; ++h) {
                int64_t base = ((page * Hkv + h) * T + j % T) * (int64_t)D;
                double v = 0.0, *dst = &bounds[page * Hkv + h];
                int nan = 0;
                for (int e = 0; e < D; ++e) {
                    double x = oracle_decode_value(dtype, pool, base + e);
                    if (isnan(x))
                        nan = 1;
                    else if (is_value)
                        v = fabs(x) > v ? fabs(x) : v;
                    else
                        v += x * x;
                }
                if (!is_value)
                    v = sqrt(v);
                if (nan || isnan(*dst))
                    *dst = NAN;
                else if (v > *dst)
                    *dst = v;
            }
        }
    }
    return 0;
}

size_t oracle_elem_size(int dtype) { return elem_size(dtype); }

/* threads the OpenMP loops above use */
int oracle_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
    return n;
}
