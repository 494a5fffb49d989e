/*
 * A plain C caller of libnbx_paged (no Python, no torch): device memory from
 * the HIP runtime, then nbx_paged_kv_append and nbx_paged_decode through the
 * C ABI of include/nbx_paged.h, checked against closed forms of softmax
 * attention that this program computes itself (nbxtensor attention_wrappers.py,
 * _math_attention: out = sum_j softmax_j(scale q . k_j) v_j).
 *
 *   A. q = 0: every key gets the same weight, so each output row is the mean
 *      of the V rows its sequence holds.
 *   B. q = 1024 e_0 with K zero except one key per (sequence, KV head) equal to
 *      e_0: that key's score exceeds every other by 1024 / sqrt(128) > 90, so
 *      each output row is that key's V row (the others weigh < e^-90).
 *
 * The key of B is the token appended through the slot mapping, so B also shows
 * that the decode reads the row the append wrote, through a shuffled block
 * table.  V elements are k / 64 with |k| <= 64 and K elements 0 or 1, all exact
 * in bf16, so both closed forms hold to fp32 rounding.  Exit status 0 when
 * every check passes.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "nbx_paged.h"

enum { B = 2, HQ = 4, HKV = 2, G = HQ / HKV, D = 128, T = 16, NPAGES = 12, MAXP = 6 };

static const int LENS[B] = {37, 70};          /* positions held after the append */
static const int PAGES[B][MAXP] = {{7, 2, 9, -1, -1, -1}, {4, 11, 0, 5, 8, -1}};

#define HIP_OK(x)                                                                          \
    do {                                                                                   \
        hipError_t e_ = (x);                                                               \
        if (e_ != hipSuccess) {                                                            \
            fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #x, hipGetErrorString(e_)); \
            exit(2);                                                                       \
        }                                                                                  \
    } while (0)

#define NBX_OK_(x)                                                                         \
    do {                                                                                   \
        int s_ = (x);                                                                      \
        if (s_ != NBX_OK) {                                                                \
            fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #x, nbx_status_str(s_)); \
            exit(2);                                                                       \
        }                                                                                  \
    } while (0)

/* bf16 bits of a float that bf16 holds exactly (the values used here) */
static uint16_t bf16_bits(float x)
{
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    return (uint16_t)(u >> 16);
}

static float bf16_value(uint16_t h)
{
    const uint32_t u = (uint32_t)h << 16;
    float x;
    memcpy(&x, &u, sizeof x);
    return x;
}

static uint32_t lcg_state = 12345u;
static int lcg_k(void)                        /* an integer in [-64, 64] */
{
    lcg_state = lcg_state * 1664525u + 1013904223u;
    return (int)((lcg_state >> 8) % 129u) - 64;
}

static size_t pool_index(int page, int h, int row, int e)
{
    return (((size_t)page * HKV + h) * T + row) * D + e;
}

static double max_err;

static void compare(const char *what, const float *got, const double *want, size_t n)
{
    double worst = 0.0;
    for (size_t i = 0; i < n; ++i) {
        const double d = fabs((double)got[i] - want[i]);
        if (!(d <= worst))                    /* NaN counts as the worst */
            worst = isnan(d) ? INFINITY : d;
    }
    printf("%s: max abs error %.3g\n", what, worst);
    if (!(worst <= max_err))
        max_err = -1.0;                       /* remember a failure */
}

int main(void)
{
    const size_t pool_elems = (size_t)NPAGES * HKV * T * D;
    uint16_t *k_host = calloc(pool_elems, sizeof(uint16_t));
    uint16_t *v_host = calloc(pool_elems, sizeof(uint16_t));
    if (!k_host || !v_host)
        return 2;
    for (size_t i = 0; i < pool_elems; ++i)
        v_host[i] = bf16_bits((float)lcg_k() / 64.0f);

    /* the appended token of each sequence: K = e_0, V = fresh values */
    uint16_t new_k[B][HKV][D], new_v[B][HKV][D];
    int32_t slots[B];
    memset(new_k, 0, sizeof new_k);
    for (int b = 0; b < B; ++b) {
        const int pos = LENS[b] - 1;
        slots[b] = PAGES[b][pos / T] * T + pos % T;
        for (int h = 0; h < HKV; ++h) {
            new_k[b][h][0] = bf16_bits(1.0f);
            for (int e = 0; e < D; ++e)
                new_v[b][h][e] = bf16_bits((float)lcg_k() / 64.0f);
        }
    }

    int32_t table[B][MAXP];
    memcpy(table, PAGES, sizeof table);
    int32_t lens[B];
    memcpy(lens, LENS, sizeof lens);

    void *k_dev, *v_dev, *nk_dev, *nv_dev, *q_dev, *ws_dev, *out_dev;
    int32_t *slot_dev, *table_dev, *lens_dev, *err_dev;
    HIP_OK(hipMalloc(&k_dev, pool_elems * 2));
    HIP_OK(hipMalloc(&v_dev, pool_elems * 2));
    HIP_OK(hipMalloc(&nk_dev, sizeof new_k));
    HIP_OK(hipMalloc(&nv_dev, sizeof new_v));
    HIP_OK(hipMalloc((void **)&slot_dev, sizeof slots));
    HIP_OK(hipMalloc((void **)&table_dev, sizeof table));
    HIP_OK(hipMalloc((void **)&lens_dev, sizeof lens));
    HIP_OK(hipMalloc((void **)&err_dev, sizeof(int32_t)));
    HIP_OK(hipMemcpy(k_dev, k_host, pool_elems * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(v_dev, v_host, pool_elems * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(nk_dev, new_k, sizeof new_k, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(nv_dev, new_v, sizeof new_v, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(slot_dev, slots, sizeof slots, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(table_dev, table, sizeof table, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(lens_dev, lens, sizeof lens, hipMemcpyHostToDevice));
    HIP_OK(hipMemset(err_dev, 0, sizeof(int32_t)));

    nbx_kv_pool kp = {k_dev, NBX_BF16, NPAGES, HKV, T, D, (int64_t)HKV * T * D, (int64_t)T * D,
                      D, 1.0f, NULL};
    nbx_kv_pool vp = kp;
    vp.data = v_dev;

    /* a request the library refuses on the host, before touching the device */
    nbx_kv_pool bad = kp;
    bad.head_dim = 96;
    bad.stride_token = 96;
    const int refused = nbx_paged_kv_append(nk_dev, NULL, NBX_BF16, B, HKV * D, D, &bad, NULL,
                                            slot_dev, err_dev, 0);
    printf("head_dim 96 refused: %s\n", nbx_status_str(refused));
    if (refused != NBX_ERR_BAD_SHAPE)
        return 1;

    NBX_OK_(nbx_paged_kv_append(nk_dev, nv_dev, NBX_BF16, B, HKV * D, D, &kp, &vp, slot_dev,
                                err_dev, 0));
    /* the host copy of the pools after the append */
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < HKV; ++h)
            for (int e = 0; e < D; ++e) {
                const size_t i = pool_index(slots[b] / T, h, slots[b] % T, e);
                k_host[i] = new_k[b][h][e];
                v_host[i] = new_v[b][h][e];
            }

    /* 16-position splits so that every sequence spans several */
    int32_t n_split = 0, split_size = 0;
    NBX_OK_(nbx_paged_decode_plan(LENS[1], 16, 64, &n_split, &split_size));
    const int64_t rows = (int64_t)B * HQ;
    const size_t ws_bytes = nbx_paged_decode_workspace_bytes(rows, n_split, D);
    HIP_OK(hipMalloc(&ws_dev, ws_bytes));
    HIP_OK(hipMalloc(&q_dev, (size_t)rows * D * 2));
    HIP_OK(hipMalloc(&out_dev, (size_t)rows * D * 4));
    printf("plan: %d splits of %d positions; workspace %zu bytes\n", n_split, split_size,
           ws_bytes);

    uint16_t q[B * HQ * D];
    float out[B * HQ * D];
    double want[B * HQ * D];
    const float scale = 1.0f / sqrtf((float)D);
    max_err = 1e-5;

    for (int pass = 0; pass < 2; ++pass) {
        memset(q, 0, sizeof q);
        if (pass == 1)
            for (int r = 0; r < B * HQ; ++r)
                q[r * D] = bf16_bits(1024.0f);
        HIP_OK(hipMemcpy(q_dev, q, sizeof q, hipMemcpyHostToDevice));
        NBX_OK_(nbx_paged_decode(q_dev, NBX_BF16, B, HQ, 1, 0, &kp, &vp, table_dev, MAXP,
                                 lens_dev, scale, split_size, n_split, ws_dev, ws_bytes, out_dev,
                                 NBX_F32, err_dev, 0));
        HIP_OK(hipMemcpy(out, out_dev, sizeof out, hipMemcpyDeviceToHost));
        for (int b = 0; b < B; ++b)
            for (int h = 0; h < HQ; ++h) {
                const int g = h / G;
                double *w = want + ((size_t)b * HQ + h) * D;
                for (int e = 0; e < D; ++e) {
                    if (pass == 0) {            /* A: the mean of the sequence's V rows */
                        double s = 0.0;
                        for (int j = 0; j < LENS[b]; ++j)
                            s += bf16_value(v_host[pool_index(PAGES[b][j / T], g, j % T, e)]);
                        w[e] = s / LENS[b];
                    } else {                    /* B: the V row of the appended key */
                        w[e] = bf16_value(new_v[b][g][e]);
                    }
                }
            }
        compare(pass == 0 ? "A (q = 0: mean of V rows)" : "B (one dominant key: its V row)", out,
                want, (size_t)rows * D);
    }

    int32_t err = -1;
    HIP_OK(hipMemcpy(&err, err_dev, sizeof err, hipMemcpyDeviceToHost));
    printf("device error flags: %d\n", err);
    const int ok = max_err > 0.0 && err == 0;
    printf("%s\n", ok ? "abi_check: pass" : "abi_check: FAIL");

    hipFree(k_dev);
    hipFree(v_dev);
    hipFree(nk_dev);
    hipFree(nv_dev);
    hipFree(slot_dev);
    hipFree(table_dev);
    hipFree(lens_dev);
    hipFree(err_dev);
    hipFree(ws_dev);
    hipFree(q_dev);
    hipFree(out_dev);
    free(k_host);
    free(v_host);
    return ok ? 0 : 1;
}
