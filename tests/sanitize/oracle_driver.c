/* oracle_driver.c -- runs every function of oracle/attn_oracle.c on small,
 * ragged problems (causal with Lq > Lk and Lq < Lk, empty rows, no keys,
 * windows, every bias kind, a row subset, one and several threads), built
 * with AddressSanitizer and UndefinedBehaviorSanitizer.  Besides the
 * sanitizers' own checks it asserts what a constant V fixes: every row that
 * sees a key averages to that constant, every other row is 0 with LSE -inf.
 * Exits non-zero on the first failed check. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_attention(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
                     const float *q, const float *k, const float *v, double scale, int causal, double softcap,
                     int window, int64_t window_left, int64_t window_right, int bias_kind, const float *bias,
                     const int64_t *bias_strides, const float *slopes, const int64_t *rows, int64_t nrows, double *o,
                     double *lse, int nthreads);
int oracle_splitk_combine(int64_t rows, int64_t S, int64_t D, const float *o_part, const float *m_part,
                          const float *l_part, double *o, double *lse);
int oracle_attention_bwd(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D, const float *q,
                         const float *k, const float *v, const float *dout, double scale, int causal, double softcap,
                         int window, int64_t window_left, int64_t window_right, int bias_kind, const float *bias,
                         const int64_t *bias_strides, const float *slopes, double *dq, double *dk, double *dv,
                         int nthreads);
int oracle_l2norm(int64_t rows, int64_t H, const float *x, int64_t x_stride, double *y, double *norm);

#define CHECK(c)                                                         \
    do {                                                                 \
        if (!(c)) {                                                      \
            printf("FAILED line %d: %s\n", __LINE__, #c);                \
            exit(1);                                                     \
        }                                                                \
    } while (0)

static uint64_t g_state = 12345;
static float rndf(void) { /* uniform in [-1, 1), splitmix64 */
    uint64_t z = (g_state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    z ^= z >> 31;
    return (float)((double)(z >> 11) / 9007199254740992.0 * 2.0 - 1.0);
}

static float *alloc_fill(int64_t n, int constant) {
    float *p = (float *)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
    for (int64_t i = 0; i < n; ++i) p[i] = constant ? 0.75f : rndf();
    return p;
}

static void run_forward(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D, int causal,
                        int window, int64_t wl, int64_t wr, int bias_kind, double softcap, int threads, int subset) {
    float *q = alloc_fill(B * Hq * Lq * D, 0), *k = alloc_fill(B * Hkv * Lk * D, 0);
    float *v = alloc_fill(B * Hkv * Lk * D, 1);
    float *bias = alloc_fill(Hq * Lq * Lk, 0);
    float *slopes = alloc_fill(Hq, 0);
    const int64_t bst[4] = {0, Lq * Lk, Lk, 1};
    const int64_t total = B * Hq * Lq;
    int64_t *rows = NULL, nrows = total;
    if (subset && total > 2) {
        nrows = total / 2;
        rows = (int64_t *)malloc((size_t)nrows * sizeof(int64_t));
        for (int64_t r = 0; r < nrows; ++r) rows[r] = (r * 7) % total;
    }
    double *o = (double *)malloc((size_t)(nrows > 0 ? nrows : 1) * (size_t)D * sizeof(double));
    double *lse = (double *)malloc((size_t)(nrows > 0 ? nrows : 1) * sizeof(double));
    CHECK(oracle_attention(B, Hq, Hkv, Lq, Lk, D, q, k, v, 0.125, causal, softcap, window, wl, wr, bias_kind, bias,
                           bias_kind == 1 ? bst : NULL, slopes, rows, rows ? nrows : 0, o, lse, threads) == 0);
    for (int64_t r = 0; r < nrows; ++r) {
        if (isinf(lse[r])) {
            CHECK(lse[r] < 0);
            for (int64_t d = 0; d < D; ++d) CHECK(o[r * D + d] == 0.0);
        } else {
            for (int64_t d = 0; d < D; ++d) CHECK(fabs(o[r * D + d] - 0.75) <= 1e-12);
        }
    }
    free(q); free(k); free(v); free(bias); free(slopes); free(rows); free(o); free(lse);
}

int main(void) {
    /* forward: shapes, masks, bias kinds, threads */
    run_forward(1, 1, 1, 17, 17, 8, 0, 0, 0, 0, 0, 0.0, 1, 0);
    run_forward(2, 4, 2, 9, 23, 16, 1, 0, 0, 0, 2, 0.0, 3, 0);      /* causal Lq < Lk, ALiBi, GQA */
    run_forward(1, 3, 1, 30, 11, 8, 1, 0, 0, 0, 1, 0.0, 4, 0);      /* causal Lq > Lk: empty rows, dense bias */
    run_forward(1, 2, 2, 12, 0, 8, 0, 0, 0, 0, 0, 0.0, 2, 0);       /* no keys */
    run_forward(1, 2, 1, 40, 40, 8, 1, 1, 5, 2, 0, 3.0, 4, 1);      /* window, cap, row subset */
    run_forward(2, 2, 2, 20, 25, 8, 0, 1, -1, 0, 2, 0.0, 2, 1);     /* one-sided window */
    run_forward(0, 2, 2, 20, 25, 8, 0, 0, 0, 0, 0, 0.0, 2, 0);      /* empty batch */

    /* split-K combine with empty chunks */
    {
        const int64_t rows = 5, S = 4, D = 8;
        float *op = alloc_fill(rows * S * D, 0), *mp = alloc_fill(rows * S, 0), *lp = alloc_fill(rows * S, 0);
        for (int64_t i = 0; i < rows * S; ++i) lp[i] = fabsf(lp[i]) + 0.5f;
        for (int64_t s = 0; s < S; ++s) { mp[0 * S + s] = -INFINITY; lp[0 * S + s] = 0.f; }   /* dead row */
        mp[1 * S + 2] = -INFINITY; lp[1 * S + 2] = 0.f;                                          /* empty chunk */
        double *o = (double *)malloc(rows * D * sizeof(double)), *lse = (double *)malloc(rows * sizeof(double));
        CHECK(oracle_splitk_combine(rows, S, D, op, mp, lp, o, lse) == 0);
        CHECK(isinf(lse[0]) && lse[0] < 0 && o[0] == 0.0);
        for (int64_t r = 1; r < rows; ++r) CHECK(isfinite(lse[r]));
        free(op); free(mp); free(lp); free(o); free(lse);
    }

    /* backward */
    {
        const int64_t B = 1, Hq = 4, Hkv = 2, Lq = 13, Lk = 19, D = 8;
        float *q = alloc_fill(B * Hq * Lq * D, 0), *k = alloc_fill(B * Hkv * Lk * D, 0);
        float *v = alloc_fill(B * Hkv * Lk * D, 0), *dout = alloc_fill(B * Hq * Lq * D, 0);
        float *slopes = alloc_fill(Hq, 0);
        double *dq = (double *)malloc(B * Hq * Lq * D * sizeof(double));
        double *dk = (double *)malloc(B * Hkv * Lk * D * sizeof(double));
        double *dv = (double *)malloc(B * Hkv * Lk * D * sizeof(double));
        CHECK(oracle_attention_bwd(B, Hq, Hkv, Lq, Lk, D, q, k, v, dout, 0.3, 1, 2.0, 1, 6, -1, 2, NULL, NULL,
                                   slopes, dq, dk, dv, 3) == 0);
        for (int64_t i = 0; i < B * Hkv * Lk * D; ++i) CHECK(isfinite(dk[i]) && isfinite(dv[i]));
        CHECK(oracle_attention_bwd(B, Hq, Hkv, Lq, Lk, D, q, k, v, dout, 0.3, 0, 0.0, 0, 0, 0, 0, NULL, NULL,
                                   NULL, dq, dk, dv, 1) == 0);
        free(q); free(k); free(v); free(dout); free(slopes); free(dq); free(dk); free(dv);
    }

    /* row L2 norm, strided rows, a zero row */
    {
        const int64_t rows = 3, H = 10, stride = 12;
        float *x = alloc_fill(rows * stride, 0);
        for (int64_t j = 0; j < H; ++j) x[stride + j] = 0.f;
        double *y = (double *)malloc(rows * H * sizeof(double)), *n = (double *)malloc(rows * sizeof(double));
        CHECK(oracle_l2norm(rows, H, x, stride, y, n) == 0);
        CHECK(n[1] == 0.0 && y[H] == 0.0);
        free(x); free(y); free(n);
    }

    /* invalid arguments are refused */
    {
        double o[8], lse[1];
        CHECK(oracle_attention(1, 3, 2, 1, 1, 8, NULL, NULL, NULL, 1.0, 0, 0.0, 0, 0, 0, 0, NULL, NULL, NULL, NULL, 0,
                               o, lse, 1) == -1);
        CHECK(oracle_splitk_combine(1, 0, 8, NULL, NULL, NULL, o, lse) == -1);
        CHECK(oracle_l2norm(1, 4, NULL, 2, NULL, NULL) == -1);
    }
    printf("oracle driver: all checks passed\n");
    return 0;
}
