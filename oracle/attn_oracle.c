/*
 * attn_oracle.c -- plain fp64 reference for fused scaled-dot-product attention
 * forward (prefill and split-K decode), for the split-K log-sum-exp combine and
 * for the gradients of the forward (dQ, dK, dV).
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the bench's
 * CPU-baseline leg load this library.  It shares no code, header, table or
 * helper with the HIP path, and the HIP path never calls it.
 *
 * Sources (web pages; cited by title and section):
 *   [Neptune notes]  "Neptune论文浅读：把FlashAttention式融合放进编译器"
 *                    (gentlecold.top, notes on the Neptune PLDI 2026 paper)
 *   [CANN FA post]   "CANN FlashAttention 不是算力加速器，它在昇腾NPU上做的是
 *                    '偷懒'的数学" (ai6s.net)
 *   [Mirage lecture] CMU 15-779 Lecture 11, "Advanced ML Compilation: ML
 *                    Superoptimization (Mirage)" (semidirectx.com)
 *   [Twill review]   "Optimal Software Pipelining and Warp Specialization for
 *                    Tensor Core GPUs" (xllm-io.github.io paper review)
 *
 * What is computed is the plain definition, not the fused algorithm.  Both the
 * rolling update and the split-K update reach this result exactly in real
 * arithmetic ([Neptune notes] section 4: the repair h(t,r,r') = t*exp(r - r')
 * distributes over the sum; [CANN FA post] section on the online softmax: the
 * one-pass result equals the two-pass one), so the reference is the definition
 * itself, evaluated in fp64:
 *
 *   [Neptune notes] section 2: the chain QK^T -> score/mask/bias -> softmax -> .V,
 *   and the stable softmax  softmax(x_j) = exp(x_j - m) / sum_k exp(x_k - m),
 *   m = max_k x_k.
 *   [CANN FA post] `softmax_standard`: find the max first, then the exponentials
 *   and their sum, then normalise (two passes over the row).
 *
 * For every output row (b, h, i):
 *   kv head        hk = h / (Hq / Hkv)      (contiguous query-head groups; the
 *                  GQA case of [Mirage lecture] section 7.1 has each group of
 *                  query heads share one K, V pair)
 *   position       p  = i + (Lk - Lq)       (queries aligned to the end of the
 *                  keys: a decode query sees the whole cache)
 *   visible keys   all j in [0, Lk); j <= p when causal; with a window,
 *                  also p - window_left <= j <= p + window_right (a negative
 *                  bound is unbounded).  The pages only name the sliding
 *                  Window operator ([Neptune notes] section 9); the bounds
 *                  follow the usual local-attention reading, relative to the
 *                  query's position p.
 *   score          t_j = scale * sum_d q[d] k_j[d]
 *                  soft cap (when softcap > 0): t_j = softcap * tanh(t_j / softcap)
 *                  (the SoftCap operator of [Neptune notes] section 9; the page
 *                  names it only, this is the plain reading: a smooth bound of
 *                  the scaled score to (-softcap, softcap), before any bias)
 *                  s_j = t_j + bias(b, h, i, j)
 *                  bias: none; dense tensor (element strides, 0 = broadcast);
 *                  or ALiBi  -slope[h] * |p - j|
 *   pass 1         m = max_j s_j
 *   pass 2         l = sum_j exp(s_j - m);  o = sum_j exp(s_j - m) v_j
 *   output         O = o / l,  LSE = m + ln(l)  (natural log)
 *   no visible key O = 0, LSE = -inf.
 *
 * Inputs are fp32 arrays holding the stored element values exactly (bf16
 * values widen exactly to fp32); every product and sum is done in double.
 * Threads split the rows; each thread keeps one row of scores (Lk doubles).
 * The per-row arithmetic does not depend on the thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>

#define ORACLE_BIAS_NONE 0
#define ORACLE_BIAS_DENSE 1
#define ORACLE_BIAS_ALIBI 2

typedef struct {
    int64_t B, Hq, Hkv, Lq, Lk, D;
    const float *q, *k, *v;
    double scale;
    int causal;
    double softcap;            /* > 0: cap the scaled score */
    int window;                /* 1: apply window_left / window_right */
    int64_t window_left, window_right;
    int bias_kind;
    const float *bias;
    int64_t bias_strides[4];
    const float *slopes;
    const int64_t *rows;
    int64_t nrows;
    double *o, *lse;
    int64_t next_row;          /* shared work counter */
    pthread_mutex_t lock;
} oracle_job;

/* The visible keys of the query at position p form one interval [jlo, jhi). */
static void visible_keys(const oracle_job *J, int64_t p, int64_t *jlo_out, int64_t *jhi_out)
{
    int64_t jlo = 0, jhi = J->Lk;
    if (J->causal && p + 1 < jhi) jhi = p + 1;
    if (J->window) {
        if (J->window_left >= 0 && p - J->window_left > jlo) jlo = p - J->window_left;
        if (J->window_right >= 0 && p + J->window_right + 1 < jhi) jhi = p + J->window_right + 1;
    }
    *jlo_out = jlo;
    *jhi_out = jhi;
}

/* Scores s[j - jlo] of row (b, h, i) for the keys jlo <= j < jhi of kbase.
 * With dcap != 0, dcap[j - jlo] receives the derivative of the score with
 * respect to the scaled product (the soft cap's slope; 1 without a cap). */
static void row_scores(const oracle_job *J, int64_t b, int64_t h, int64_t i, int64_t p,
                       int64_t jlo, int64_t jhi, const float *qrow, const float *kbase,
                       double *s, double *dcap)
{
    const int64_t D = J->D;
    for (int64_t j = jlo; j < jhi; ++j) {
        const float *krow = kbase + j * D;
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d) dot += (double)qrow[d] * (double)krow[d];
        double sj = J->scale * dot, slope = 1.0;
        if (J->softcap > 0.0) {
            const double th = tanh(sj / J->softcap);
            sj = J->softcap * th;
            slope = 1.0 - th * th;
        }
        if (J->bias_kind == ORACLE_BIAS_DENSE) {
            const int64_t *st = J->bias_strides;
            sj += (double)J->bias[b * st[0] + h * st[1] + i * st[2] + j * st[3]];
        } else if (J->bias_kind == ORACLE_BIAS_ALIBI) {
            double dist = (double)(p - j);
            if (dist < 0) dist = -dist;
            sj += -(double)J->slopes[h] * dist;
        }
        s[j - jlo] = sj;
        if (dcap) dcap[j - jlo] = slope;
    }
}

/* One output row, two passes over its visible keys. */
static void oracle_row(const oracle_job *J, int64_t flat, double *o, double *lse, double *s)
{
    const int64_t i = flat % J->Lq;
    const int64_t h = (flat / J->Lq) % J->Hq;
    const int64_t b = flat / (J->Lq * J->Hq);
    const int64_t G = J->Hq / J->Hkv;
    const int64_t hk = h / G;
    const int64_t D = J->D;
    const int64_t p = i + (J->Lk - J->Lq);

    const float *qrow = J->q + ((b * J->Hq + h) * J->Lq + i) * D;
    const float *kbase = J->k + (b * J->Hkv + hk) * J->Lk * D;
    const float *vbase = J->v + (b * J->Hkv + hk) * J->Lk * D;

    int64_t jlo, jhi;
    visible_keys(J, p, &jlo, &jhi);

    for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
    if (jhi <= jlo) {
        *lse = -INFINITY;
        return;
    }

    row_scores(J, b, h, i, p, jlo, jhi, qrow, kbase, s, 0);

    /* pass 1: the row maximum */
    double m = -INFINITY;
    for (int64_t j = jlo; j < jhi; ++j)
        if (s[j - jlo] > m) m = s[j - jlo];
    if (m == -INFINITY) {          /* every visible score is -inf (a -inf bias) */
        *lse = -INFINITY;
        return;
    }

    /* pass 2: exponentials, their sum, and the weighted sum of values */
    double l = 0.0;
    for (int64_t j = jlo; j < jhi; ++j) {
        const double e = exp(s[j - jlo] - m);
        l += e;
        const float *vrow = vbase + j * D;
        for (int64_t d = 0; d < D; ++d) o[d] += e * (double)vrow[d];
    }

    /* normalise */
    for (int64_t d = 0; d < D; ++d) o[d] /= l;
    *lse = m + log(l);
}

static void *oracle_worker(void *arg)
{
    oracle_job *J = (oracle_job *)arg;
    double *s = (double *)malloc(sizeof(double) * (size_t)(J->Lk > 0 ? J->Lk : 1));
    if (!s) return (void *)1;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        const int64_t r = J->next_row;
        J->next_row += 1;
        pthread_mutex_unlock(&J->lock);
        if (r >= J->nrows) break;
        const int64_t flat = J->rows ? J->rows[r] : r;
        oracle_row(J, flat, J->o + r * J->D, J->lse + r, s);
    }
    free(s);
    return 0;
}

/*
 * oracle_attention: O and LSE for the requested rows.
 *   q [B,Hq,Lq,D], k and v [B,Hkv,Lk,D]: contiguous fp32.
 *   scale: the softmax scale (pass the fp32 value the device receives).
 *   softcap: > 0 caps the scaled score (0 = off).
 *   window: 1 applies window_left / window_right (negative = unbounded), 0 = no window.
 *   bias_kind 0 none / 1 dense (bias + strides in elements, b,h,i,j) / 2 ALiBi (slopes[Hq]).
 *   rows: flat row ids (b*Hq + h)*Lq + i, or NULL for all B*Hq*Lq rows in order.
 *   o [nrows][D] and lse [nrows] are written in fp64.
 * Returns 0 on success, -1 on an invalid argument, -2 when out of memory.
 */
int oracle_attention(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
                     const float *q, const float *k, const float *v,
                     double scale, int causal, double softcap,
                     int window, int64_t window_left, int64_t window_right,
                     int bias_kind, const float *bias, const int64_t *bias_strides,
                     const float *slopes,
                     const int64_t *rows, int64_t nrows,
                     double *o, double *lse, int nthreads)
{
    if (B < 0 || Hq < 1 || Hkv < 1 || Lq < 0 || Lk < 0 || D < 1) return -1;
    if (Hq % Hkv != 0) return -1;
    if (!o || !lse) return -1;
    if ((Lq > 0 && !q) || (Lk > 0 && (!k || !v))) return -1;
    if (bias_kind == ORACLE_BIAS_DENSE && (!bias || !bias_strides)) return -1;
    if (bias_kind == ORACLE_BIAS_ALIBI && !slopes) return -1;
    if (bias_kind < 0 || bias_kind > 2) return -1;
    if (!(softcap >= 0.0) || window < 0 || window > 1) return -1;

    const int64_t total = B * Hq * Lq;
    if (!rows) nrows = total;
    for (int64_t r = 0; rows && r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= total) return -1;

    oracle_job J;
    J.B = B; J.Hq = Hq; J.Hkv = Hkv; J.Lq = Lq; J.Lk = Lk; J.D = D;
    J.q = q; J.k = k; J.v = v;
    J.scale = scale; J.causal = causal;
    J.softcap = softcap; J.window = window;
    J.window_left = window_left; J.window_right = window_right;
    J.bias_kind = bias_kind; J.bias = bias; J.slopes = slopes;
    for (int t = 0; t < 4; ++t) J.bias_strides[t] = bias_strides ? bias_strides[t] : 0;
    J.rows = rows; J.nrows = nrows;
    J.o = o; J.lse = lse;
    J.next_row = 0;
    pthread_mutex_init(&J.lock, 0);

    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads > nrows) nthreads = nrows > 0 ? (int)nrows : 1;

    int rc = 0;
    if (nthreads == 1) {
        if (oracle_worker(&J)) rc = -2;
    } else {
        pthread_t th[256];
        int started = 0;
        for (int t = 0; t < nthreads; ++t) {
            if (pthread_create(&th[t], 0, oracle_worker, &J) != 0) break;
            ++started;
        }
        if (started == 0 && oracle_worker(&J)) rc = -2;
        for (int t = 0; t < started; ++t) {
            void *ret = 0;
            pthread_join(th[t], &ret);
            if (ret) rc = -2;
        }
    }
    pthread_mutex_destroy(&J.lock);
    return rc;
}

/*
 * oracle_splitk_combine: the global step of the split-K update, in fp64.
 *
 * [Neptune notes] section 6: the key dimension is split into local reductions
 * whose max, sum and output are computed independently; the global step
 * repairs each local sum and output with the global max and adds them up.
 * With the repair term of section 4, h(t, r, r') = t * exp(r - r'):
 *
 *   M   = max_s m_s
 *   w_s = exp(m_s - M)          (0 for a chunk with no key: m_s = -inf)
 *   L   = sum_s w_s l_s
 *   O   = sum_s w_s o_s / L,    LSE = M + ln L
 *   a row with L == 0 (no key anywhere) gives O = 0 and LSE = -inf.
 *
 * o_part [rows][S][D], m_part and l_part [rows][S]: o_s = sum_j exp(s_j - m_s) v_j
 * and l_s = sum_j exp(s_j - m_s) over chunk s; m_s may be any finite reference
 * value (the result does not depend on it, [Mirage lecture] section 5.5).
 */
int oracle_splitk_combine(int64_t rows, int64_t S, int64_t D,
                          const float *o_part, const float *m_part, const float *l_part,
                          double *o, double *lse)
{
    if (rows < 0 || S < 1 || D < 1) return -1;
    if (rows > 0 && (!o_part || !m_part || !l_part || !o || !lse)) return -1;
    for (int64_t r = 0; r < rows; ++r) {
        double M = -INFINITY;
        for (int64_t s = 0; s < S; ++s) {
            const double ms = (double)m_part[r * S + s];
            if (ms > M) M = ms;
        }
        double *orow = o + r * D;
        for (int64_t d = 0; d < D; ++d) orow[d] = 0.0;
        if (M == -INFINITY) {
            lse[r] = -INFINITY;
            continue;
        }
        double L = 0.0;
        for (int64_t s = 0; s < S; ++s) {
            const double ms = (double)m_part[r * S + s];
            if (ms == -INFINITY) continue;
            const double w = exp(ms - M);
            L += w * (double)l_part[r * S + s];
            const float *os = o_part + (r * S + s) * D;
            for (int64_t d = 0; d < D; ++d) orow[d] += w * (double)os[d];
        }
        if (L == 0.0) {
            for (int64_t d = 0; d < D; ++d) orow[d] = 0.0;
            lse[r] = -INFINITY;
            continue;
        }
        for (int64_t d = 0; d < D; ++d) orow[d] /= L;
        lse[r] = M + log(L);
    }
    return 0;
}

/*
 * oracle_attention_bwd: gradients of the attention forward above, in fp64.
 *
 * For each row (b, h, i) with forward weights P_j = exp(s_j - LSE) over its
 * visible keys (the definition of oracle_attention, recomputed here) and an
 * output gradient dO_i, the chain rule through O_i = sum_j P_j v_j, the
 * softmax, the soft cap and the scale gives
 *   dv_j  += P_j dO_i
 *   dP_j   = dO_i . v_j,   Delta_i = sum_j P_j dP_j  (= dO_i . O_i)
 *   dS_j   = P_j (dP_j - Delta_i)                    (softmax Jacobian)
 *   dU_j   = dS_j * (1 - tanh^2(u_j / c))  with a cap c, else dS_j
 *            (u_j = scale * q_i . k_j; d/du [c tanh(u / c)] = 1 - tanh^2(u / c);
 *             the bias is a constant and passes dS_j through unchanged)
 *   dq_i  += scale * dU_j k_j,   dk_j += scale * dU_j q_i.
 * K/V head hk collects the gradients of every query head of its group (the
 * GQA sharing of [Mirage lecture] section 7.1).  No bias gradient is formed.
 * A row with no visible key (or only -inf scores) contributes nothing and
 * gets dq = 0.  The pages give the backward pass only by its shape ([Twill
 * review] section 7.2: one pass with five matrix products and one
 * exponential, benchmarked non-causal at batch 4, 32 heads, head dim 128);
 * the gradient itself is the plain derivative of the forward definition.
 *
 * Work is split by (b, hk): each unit owns dk, dv of its K/V head and dq of
 * the rows of its query heads, so no two threads write the same element.
 */
typedef struct {
    oracle_job f;              /* forward problem (rows, o, lse unused) */
    const float *dout;
    double *dq, *dk, *dv;
    int64_t next_unit;
} oracle_bwd_job;

static void oracle_bwd_unit(oracle_bwd_job *W, int64_t unit, double *s, double *dc, double *orow)
{
    const oracle_job *J = &W->f;
    const int64_t b = unit / J->Hkv, hk = unit % J->Hkv;
    const int64_t G = J->Hq / J->Hkv, D = J->D;
    const float *kbase = J->k + (b * J->Hkv + hk) * J->Lk * D;
    const float *vbase = J->v + (b * J->Hkv + hk) * J->Lk * D;
    double *dkbase = W->dk + (b * J->Hkv + hk) * J->Lk * D;
    double *dvbase = W->dv + (b * J->Hkv + hk) * J->Lk * D;

    for (int64_t h = hk * G; h < (hk + 1) * G; ++h) {
        for (int64_t i = 0; i < J->Lq; ++i) {
            const int64_t p = (J->Lk - J->Lq) + i;   /* as in the forward */
            const int64_t row = (b * J->Hq + h) * J->Lq + i;
            const float *qrow = J->q + row * D;
            const float *dorow = W->dout + row * D;
            double *dqrow = W->dq + row * D;

            int64_t jlo, jhi;
            visible_keys(J, p, &jlo, &jhi);
            if (jhi <= jlo) continue;

            /* forward scores, and the cap's slope */
            row_scores(J, b, h, i, p, jlo, jhi, qrow, kbase, s, dc);
            double m = -INFINITY;
            for (int64_t j = jlo; j < jhi; ++j)
                if (s[j - jlo] > m) m = s[j - jlo];
            if (m == -INFINITY) continue;
            double l = 0.0;
            for (int64_t j = jlo; j < jhi; ++j) l += exp(s[j - jlo] - m);

            /* P, O, Delta */
            for (int64_t d = 0; d < D; ++d) orow[d] = 0.0;
            for (int64_t j = jlo; j < jhi; ++j) {
                s[j - jlo] = exp(s[j - jlo] - m) / l;          /* now P_j */
                const float *vrow = vbase + j * D;
                for (int64_t d = 0; d < D; ++d) orow[d] += s[j - jlo] * (double)vrow[d];
            }
            double delta = 0.0;
            for (int64_t d = 0; d < D; ++d) delta += (double)dorow[d] * orow[d];

            /* gradients */
            for (int64_t j = jlo; j < jhi; ++j) {
                const double P = s[j - jlo];
                const float *vrow = vbase + j * D;
                const float *krow = kbase + j * D;
                double dP = 0.0;
                for (int64_t d = 0; d < D; ++d) dP += (double)dorow[d] * (double)vrow[d];
                const double dU = P * (dP - delta) * dc[j - jlo];
                double *dkrow = dkbase + j * D, *dvrow = dvbase + j * D;
                for (int64_t d = 0; d < D; ++d) {
                    dqrow[d] += J->scale * dU * (double)krow[d];
                    dkrow[d] += J->scale * dU * (double)qrow[d];
                    dvrow[d] += P * (double)dorow[d];
                }
            }
        }
    }
}

static void *oracle_bwd_worker(void *arg)
{
    oracle_bwd_job *W = (oracle_bwd_job *)arg;
    const int64_t n = W->f.Lk > 0 ? W->f.Lk : 1;
    double *s = (double *)malloc(sizeof(double) * (size_t)n);
    double *dc = (double *)malloc(sizeof(double) * (size_t)n);
    double *orow = (double *)malloc(sizeof(double) * (size_t)W->f.D);
    if (!s || !dc || !orow) {
        free(s); free(dc); free(orow);
        return (void *)1;
    }
    const int64_t units = W->f.B * W->f.Hkv;
    for (;;) {
        pthread_mutex_lock(&W->f.lock);
        const int64_t u = W->next_unit;
        W->next_unit += 1;
        pthread_mutex_unlock(&W->f.lock);
        if (u >= units) break;
        oracle_bwd_unit(W, u, s, dc, orow);
    }
    free(s); free(dc); free(orow);
    return 0;
}

/*
 * q [B,Hq,Lq,D], k and v [B,Hkv,Lk,D], dout [B,Hq,Lq,D]: contiguous fp32;
 * the other arguments as for oracle_attention.  dq [B,Hq,Lq,D], dk and dv
 * [B,Hkv,Lk,D] are written in fp64.  Returns 0, -1 (invalid argument) or -2.
 */
int oracle_attention_bwd(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
                         const float *q, const float *k, const float *v, const float *dout,
                         double scale, int causal, double softcap,
                         int window, int64_t window_left, int64_t window_right,
                         int bias_kind, const float *bias, const int64_t *bias_strides,
                         const float *slopes,
                         double *dq, double *dk, double *dv, int nthreads)
{
    if (B < 0 || Hq < 1 || Hkv < 1 || Lq < 0 || Lk < 0 || D < 1) return -1;
    if (Hq % Hkv != 0) return -1;
    if ((B * Hq * Lq > 0 && (!q || !dout || !dq)) || (B * Hkv * Lk > 0 && (!k || !v || !dk || !dv))) return -1;
    if (bias_kind < 0 || bias_kind > 2) return -1;
    if (bias_kind == ORACLE_BIAS_DENSE && (!bias || !bias_strides)) return -1;
    if (bias_kind == ORACLE_BIAS_ALIBI && !slopes) return -1;
    if (!(softcap >= 0.0) || window < 0 || window > 1) return -1;

    for (int64_t t = 0; t < B * Hq * Lq * D; ++t) dq[t] = 0.0;
    for (int64_t t = 0; t < B * Hkv * Lk * D; ++t) { dk[t] = 0.0; dv[t] = 0.0; }

    oracle_bwd_job W;
    oracle_job *J = &W.f;
    J->B = B; J->Hq = Hq; J->Hkv = Hkv; J->Lq = Lq; J->Lk = Lk; J->D = D;
    J->q = q; J->k = k; J->v = v;
    J->scale = scale; J->causal = causal;
    J->softcap = softcap; J->window = window;
    J->window_left = window_left; J->window_right = window_right;
    J->bias_kind = bias_kind; J->bias = bias; J->slopes = slopes;
    for (int t = 0; t < 4; ++t) J->bias_strides[t] = bias_strides ? bias_strides[t] : 0;
    J->rows = 0; J->nrows = 0; J->o = 0; J->lse = 0; J->next_row = 0;
    pthread_mutex_init(&J->lock, 0);
    W.dout = dout; W.dq = dq; W.dk = dk; W.dv = dv; W.next_unit = 0;

    const int64_t units = B * Hkv;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads > units) nthreads = units > 0 ? (int)units : 1;
    int rc = 0;
    if (nthreads == 1) {
        if (oracle_bwd_worker(&W)) rc = -2;
    } else {
        pthread_t th[256];
        int started = 0;
        for (int t = 0; t < nthreads; ++t) {
            if (pthread_create(&th[t], 0, oracle_bwd_worker, &W) != 0) break;
            ++started;
        }
        if (started == 0 && oracle_bwd_worker(&W)) rc = -2;
        for (int t = 0; t < started; ++t) {
            void *ret = 0;
            pthread_join(th[t], &ret);
            if (ret) rc = -2;
        }
    }
    pthread_mutex_destroy(&J->lock);
    return rc;
}

/*
 * oracle_l2norm: the Euclidean norm of each row and the row divided by it,
 * in fp64:
 *   norm_i = sqrt(sum_j x_ij^2),   y_ij = x_ij / norm_i   (y = 0 for a zero row).
 * The [Neptune notes] list the numerically stable L2 norm among the
 * reductions their repair algebra fuses (section 4, and the non-attention
 * operators of section 9); this is the plain definition that any fused or
 * split form must reach.  In fp64 the squares of every finite fp32 value are
 * finite and normal, so the definition needs no scaling here.
 * x: rows x H fp32, row r at x + r * x_stride.  y: rows x H fp64 (contiguous)
 * or NULL; norm: rows fp64 or NULL.  Returns 0 or -1 (invalid argument).
 */
int oracle_l2norm(int64_t rows, int64_t H, const float *x, int64_t x_stride, double *y, double *norm)
{
    if (rows < 0 || H < 0 || x_stride < H) return -1;
    if (rows * H > 0 && !x) return -1;
    for (int64_t r = 0; r < rows; ++r) {
        const float *xr = x + r * x_stride;
        double ss = 0.0;
        for (int64_t j = 0; j < H; ++j) ss += (double)xr[j] * (double)xr[j];
        const double n = sqrt(ss);
        if (norm) norm[r] = n;
        if (y) {
            for (int64_t j = 0; j < H; ++j) y[r * H + j] = n > 0.0 ? (double)xr[j] / n : 0.0;
        }
    }
    return 0;
}
