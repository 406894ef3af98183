/*
 * FP64 CPU oracle for exact scaled-dot-product attention and row softmax.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the tests, the smoke check and the benchmark's CPU
 * baseline do.  It shares no code, header or table with the HIP path.
 *
 * What it computes (plain definitions, no blocking, no fusion, no online
 * recurrence):
 *
 *   Attention, from "CUDA FlashAttention: from online softmax to long-sequence
 *   IO limits" (chengzipai.xyz), section 1 (the definition of O and of the
 *   causal mask) and section 3 (the naive three-stage path):
 *     stage 1  s_ij = (sum_d q_id * k_jd) / sqrt(D)      for the keys j of row i
 *     stage 2  m_i = max_j s_ij, p_ij = exp(s_ij - m_i), l_i = sum_j p_ij,
 *              p_ij = p_ij / l_i                          (safe softmax)
 *     stage 3  o_id = sum_j p_ij * v_jd
 *   The causal mask keeps key j for query i iff j <= i (top-left aligned, Q
 *   and K have the same length N), so every row has at least one key.  The
 *   log-sum-exp of a row is lse_i = m_i + ln(l_i), the natural log of
 *   sum_j exp(s_ij) over the same keys (the page's section 7 only says the
 *   LSE is saved for the backward pass; this is the plain reading).
 *
 *   Attention backward: the pages only say that training keeps (or
 *   recomputes) the log-sum-exp for the backward pass (FA page, section 7)
 *   and that their kernels are forward-only (section 9).  The gradients are
 *   therefore the calculus of the definition above: for the loss L with
 *   dL/dO = dO and P the softmax weights of row i,
 *     dV_j = sum_i P_ij dO_i,       dP_ij = dO_i . v_j,
 *     D_i  = sum_j P_ij dP_ij,      dS_ij = P_ij (dP_ij - D_i),
 *     dQ_i = sum_j dS_ij k_j / sqrt(D),   dK_j = sum_i dS_ij q_i / sqrt(D),
 *   over the visible pairs (j <= i when causal).  Pass 1 walks the rows
 *   (P, dP, D_i, dS and dQ_i; m_i, l_i, D_i kept); pass 2 walks the keys,
 *   recomputing P_ij and dS_ij from the kept row statistics, so every sum
 *   runs in a fixed order whatever the thread count.
 *
 *   Paged decode, from "CUDA KV Cache: paged storage and long-context
 *   decode" (chengzipai.xyz), sections 2, 3 and 5: one query per (request b,
 *   query head h) attends over the request's len_b cached tokens.  Token t of
 *   request b is slot t mod T of physical page block_table[b][t / T] in the
 *   cache [P][2][T][Hkv][D] (kind 0 = K, 1 = V), read for K/V head
 *   floor(h / (Hq / Hkv)).  The three stages are those of attention, with every
 *   cached token visible.  A request whose length is outside [1, max_pages*T]
 *   or which uses a page id outside [0, P) gets NaN outputs (the convention of
 *   the interface this oracle checks).  The cache arrives as raw fp16 or bf16
 *   bits and each element is decoded exactly to double here (IEEE binary16
 *   and bfloat16 formats).
 *
 *   Row softmax, from the softmax kernel study (lpnh.cn/news/2830604),
 *   section 3.1: a double-precision stable softmax per row,
 *     m = max_j x_j, e_j = exp(x_j - m), d = sum_j e_j, y_j = e_j / d.
 *
 * Every sum runs in increasing index order, so results are deterministic for
 * any thread count.  One query row is materialised at a time (a full score
 * matrix at N = 8192 would be 512 MiB per head in FP64); that changes memory
 * use only, not the arithmetic.
 *
 * Layouts: q, k, v, o are [B, H, N, D] row-major, element ((b*H+h)*N+n)*D+d;
 * lse is [B, H, N]; x, y are [M, N] row-major.  All buffers are host memory
 * owned by the caller.  Entry points return 0 on success, -1 on a bad
 * argument (null pointer or non-positive size), -2 if a work buffer could not
 * be allocated.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- attention */

/* Stage 1 for one query row i of one head: s_j for j in J_i, written to s[0..nkeys). */
static int64_t scores_row(const double *q, const double *k, int64_t N, int64_t D,
                          int causal, int64_t i, double *s)
{
    const int64_t nkeys = causal ? i + 1 : N;
    const double root_d = sqrt((double)D);
    const double *qi = q + i * D;
    for (int64_t j = 0; j < nkeys; ++j) {
        const double *kj = k + j * D;
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d)
            dot += qi[d] * kj[d];
        s[j] = dot / root_d;
    }
    return nkeys;
}

/* Stages 1-3 for one query row.  s is a work row of at least N doubles. */
static void attn_row(const double *q, const double *k, const double *v, int64_t N,
                     int64_t D, int causal, int64_t i, double *s, double *o_row,
                     double *lse_out)
{
    const int64_t nkeys = scores_row(q, k, N, D, causal, i, s);

    /* stage 2: safe softmax over the materialised row */
    double m = s[0];
    for (int64_t j = 1; j < nkeys; ++j)
        if (s[j] > m)
            m = s[j];
    double l = 0.0;
    for (int64_t j = 0; j < nkeys; ++j) {
        s[j] = exp(s[j] - m);
        l += s[j];
    }
    for (int64_t j = 0; j < nkeys; ++j)
        s[j] = s[j] / l;

    /* stage 3: P times V */
    for (int64_t d = 0; d < D; ++d)
        o_row[d] = 0.0;
    for (int64_t j = 0; j < nkeys; ++j) {
        const double p = s[j];
        const double *vj = v + j * D;
        for (int64_t d = 0; d < D; ++d)
            o_row[d] += p * vj[d];
    }
    *lse_out = m + log(l);
}

typedef struct {
    const double *q, *k, *v;
    double *o, *lse;
    int64_t H, N, D;
    int causal;
    const int64_t *rows; /* flat row ids ((b*H+h)*N+i), or NULL for all rows */
    int64_t nrows;
    int64_t begin, end;  /* range of the row list this thread owns */
    int status;
} attn_job;

static void *attn_worker(void *arg)
{
    attn_job *jb = (attn_job *)arg;
    double *s = (double *)malloc((size_t)jb->N * sizeof(double));
    if (!s) {
        jb->status = -2;
        return NULL;
    }
    for (int64_t r = jb->begin; r < jb->end; ++r) {
        const int64_t flat = jb->rows ? jb->rows[r] : r;
        const int64_t bh = flat / jb->N, i = flat % jb->N;
        const int64_t head = bh * jb->N * jb->D;
        attn_row(jb->q + head, jb->k + head, jb->v + head, jb->N, jb->D, jb->causal, i, s,
                 jb->o + r * jb->D, jb->lse + r);
    }
    free(s);
    jb->status = 0;
    return NULL;
}

static int run_attn(const double *q, const double *k, const double *v, double *o,
                    double *lse, int64_t B, int64_t H, int64_t N, int64_t D, int causal,
                    const int64_t *rows, int64_t nrows, int nthreads)
{
    if (!q || !k || !v || !o || !lse || B < 1 || H < 1 || N < 1 || D < 1 || nrows < 0)
        return -1;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    if ((int64_t)nthreads > nrows)
        nthreads = nrows > 0 ? (int)nrows : 1;
    attn_job jobs[256];
    pthread_t tid[256];
    int started[256] = {0};
    for (int t = 0; t < nthreads; ++t) {
        attn_job jb = {q, k, v, o, lse, H, N, D, causal, rows, nrows,
                       nrows * t / nthreads, nrows * (t + 1) / nthreads, -2};
        jobs[t] = jb;
    }
    for (int t = 1; t < nthreads; ++t)
        started[t] = pthread_create(&tid[t], NULL, attn_worker, &jobs[t]) == 0;
    attn_worker(&jobs[0]);
    int status = jobs[0].status;
    for (int t = 1; t < nthreads; ++t) {
        if (started[t])
            pthread_join(tid[t], NULL);
        else
            attn_worker(&jobs[t]); /* could not spawn: do the share here */
        if (jobs[t].status != 0)
            status = jobs[t].status;
    }
    return status;
}

/* All B*H*N rows: o is [B,H,N,D], lse is [B,H,N]. */
int oracle_attn_fwd(const double *q, const double *k, const double *v, double *o, double *lse,
                    int64_t B, int64_t H, int64_t N, int64_t D, int causal, int nthreads)
{
    if (B < 1 || H < 1 || N < 1)
        return -1;
    return run_attn(q, k, v, o, lse, B, H, N, D, causal, NULL, B * H * N, nthreads);
}

/* Selected rows only: rows[r] = (b*H+h)*N+i; o_rows is [nrows,D], lse_rows is [nrows]. */
int oracle_attn_rows(const double *q, const double *k, const double *v, int64_t B, int64_t H,
                     int64_t N, int64_t D, int causal, const int64_t *rows, int64_t nrows,
                     double *o_rows, double *lse_rows, int nthreads)
{
    if (!rows)
        return -1;
    for (int64_t r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= B * H * N)
            return -1;
    return run_attn(q, k, v, o_rows, lse_rows, B, H, N, D, causal, rows, nrows, nthreads);
}

/* Stage 1 alone for one row of one head ([N,D] q and k): returns the key count. */
int64_t oracle_attn_scores(const double *q, const double *k, int64_t N, int64_t D, int causal,
                           int64_t i, double *s)
{
    if (!q || !k || !s || N < 1 || D < 1 || i < 0 || i >= N)
        return -1;
    return scores_row(q, k, N, D, causal, i, s);
}

/* ------------------------------------------------------- attention backward */

typedef struct {
    const double *q, *k, *v, *dout;   /* one head: [N, D] each */
    double *dq, *dk, *dv;             /* one head: [N, D] each */
    double *m, *l, *dd;               /* row statistics [N] */
    int64_t N, D;
    int causal;
    int64_t begin, end;               /* rows (pass 1) or keys (pass 2) */
    int pass;
    int status;
} bwd_job;

static void *bwd_worker(void *arg)
{
    bwd_job *jb = (bwd_job *)arg;
    const int64_t N = jb->N, D = jb->D;
    const double root_d = sqrt((double)D);
    if (jb->pass == 1) {
        double *s = (double *)malloc((size_t)N * sizeof(double));
        double *dp = (double *)malloc((size_t)N * sizeof(double));
        if (!s || !dp) {
            free(s);
            free(dp);
            jb->status = -2;
            return NULL;
        }
        for (int64_t i = jb->begin; i < jb->end; ++i) {
            const int64_t nkeys = scores_row(jb->q, jb->k, N, D, jb->causal, i, s);
            double m = s[0];
            for (int64_t j = 1; j < nkeys; ++j)
                if (s[j] > m)
                    m = s[j];
            double l = 0.0;
            for (int64_t j = 0; j < nkeys; ++j) {
                s[j] = exp(s[j] - m);
                l += s[j];
            }
            for (int64_t j = 0; j < nkeys; ++j)
                s[j] = s[j] / l;                       /* P_ij */
            const double *doi = jb->dout + i * D;
            double dd = 0.0;
            for (int64_t j = 0; j < nkeys; ++j) {
                const double *vj = jb->v + j * D;
                double dot = 0.0;
                for (int64_t d = 0; d < D; ++d)
                    dot += doi[d] * vj[d];
                dp[j] = dot;                           /* dP_ij */
                dd += s[j] * dot;
            }
            double *dqi = jb->dq + i * D;
            for (int64_t d = 0; d < D; ++d)
                dqi[d] = 0.0;
            for (int64_t j = 0; j < nkeys; ++j) {
                const double ds = s[j] * (dp[j] - dd);  /* dS_ij */
                const double *kj = jb->k + j * D;
                for (int64_t d = 0; d < D; ++d)
                    dqi[d] += ds * kj[d];
            }
            for (int64_t d = 0; d < D; ++d)
                dqi[d] /= root_d;
            jb->m[i] = m;
            jb->l[i] = l;
            jb->dd[i] = dd;
        }
        free(s);
        free(dp);
    } else {
        for (int64_t j = jb->begin; j < jb->end; ++j) {
            const double *kj = jb->k + j * D, *vj = jb->v + j * D;
            double *dkj = jb->dk + j * D, *dvj = jb->dv + j * D;
            for (int64_t d = 0; d < D; ++d) {
                dkj[d] = 0.0;
                dvj[d] = 0.0;
            }
            for (int64_t i = jb->causal ? j : 0; i < N; ++i) {
                const double *qi = jb->q + i * D, *doi = jb->dout + i * D;
                double sdot = 0.0, pdot = 0.0;
                for (int64_t d = 0; d < D; ++d) {
                    sdot += qi[d] * kj[d];
                    pdot += doi[d] * vj[d];
                }
                const double p = exp(sdot / root_d - jb->m[i]) / jb->l[i];
                const double ds = p * (pdot - jb->dd[i]);
                for (int64_t d = 0; d < D; ++d) {
                    dvj[d] += p * doi[d];
                    dkj[d] += ds * qi[d];
                }
            }
            for (int64_t d = 0; d < D; ++d)
                dkj[d] /= root_d;
        }
    }
    jb->status = 0;
    return NULL;
}

static int run_bwd_pass(bwd_job proto, int pass, int nthreads)
{
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    if ((int64_t)nthreads > proto.N)
        nthreads = (int)proto.N;
    bwd_job jobs[256];
    pthread_t tid[256];
    int started[256] = {0};
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = proto;
        jobs[t].pass = pass;
        jobs[t].begin = proto.N * t / nthreads;
        jobs[t].end = proto.N * (t + 1) / nthreads;
        jobs[t].status = -2;
    }
    for (int t = 1; t < nthreads; ++t)
        started[t] = pthread_create(&tid[t], NULL, bwd_worker, &jobs[t]) == 0;
    bwd_worker(&jobs[0]);
    int status = jobs[0].status;
    for (int t = 1; t < nthreads; ++t) {
        if (started[t])
            pthread_join(tid[t], NULL);
        else
            bwd_worker(&jobs[t]);
        if (jobs[t].status != 0)
            status = jobs[t].status;
    }
    return status;
}

/* Gradients of the selected heads heads[h] = b*H + h' of [B,H,N,D] inputs;
 * dq, dk, dv are [nheads, N, D]. */
int oracle_attn_bwd(const double *q, const double *k, const double *v, const double *dout,
                    int64_t B, int64_t H, int64_t N, int64_t D, int causal, const int64_t *heads,
                    int64_t nheads, double *dq, double *dk, double *dv, int nthreads)
{
    if (!q || !k || !v || !dout || !heads || !dq || !dk || !dv || B < 1 || H < 1 || N < 1 ||
        D < 1 || nheads < 0)
        return -1;
    for (int64_t h = 0; h < nheads; ++h)
        if (heads[h] < 0 || heads[h] >= B * H)
            return -1;
    double *m = (double *)malloc((size_t)N * sizeof(double));
    double *l = (double *)malloc((size_t)N * sizeof(double));
    double *dd = (double *)malloc((size_t)N * sizeof(double));
    int status = 0;
    if (!m || !l || !dd)
        status = -2;
    for (int64_t h = 0; status == 0 && h < nheads; ++h) {
        const int64_t off = heads[h] * N * D, out = h * N * D;
        bwd_job proto = {q + off, k + off, v + off, dout + off, dq + out, dk + out, dv + out,
                         m, l, dd, N, D, causal, 0, 0, 0, 0};
        status = run_bwd_pass(proto, 1, nthreads);
        if (status == 0)
            status = run_bwd_pass(proto, 2, nthreads);
    }
    free(m);
    free(l);
    free(dd);
    return status;
}

/* ------------------------------------------------------------- paged decode */

/* Exact value of a binary16 bit pattern. */
static double half_bits_to_double(uint16_t h)
{
    const int sign = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24); /* subnormal or zero */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);
    return sign ? -v : v;
}

/* Exact value of a bfloat16 bit pattern (the high half of a binary32). */
static double bf16_bits_to_double(uint16_t h)
{
    const uint32_t w = (uint32_t)h << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

typedef struct {
    const double *q;               /* [B, Hq, D] */
    const uint16_t *cache;         /* [P, 2, T, Hkv, D] raw bits */
    int is_bf16;
    const int32_t *block_table;    /* [B, max_pages] */
    const int32_t *lengths;        /* [B] */
    double *o, *lse;               /* [nrows, D], [nrows] */
    int64_t Hq, Hkv, D, T, P, max_pages;
    const int64_t *rows;           /* flat ids b*Hq + h */
    int64_t begin, end;
    int status;
} dec_job;

static double cache_at(const dec_job *jb, int64_t page, int kind, int64_t slot, int64_t kvh,
                       int64_t d)
{
    const int64_t idx = (((page * 2 + kind) * jb->T + slot) * jb->Hkv + kvh) * jb->D + d;
    return jb->is_bf16 ? bf16_bits_to_double(jb->cache[idx]) : half_bits_to_double(jb->cache[idx]);
}

static void *dec_worker(void *arg)
{
    dec_job *jb = (dec_job *)arg;
    const int64_t cap = jb->max_pages * jb->T;
    double *s = (double *)malloc((size_t)cap * sizeof(double));
    if (!s) {
        jb->status = -2;
        return NULL;
    }
    const double root_d = sqrt((double)jb->D);
    for (int64_t r = jb->begin; r < jb->end; ++r) {
        const int64_t flat = jb->rows[r];
        const int64_t b = flat / jb->Hq, h = flat % jb->Hq;
        const int64_t kvh = h / (jb->Hq / jb->Hkv);
        const int64_t len = jb->lengths[b];
        double *o_row = jb->o + r * jb->D;
        int valid = len >= 1 && len <= cap;
        for (int64_t t = 0; valid && t < len; t += jb->T) {
            const int64_t page = jb->block_table[b * jb->max_pages + t / jb->T];
            if (page < 0 || page >= jb->P)
                valid = 0;
        }
        if (!valid) {
            for (int64_t d = 0; d < jb->D; ++d)
                o_row[d] = NAN;
            jb->lse[r] = NAN;
            continue;
        }
        /* stage 1: the score of every cached token */
        const double *qr = jb->q + flat * jb->D;
        for (int64_t t = 0; t < len; ++t) {
            const int64_t page = jb->block_table[b * jb->max_pages + t / jb->T];
            double dot = 0.0;
            for (int64_t d = 0; d < jb->D; ++d)
                dot += qr[d] * cache_at(jb, page, 0, t % jb->T, kvh, d);
            s[t] = dot / root_d;
        }
        /* stage 2: safe softmax */
        double m = s[0];
        for (int64_t t = 1; t < len; ++t)
            if (s[t] > m)
                m = s[t];
        double l = 0.0;
        for (int64_t t = 0; t < len; ++t) {
            s[t] = exp(s[t] - m);
            l += s[t];
        }
        for (int64_t t = 0; t < len; ++t)
            s[t] = s[t] / l;
        /* stage 3: P times V */
        for (int64_t d = 0; d < jb->D; ++d)
            o_row[d] = 0.0;
        for (int64_t t = 0; t < len; ++t) {
            const int64_t page = jb->block_table[b * jb->max_pages + t / jb->T];
            for (int64_t d = 0; d < jb->D; ++d)
                o_row[d] += s[t] * cache_at(jb, page, 1, t % jb->T, kvh, d);
        }
        jb->lse[r] = m + log(l);
    }
    free(s);
    jb->status = 0;
    return NULL;
}

/* Selected (request, query head) pairs rows[r] = b*Hq + h; o_rows [nrows, D], lse_rows [nrows]. */
int oracle_paged_decode(const double *q, const uint16_t *cache, int is_bf16,
                        const int32_t *block_table, const int32_t *lengths, int64_t B, int64_t Hq,
                        int64_t Hkv, int64_t D, int64_t T, int64_t P, int64_t max_pages,
                        const int64_t *rows, int64_t nrows, double *o_rows, double *lse_rows,
                        int nthreads)
{
    if (!q || !cache || !block_table || !lengths || !rows || !o_rows || !lse_rows || B < 1 ||
        Hq < 1 || Hkv < 1 || Hq % Hkv || D < 1 || T < 1 || P < 1 || max_pages < 1 || nrows < 0)
        return -1;
    for (int64_t r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= B * Hq)
            return -1;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    if ((int64_t)nthreads > nrows)
        nthreads = nrows > 0 ? (int)nrows : 1;
    dec_job jobs[256];
    pthread_t tid[256];
    int started[256] = {0};
    for (int t = 0; t < nthreads; ++t) {
        dec_job jb = {q, cache, is_bf16, block_table, lengths, o_rows, lse_rows, Hq, Hkv, D, T, P,
                      max_pages, rows, nrows * t / nthreads, nrows * (t + 1) / nthreads, -2};
        jobs[t] = jb;
    }
    for (int t = 1; t < nthreads; ++t)
        started[t] = pthread_create(&tid[t], NULL, dec_worker, &jobs[t]) == 0;
    dec_worker(&jobs[0]);
    int status = jobs[0].status;
    for (int t = 1; t < nthreads; ++t) {
        if (started[t])
            pthread_join(tid[t], NULL);
        else
            dec_worker(&jobs[t]);
        if (jobs[t].status != 0)
            status = jobs[t].status;
    }
    return status;
}

/* Exact decoding of n raw 16-bit values (is_bf16: bfloat16, else binary16). */
int oracle_bits_to_double(const uint16_t *bits, int is_bf16, int64_t n, double *out)
{
    if (!bits || !out || n < 0)
        return -1;
    for (int64_t i = 0; i < n; ++i)
        out[i] = is_bf16 ? bf16_bits_to_double(bits[i]) : half_bits_to_double(bits[i]);
    return 0;
}

/* -------------------------------------------------------------- row softmax */

static void softmax_row(const double *x, double *y, int64_t N)
{
    double m = x[0];
    for (int64_t j = 1; j < N; ++j)
        if (x[j] > m)
            m = x[j];
    double d = 0.0;
    for (int64_t j = 0; j < N; ++j) {
        y[j] = exp(x[j] - m);
        d += y[j];
    }
    for (int64_t j = 0; j < N; ++j)
        y[j] = y[j] / d;
}

typedef struct {
    const double *x;
    double *y;
    int64_t N;
    const int64_t *rows;
    int64_t begin, end;
} sm_job;

static void *sm_worker(void *arg)
{
    sm_job *jb = (sm_job *)arg;
    for (int64_t r = jb->begin; r < jb->end; ++r) {
        const int64_t src = jb->rows ? jb->rows[r] : r;
        softmax_row(jb->x + src * jb->N, jb->y + r * jb->N, jb->N);
    }
    return NULL;
}

static int run_softmax(const double *x, double *y, int64_t N, const int64_t *rows,
                       int64_t nrows, int nthreads)
{
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    if ((int64_t)nthreads > nrows)
        nthreads = nrows > 0 ? (int)nrows : 1;
    sm_job jobs[256];
    pthread_t tid[256];
    int started[256] = {0};
    for (int t = 0; t < nthreads; ++t) {
        sm_job jb = {x, y, N, rows, nrows * t / nthreads, nrows * (t + 1) / nthreads};
        jobs[t] = jb;
    }
    for (int t = 1; t < nthreads; ++t)
        started[t] = pthread_create(&tid[t], NULL, sm_worker, &jobs[t]) == 0;
    sm_worker(&jobs[0]);
    for (int t = 1; t < nthreads; ++t) {
        if (started[t])
            pthread_join(tid[t], NULL);
        else
            sm_worker(&jobs[t]);
    }
    return 0;
}

/* All M rows of x [M,N] into y [M,N]. */
int oracle_row_softmax(const double *x, double *y, int64_t M, int64_t N, int nthreads)
{
    if (!x || !y || M < 1 || N < 1)
        return -1;
    return run_softmax(x, y, N, NULL, M, nthreads);
}

/* Selected rows: y_rows is [nrows,N], row r is softmax of x[rows[r], :]. */
int oracle_row_softmax_rows(const double *x, int64_t M, int64_t N, const int64_t *rows,
                            int64_t nrows, double *y_rows, int nthreads)
{
    if (!x || !y_rows || !rows || M < 1 || N < 1 || nrows < 0)
        return -1;
    for (int64_t r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= M)
            return -1;
    return run_softmax(x, y_rows, N, rows, nrows, nthreads);
}
