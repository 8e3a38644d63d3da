/*
 * cp_oracle.c -- plain C + OpenMP float64 definition of attention with
 * per-row log-sum-exp, for selected query rows of large inputs.
 *
 * TEST INFRASTRUCTURE ONLY: called by the tests, by the smoke check and by
 * the cpu_baseline leg of the benchmark.  It shares nothing with the HIP
 * library (no headers, helpers or constants).
 *
 * Definition followed: the handbook page "上下文并行：Ring Attention 与
 * Ulysses" (Context parallelism: Ring Attention and Ulysses), section
 * "哪些运算可以直接切", function attention(q, k, v, causal, q_offset,
 * k_offset):
 *   s_j   = (q_i . k_j) / sqrt(D)          for every visible key j,
 *   key j visible  <=>  not causal, or k_offset + j <= q_offset + i,
 *   lse_i = log sum_j exp(s_j)             (natural log, max-shifted),
 *   out_i = sum_j exp(s_j - lse_i) v_j.
 * Readings: a row with no visible key gets lse = -inf and out = 0; query
 * head h reads KV head h / (Hq / Hkv).
 *
 * Layouts: q [Sq][Hq][D], k and v [Sk][Hkv][D], elements float32
 * (dtype 0) or bfloat16 bit patterns (dtype 1, widened exactly).  The
 * selected rows are rows[0..n_rows) (NULL = all Sq rows in order); out is
 * [n_rows][Hq][D] and lse is [Hq][n_rows], both float64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double widen(const void *base, int dtype, int64_t idx)
{
    if (dtype == 0)
        return (double)((const float *)base)[idx];
    uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* Returns 0 on success, 1 on bad arguments, 2 on allocation failure. */
int cp_oracle_attention(const void *q, const void *k, const void *v, int dtype,
                        int64_t Sq, int64_t Sk, int Hq, int Hkv, int D,
                        int64_t q_offset, int64_t k_offset, int causal,
                        const int64_t *rows, int64_t n_rows,
                        double *out, double *lse, int n_threads)
{
    if (!q || !k || !v || !out || !lse || Sq < 0 || Sk < 0 || Hq <= 0 || Hkv <= 0 ||
        D <= 0 || Hq % Hkv != 0 || (dtype != 0 && dtype != 1))
        return 1;
    if (!rows)
        n_rows = Sq;
    for (int64_t r = 0; rows && r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= Sq)
            return 1;
    const int group = Hq / Hkv;
    const double inv_sqrt_d = 1.0 / sqrt((double)D);
    int failed = 0;
    if (n_threads <= 0)
        n_threads = 1;

#pragma omp parallel num_threads(n_threads)
    {
        double *s = (double *)malloc((size_t)(Sk > 0 ? Sk : 1) * sizeof(double));
        double *qi = (double *)malloc((size_t)D * sizeof(double));
        double *acc = (double *)malloc((size_t)D * sizeof(double));
        if (!s || !qi || !acc) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < (int64_t)Hq * n_rows; ++t) {
            if (failed)
                continue;
            const int h = (int)(t / n_rows);
            const int64_t r = t % n_rows;
            const int64_t i = rows ? rows[r] : r;
            const int g = h / group;
            const int64_t pos_q = q_offset + i;
            for (int d = 0; d < D; ++d)
                qi[d] = widen(q, dtype, (i * Hq + h) * (int64_t)D + d);

            /* scores of the visible keys and their maximum */
            double m = -INFINITY;
            int64_t n_vis = 0;
            for (int64_t j = 0; j < Sk; ++j) {
                if (causal && k_offset + j > pos_q) {
                    s[j] = -INFINITY;
                    continue;
                }
                double dot = 0.0;
                for (int d = 0; d < D; ++d)
                    dot += qi[d] * widen(k, dtype, (j * Hkv + g) * (int64_t)D + d);
                s[j] = dot * inv_sqrt_d;
                if (s[j] > m)
                    m = s[j];
                ++n_vis;
            }
            double *o = out + (r * Hq + h) * (int64_t)D;
            if (n_vis == 0) {
                lse[(int64_t)h * n_rows + r] = -INFINITY;
                for (int d = 0; d < D; ++d)
                    o[d] = 0.0;
                continue;
            }
            double sum = 0.0;
            for (int64_t j = 0; j < Sk; ++j)
                if (s[j] != -INFINITY)
                    sum += exp(s[j] - m);
            const double l = m + log(sum);
            lse[(int64_t)h * n_rows + r] = l;

            for (int d = 0; d < D; ++d)
                acc[d] = 0.0;
            for (int64_t j = 0; j < Sk; ++j) {
                if (s[j] == -INFINITY)
                    continue;
                const double w = exp(s[j] - l);
                for (int d = 0; d < D; ++d)
                    acc[d] += w * widen(v, dtype, (j * Hkv + g) * (int64_t)D + d);
            }
            for (int d = 0; d < D; ++d)
                o[d] = acc[d];
        }
        free(s);
        free(qi);
        free(acc);
    }
    return failed ? 2 : 0;
}

/*
 * Gradients of L = sum(dout * out) for selected rows (the plain chain rule
 * through the definition above):
 *   P_ij  = exp(s_ij - lse_i),  Dv_i = dout_i . out_i,
 *   ds_ij = P_ij (dout_i . v_j - Dv_i),
 *   dq_i  = sum_j ds_ij k_j / sqrt(D),
 *   dk_j  = sum over heads of the group, sum_i ds_ij q_i / sqrt(D),
 *   dv_j  = sum over heads of the group, sum_i P_ij dout_i.
 * dout has q's layout and dtype.  dq is [n_q][Hq][D] for query rows
 * q_rows[0..n_q); dk and dv are [n_k][Hkv][D] for key rows k_rows[0..n_k)
 * (either list may be empty).  lse_i and Dv_i of every query row that a
 * requested gradient needs are recomputed here from the definition.
 * Returns 0, 1 on bad arguments, 2 on allocation failure.
 */
static void row_stats(const void *q, const void *k, const void *v, const void *dout, int dtype,
                      int64_t Sk, int Hq, int Hkv, int D, int64_t q_offset, int64_t k_offset,
                      int causal, int h, int64_t i, double *s, double *qi, double *acc,
                      double *lse_out, double *dv_out)
{
    const int g = h / (Hq / Hkv);
    const double inv_sqrt_d = 1.0 / sqrt((double)D);
    for (int d = 0; d < D; ++d)
        qi[d] = widen(q, dtype, (i * Hq + h) * (int64_t)D + d);
    double m = -INFINITY;
    for (int64_t j = 0; j < Sk; ++j) {
        if (causal && k_offset + j > q_offset + i) {
            s[j] = -INFINITY;
            continue;
        }
        double dot = 0.0;
        for (int d = 0; d < D; ++d)
            dot += qi[d] * widen(k, dtype, (j * Hkv + g) * (int64_t)D + d);
        s[j] = dot * inv_sqrt_d;
        if (s[j] > m)
            m = s[j];
    }
    if (m == -INFINITY) {
        *lse_out = -INFINITY;
        *dv_out = 0.0;
        return;
    }
    double sum = 0.0;
    for (int64_t j = 0; j < Sk; ++j)
        if (s[j] != -INFINITY)
            sum += exp(s[j] - m);
    const double l = m + log(sum);
    for (int d = 0; d < D; ++d)
        acc[d] = 0.0;
    for (int64_t j = 0; j < Sk; ++j) {
        if (s[j] == -INFINITY)
            continue;
        const double w = exp(s[j] - l);
        for (int d = 0; d < D; ++d)
            acc[d] += w * widen(v, dtype, (j * Hkv + g) * (int64_t)D + d);
    }
    double dvi = 0.0;
    for (int d = 0; d < D; ++d)
        dvi += widen(dout, dtype, (i * Hq + h) * (int64_t)D + d) * acc[d];
    *lse_out = l;
    *dv_out = dvi;
}

int cp_oracle_attention_bwd(const void *q, const void *k, const void *v, const void *dout,
                            int dtype, int64_t Sq, int64_t Sk, int Hq, int Hkv, int D,
                            int64_t q_offset, int64_t k_offset, int causal,
                            const int64_t *q_rows, int64_t n_q, const int64_t *k_rows,
                            int64_t n_k, double *dq, double *dk, double *dv, int n_threads)
{
    if (!q || !k || !v || !dout || Sq < 0 || Sk < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 ||
        Hq % Hkv != 0 || (dtype != 0 && dtype != 1) || n_q < 0 || n_k < 0 ||
        (n_q > 0 && (!q_rows || !dq)) || (n_k > 0 && (!k_rows || !dk || !dv)))
        return 1;
    for (int64_t r = 0; r < n_q; ++r)
        if (q_rows[r] < 0 || q_rows[r] >= Sq)
            return 1;
    for (int64_t r = 0; r < n_k; ++r)
        if (k_rows[r] < 0 || k_rows[r] >= Sk)
            return 1;
    const int group = Hq / Hkv;
    const double inv_sqrt_d = 1.0 / sqrt((double)D);
    if (n_threads <= 0)
        n_threads = 1;
    /* per (head, query row) statistics: all rows when key rows are asked */
    const int64_t n_stat = n_k > 0 ? Sq : n_q;
    double *lse = (double *)malloc((size_t)(Hq * (n_stat > 0 ? n_stat : 1)) * sizeof(double));
    double *dvec = (double *)malloc((size_t)(Hq * (n_stat > 0 ? n_stat : 1)) * sizeof(double));
    if (!lse || !dvec) {
        free(lse);
        free(dvec);
        return 2;
    }
    int failed = 0;
#pragma omp parallel num_threads(n_threads)
    {
        double *s = (double *)malloc((size_t)(Sk > 0 ? Sk : 1) * sizeof(double));
        double *qi = (double *)malloc((size_t)D * sizeof(double));
        double *acc = (double *)malloc((size_t)D * sizeof(double));
        double *acc2 = (double *)malloc((size_t)D * sizeof(double));
        if (!s || !qi || !acc || !acc2) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < (int64_t)Hq * n_stat; ++t) {
            if (failed)
                continue;
            const int h = (int)(t / n_stat);
            const int64_t r = t % n_stat;
            const int64_t i = n_k > 0 ? r : q_rows[r];
            row_stats(q, k, v, dout, dtype, Sk, Hq, Hkv, D, q_offset, k_offset, causal, h, i, s,
                      qi, acc, &lse[(int64_t)h * n_stat + r], &dvec[(int64_t)h * n_stat + r]);
        }
        /* dq rows */
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < (int64_t)Hq * n_q; ++t) {
            if (failed)
                continue;
            const int h = (int)(t / n_q);
            const int64_t r = t % n_q;
            const int64_t i = q_rows[r];
            const int g = h / group;
            const int64_t sr = n_k > 0 ? i : r;
            const double l = lse[(int64_t)h * n_stat + sr], dvi = dvec[(int64_t)h * n_stat + sr];
            double *o = dq + (r * Hq + h) * (int64_t)D;
            for (int d = 0; d < D; ++d) {
                o[d] = 0.0;
                qi[d] = widen(q, dtype, (i * Hq + h) * (int64_t)D + d);
                acc[d] = widen(dout, dtype, (i * Hq + h) * (int64_t)D + d);
            }
            if (l == -INFINITY)
                continue;
            for (int64_t j = 0; j < Sk; ++j) {
                if (causal && k_offset + j > q_offset + i)
                    continue;
                double dot = 0.0, dp = 0.0;
                for (int d = 0; d < D; ++d) {
                    dot += qi[d] * widen(k, dtype, (j * Hkv + g) * (int64_t)D + d);
                    dp += acc[d] * widen(v, dtype, (j * Hkv + g) * (int64_t)D + d);
                }
                const double p = exp(dot * inv_sqrt_d - l);
                const double ds = p * (dp - dvi);
                for (int d = 0; d < D; ++d)
                    o[d] += ds * widen(k, dtype, (j * Hkv + g) * (int64_t)D + d) * inv_sqrt_d;
            }
        }
        /* dk, dv rows */
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < (int64_t)Hkv * n_k; ++t) {
            if (failed)
                continue;
            const int g = (int)(t / n_k);
            const int64_t r = t % n_k;
            const int64_t j = k_rows[r];
            double *ok = dk + (r * Hkv + g) * (int64_t)D;
            double *ov = dv + (r * Hkv + g) * (int64_t)D;
            for (int d = 0; d < D; ++d) {
                ok[d] = 0.0;
                ov[d] = 0.0;
                qi[d] = widen(k, dtype, (j * Hkv + g) * (int64_t)D + d);     /* k_j */
                acc2[d] = widen(v, dtype, (j * Hkv + g) * (int64_t)D + d);   /* v_j */
            }
            for (int h = g * group; h < (g + 1) * group; ++h) {
                for (int64_t i = 0; i < Sq; ++i) {
                    if (causal && k_offset + j > q_offset + i)
                        continue;
                    const double l = lse[(int64_t)h * n_stat + i];
                    if (l == -INFINITY)
                        continue;
                    double dot = 0.0, dp = 0.0;
                    for (int d = 0; d < D; ++d) {
                        dot += widen(q, dtype, (i * Hq + h) * (int64_t)D + d) * qi[d];
                        dp += widen(dout, dtype, (i * Hq + h) * (int64_t)D + d) * acc2[d];
                    }
                    const double p = exp(dot * inv_sqrt_d - l);
                    const double ds = p * (dp - dvec[(int64_t)h * n_stat + i]);
                    for (int d = 0; d < D; ++d) {
                        const double di = widen(dout, dtype, (i * Hq + h) * (int64_t)D + d);
                        ov[d] += p * di;
                        ok[d] += ds * widen(q, dtype, (i * Hq + h) * (int64_t)D + d) * inv_sqrt_d;
                    }
                }
            }
        }
        free(s);
        free(qi);
        free(acc);
        free(acc2);
    }
    free(lse);
    free(dvec);
    return failed ? 2 : 0;
}

/* Number of threads an OpenMP parallel region would use by default. */
int cp_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
