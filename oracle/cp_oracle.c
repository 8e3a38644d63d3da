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

/* Number of threads an OpenMP parallel region would use by default. */
int cp_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
