/*
 * Parallax attention oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, double-precision CPU implementation of what the Parallax
 * attention readout computes. Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load it; the product library never does.
 * It shares no code, header or table with the GPU library.
 *
 * Definition followed (one output row; "Parallax: Parameterized Local Linear
 * Attention for Language Modeling", the neuraltrendhub summary "What the paper
 * found" and the original abstract: the softmax readout is kept and a learned
 * query-like projector R probes the key-value covariance; the
 * encorp.ai article, section on removing the conjugate-gradient solver: the
 * projector W_R replaces the local-linear solve and W_R = 0 gives softmax
 * attention back exactly). With visible keys J, query q and probe r:
 *
 *   z_j  = tau * <q, k_j>                      softmax logits
 *   w_j  = exp(z_j - max z) / sum exp(. - max z)
 *   s_j  = rho * <r, k_j>                      probe scores
 *   sbar = sum_j w_j s_j
 *   o    = sum_j w_j v_j  +  sum_j w_j (s_j - sbar) v_j
 *
 * The second sum is the w-weighted covariance of (s, v): the local-linear
 * intercept vbar + Cov_w(v, k) r with the solver's output replaced by r.
 * Two passes, no streaming, no splitting, every step in double from the
 * exact input values widened to double.
 *
 * Readings where the pages are silent: the correction enters with a plus
 * sign; s is not scaled by tau (rho defaults to 1); query head h reads KV
 * head h / (Hq / Hkv); prefill is causal with key j visible to query i iff
 * j <= i; decode sees every cached key of its sequence; an empty key set
 * gives o = 0, lse = -inf, sbar = 0.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1
#define ORC_F64 2 /* used by the pins, so that they run at full double precision */

static double elem(const void *p, int dtype, size_t i)
{
    if (dtype == ORC_F32)
        return (double)((const float *)p)[i];
    if (dtype == ORC_F64)
        return ((const double *)p)[i];
    uint32_t b = ((uint32_t)((const uint16_t *)p)[i]) << 16;
    float f;
    memcpy(&f, &b, 4);
    return (double)f;
}

/*
 * One output row. q/r at element offsets q_off/r_off (r may be NULL: r = 0).
 * Key/value j (0 <= j < n) starts at element kv_off + j * kv_stride.
 * z and s are caller scratch of n doubles each.
 */
static void one_row(const void *q, size_t q_off, const void *r, size_t r_off,
                    const void *k, const void *v, size_t kv_off, size_t kv_stride, int64_t n,
                    int D, int dtype, double tau, double rho, double *o, double *lse,
                    double *sbar, double *z, double *s)
{
    if (n <= 0) {
        for (int d = 0; d < D; ++d)
            o[d] = 0.0;
        if (lse)
            *lse = -INFINITY;
        if (sbar)
            *sbar = 0.0;
        return;
    }
    /* logits and probe scores */
    for (int64_t j = 0; j < n; ++j) {
        size_t kb = kv_off + (size_t)j * kv_stride;
        double zq = 0.0, sr = 0.0;
        for (int d = 0; d < D; ++d) {
            double kd = elem(k, dtype, kb + d);
            zq += elem(q, dtype, q_off + d) * kd;
            if (r)
                sr += elem(r, dtype, r_off + d) * kd;
        }
        z[j] = tau * zq;
        s[j] = r ? rho * sr : 0.0;
    }
    /* softmax weights (stored back into z) */
    double m = z[0];
    for (int64_t j = 1; j < n; ++j)
        if (z[j] > m)
            m = z[j];
    double l = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        z[j] = exp(z[j] - m);
        l += z[j];
    }
    for (int64_t j = 0; j < n; ++j)
        z[j] /= l;
    /* first pass: weighted mean of the probe scores */
    double sb = 0.0;
    for (int64_t j = 0; j < n; ++j)
        sb += z[j] * s[j];
    /* second pass: softmax readout plus the centred correction */
    for (int d = 0; d < D; ++d)
        o[d] = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        size_t vb = kv_off + (size_t)j * kv_stride;
        double wj = z[j];
        double cj = z[j] * (s[j] - sb);
        for (int d = 0; d < D; ++d) {
            double vd = elem(v, dtype, vb + d);
            o[d] += wj * vd + cj * vd;
        }
    }
    if (lse)
        *lse = m + log(l);
    if (sbar)
        *sbar = sb;
}

/*
 * Decode: q, r [B, Hq, D]; K, V rows [tokens, Hkv, D] with sequence b at
 * tokens seq_start[b] .. seq_start[b] + seq_len[b] - 1 (dense [B, L, Hkv, D]
 * has seq_start[b] = b * L). rows: n_rows (b, h) pairs, or NULL for all
 * B * Hq rows in order. o: [n_rows, D].
 */
int oracle_decode(const void *q, const void *r, const void *k, const void *v, int dtype,
                  const int64_t *seq_start, const int64_t *seq_len, int B, int Hq, int Hkv, int D,
                  double tau, double rho, int64_t n_rows, const int64_t *rows, double *o)
{
    if (Hkv <= 0 || Hq % Hkv != 0 || D <= 0 || B <= 0)
        return 1;
    int g = Hq / Hkv;
    int64_t total = rows ? n_rows : (int64_t)B * Hq;
    int64_t nmax = 0;
    for (int b = 0; b < B; ++b)
        if (seq_len[b] > nmax)
            nmax = seq_len[b];
    int bad = 0;
#pragma omp parallel
    {
        double *z = (double *)malloc(sizeof(double) * (size_t)(nmax > 0 ? nmax : 1));
        double *s = (double *)malloc(sizeof(double) * (size_t)(nmax > 0 ? nmax : 1));
        if (!z || !s) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t t = 0; t < total; ++t) {
                int64_t b = rows ? rows[2 * t] : t / Hq;
                int64_t h = rows ? rows[2 * t + 1] : t % Hq;
                int64_t hk = h / g;
                size_t qo = ((size_t)b * Hq + (size_t)h) * (size_t)D;
                size_t kvo = ((size_t)seq_start[b] * Hkv + (size_t)hk) * (size_t)D;
                one_row(q, qo, r, qo, k, v, kvo, (size_t)Hkv * D, seq_len[b], D, dtype, tau, rho,
                        o + (size_t)t * D, NULL, NULL, z, s);
            }
        }
        free(z);
        free(s);
    }
    return bad ? 2 : 0;
}

/*
 * Causal prefill: q, r [B, Hq, L, D]; K, V [B, Hkv, L, D]. rows: n_rows
 * (b, h, i) triples, or NULL for all B * Hq * L rows in order.
 * o: [n_rows, D]; lse, sbar: [n_rows] or NULL.
 */
int oracle_prefill(const void *q, const void *r, const void *k, const void *v, int dtype, int B,
                   int Hq, int Hkv, int L, int D, double tau, double rho, int64_t n_rows,
                   const int64_t *rows, double *o, double *lse, double *sbar)
{
    if (Hkv <= 0 || Hq % Hkv != 0 || D <= 0 || B <= 0 || L <= 0)
        return 1;
    int g = Hq / Hkv;
    int64_t total = rows ? n_rows : (int64_t)B * Hq * L;
    int bad = 0;
#pragma omp parallel
    {
        double *z = (double *)malloc(sizeof(double) * (size_t)L);
        double *s = (double *)malloc(sizeof(double) * (size_t)L);
        if (!z || !s) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t t = 0; t < total; ++t) {
                int64_t b, h, i;
                if (rows) {
                    b = rows[3 * t];
                    h = rows[3 * t + 1];
                    i = rows[3 * t + 2];
                } else {
                    i = t % L;
                    h = (t / L) % Hq;
                    b = t / ((int64_t)L * Hq);
                }
                int64_t hk = h / g;
                size_t qo = (((size_t)b * Hq + (size_t)h) * (size_t)L + (size_t)i) * (size_t)D;
                size_t kvo = ((size_t)b * Hkv + (size_t)hk) * (size_t)L * (size_t)D;
                one_row(q, qo, r, qo, k, v, kvo, (size_t)D, i + 1, D, dtype, tau, rho,
                        o + (size_t)t * D, lse ? lse + t : NULL, sbar ? sbar + t : NULL, z, s);
            }
        }
        free(z);
        free(s);
    }
    return bad ? 2 : 0;
}
