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
 *
 * Sliding window (the PyPI README's overview calls sliding windows
 * structurally compatible with Parallax and defines none): with window W > 0
 * a prefill query i sees keys max(0, i - W + 1) .. i (itself and the W - 1
 * before it), and a decode query of a sequence of n cached keys sees its last
 * min(n, W) keys. W = 0 means no window.
 *
 * Block-sparse masks (the same overview calls block sparsity structurally
 * compatible and defines none): keys and prefill queries are cut into blocks
 * of `block` positions from the start of their sequence; a byte mask per
 * (sequence, KV head) marks which key blocks a query block sees, on top of
 * causality and the window. A query always sees its own block (prefill: the
 * diagonal block; decode: the block holding the sequence's last key), so no
 * row is left without keys.
 */
#include <math.h>
#include <omp.h>
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
 * The n visible keys are positions keys[0 .. n-1] (keys == NULL: 0 .. n-1);
 * key/value at position p starts at element kv_off + p * kv_stride.
 * z and s are caller scratch of n doubles each.
 */
static void one_row(const void *q, size_t q_off, const void *r, size_t r_off,
                    const void *k, const void *v, size_t kv_off, size_t kv_stride,
                    const int64_t *keys, int64_t n, int D, int dtype, double tau, double rho,
                    double *o, double *lse, double *sbar, double *z, double *s)
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
        size_t kb = kv_off + (size_t)(keys ? keys[j] : j) * kv_stride;
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
        size_t vb = kv_off + (size_t)(keys ? keys[j] : j) * kv_stride;
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
/*
 * block_mask: NULL, or bytes [B, Hkv, mask_cols]; byte kb (nonzero: visible)
 * covers key positions kb * block .. kb * block + block - 1 of the sequence.
 */
/* Thread count of the OpenMP regions below (for timing the oracle on a given
 * number of cores; the forward's results do not depend on it). */
void oracle_set_num_threads(int n)
{
    if (n > 0)
        omp_set_num_threads(n);
}

int oracle_max_threads(void) { return omp_get_max_threads(); }

int oracle_decode(const void *q, const void *r, const void *k, const void *v, int dtype,
                  const int64_t *seq_start, const int64_t *seq_len, int B, int Hq, int Hkv, int D,
                  double tau, double rho, int64_t window, const uint8_t *block_mask,
                  int64_t block, int64_t mask_cols, int64_t n_rows, const int64_t *rows,
                  double *o)
{
    if (block_mask && block <= 0)
        return 1;
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
        int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * (size_t)(nmax > 0 ? nmax : 1));
        if (!z || !s || !keys) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t t = 0; t < total; ++t) {
                int64_t b = rows ? rows[2 * t] : t / Hq;
                int64_t h = rows ? rows[2 * t + 1] : t % Hq;
                int64_t hk = h / g;
                size_t qo = ((size_t)b * Hq + (size_t)h) * (size_t)D;
                int64_t len = seq_len[b], first = 0; /* window: the last min(len, W) */
                if (window > 0 && len > window)
                    first = len - window;
                size_t kvo = ((size_t)seq_start[b] * Hkv + (size_t)hk) * (size_t)D;
                /* visible positions: first .. len - 1, minus masked blocks
                   other than the one holding the last key */
                int64_t n = 0;
                for (int64_t p = first; p < len; ++p) {
                    int vis = 1;
                    if (block_mask && p / block != (len - 1) / block)
                        vis = block_mask[((size_t)b * Hkv + (size_t)hk) * (size_t)mask_cols +
                                         (size_t)(p / block)] != 0;
                    if (vis)
                        keys[n++] = p;
                }
                one_row(q, qo, r, qo, k, v, kvo, (size_t)Hkv * D, keys, n, D, dtype, tau, rho,
                        o + (size_t)t * D, NULL, NULL, z, s);
            }
        }
        free(z);
        free(s);
        free(keys);
    }
    return bad ? 2 : 0;
}

/*
 * Causal prefill: q, r [B, Hq, L, D]; K, V [B, Hkv, L, D]. rows: n_rows
 * (b, h, i) triples, or NULL for all B * Hq * L rows in order.
 * o: [n_rows, D]; lse, sbar: [n_rows] or NULL.
 * block_mask: NULL, or bytes [B, Hkv, nb, nb], nb = ceil(L / block); byte
 * [qb][kb] (nonzero: visible) lets query block qb see key block kb.
 */

/* Visible key positions of prefill row i (of KV head unit mask row `mrow`,
   nb blocks per side, or mrow == NULL for no mask) into keys; returns the count. */
static int64_t prefill_keys(int64_t i, int64_t window, const uint8_t *mrow, int64_t block,
                            int64_t nb, int64_t *keys)
{
    int64_t first = (window > 0 && i + 1 > window) ? i + 1 - window : 0, n = 0;
    for (int64_t p = first; p <= i; ++p)
        if (!mrow || p / block == i / block || mrow[(size_t)(i / block) * nb + p / block])
            keys[n++] = p;
    return n;
}

int oracle_prefill(const void *q, const void *r, const void *k, const void *v, int dtype, int B,
                   int Hq, int Hkv, int L, int D, double tau, double rho, int64_t window,
                   const uint8_t *block_mask, int64_t block, int64_t n_rows, const int64_t *rows,
                   double *o, double *lse, double *sbar)
{
    if (Hkv <= 0 || Hq % Hkv != 0 || D <= 0 || B <= 0 || L <= 0 || (block_mask && block <= 0))
        return 1;
    int64_t nb = block_mask ? (L + block - 1) / block : 0;
    int g = Hq / Hkv;
    int64_t total = rows ? n_rows : (int64_t)B * Hq * L;
    int bad = 0;
#pragma omp parallel
    {
        double *z = (double *)malloc(sizeof(double) * (size_t)L);
        double *s = (double *)malloc(sizeof(double) * (size_t)L);
        int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * (size_t)L);
        if (!z || !s || !keys) {
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
                const uint8_t *mrow =
                    block_mask ? block_mask + ((size_t)b * Hkv + (size_t)hk) * (size_t)(nb * nb)
                               : NULL;
                int64_t n = prefill_keys(i, window, mrow, block, nb, keys);
                one_row(q, qo, r, qo, k, v, kvo, (size_t)D, keys, n, D, dtype, tau, rho,
                        o + (size_t)t * D, lse ? lse + t : NULL, sbar ? sbar + t : NULL, z, s);
            }
        }
        free(z);
        free(s);
        free(keys);
    }
    return bad ? 2 : 0;
}

/*
 * Gradients of the causal prefill (PyPI README of parallax-kernel, "Training
 * (Triton)": o = parallax_func(q, r, k, v) is differentiated by autograd;
 * the "Helion" section holds the four gradients to the same 1e-2 tolerance
 * as the output). Given go = dLoss/do, returns dLoss/dq, dr, dk, dv.
 *
 * Plain reverse-mode differentiation of one_row's steps, taken in reverse
 * order for every row: the readout o = sum w (1 + s - sbar) v, the mean
 * sbar = sum w s, the probe scores s = rho r.k, the softmax w = softmax(z),
 * the logits z = tau q.k. Each adjoint is the transpose of its own step;
 * no identity beyond the softmax Jacobian w_j (delta_jl - w_l) is used.
 *
 * Work unit: one (b, KV head); it owns every query row of the g query heads
 * that read that KV head, so its dk / dv sums are complete within the unit.
 * units: n_units (b, hkv) pairs, or NULL for all B * Hkv units in order.
 * Outputs: dq, dr [n_units, g, L, D]; dk, dv [n_units, L, D]. r may be NULL
 * (r = 0); dr is still the gradient at r = 0.
 */
static void row_backward(const void *q, const void *r, const void *k, const void *v,
                         const void *go, size_t q_off, size_t kv_off, const int64_t *keys,
                         int64_t n, int D, int dtype, double tau, double rho, double *dq,
                         double *dr, double *dk, double *dv, double *w, double *s, double *aw,
                         double *as)
{
    /* forward steps: logits, probe scores, softmax, probe mean */
    for (int64_t j = 0; j < n; ++j) {
        size_t kb = kv_off + (size_t)keys[j] * D;
        double zq = 0.0, sr = 0.0;
        for (int d = 0; d < D; ++d) {
            double kd = elem(k, dtype, kb + d);
            zq += elem(q, dtype, q_off + d) * kd;
            if (r)
                sr += elem(r, dtype, q_off + d) * kd;
        }
        w[j] = tau * zq;
        s[j] = r ? rho * sr : 0.0;
    }
    double m = w[0];
    for (int64_t j = 1; j < n; ++j)
        if (w[j] > m)
            m = w[j];
    double l = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        w[j] = exp(w[j] - m);
        l += w[j];
    }
    for (int64_t j = 0; j < n; ++j)
        w[j] /= l;
    double sb = 0.0;
    for (int64_t j = 0; j < n; ++j)
        sb += w[j] * s[j];

    /* reverse of o = sum_j w_j v_j + sum_j w_j (s_j - sbar) v_j */
    double a_sb = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        size_t vb = kv_off + (size_t)keys[j] * D;
        double t = 0.0;
        for (int d = 0; d < D; ++d)
            t += elem(go, dtype, q_off + d) * elem(v, dtype, vb + d);
        aw[j] = (1.0 + s[j] - sb) * t;
        as[j] = w[j] * t;
        a_sb -= w[j] * t;
        double cv = w[j] * (1.0 + s[j] - sb);
        for (int d = 0; d < D; ++d)
            dv[(size_t)keys[j] * D + d] += cv * elem(go, dtype, q_off + d);
    }
    /* reverse of sbar = sum_j w_j s_j */
    for (int64_t j = 0; j < n; ++j) {
        aw[j] += a_sb * s[j];
        as[j] += a_sb * w[j];
    }
    /* reverse of w = softmax(z): a_z = w (a_w - <w, a_w>) (stored into aw) */
    double waw = 0.0;
    for (int64_t j = 0; j < n; ++j)
        waw += w[j] * aw[j];
    for (int64_t j = 0; j < n; ++j)
        aw[j] = w[j] * (aw[j] - waw);
    /* reverse of s_j = rho r.k_j and z_j = tau q.k_j */
    for (int64_t j = 0; j < n; ++j) {
        size_t kb = kv_off + (size_t)keys[j] * D;
        double cz = tau * aw[j], cs = rho * as[j];
        for (int d = 0; d < D; ++d) {
            double kd = elem(k, dtype, kb + d);
            dq[d] += cz * kd;
            dr[d] += cs * kd;
            dk[(size_t)keys[j] * D + d] += cz * elem(q, dtype, q_off + d) +
                                     (r ? cs * elem(r, dtype, q_off + d) : 0.0);
        }
    }
}

int oracle_prefill_backward(const void *q, const void *r, const void *k, const void *v,
                            const void *go, int dtype, int B, int Hq, int Hkv, int L, int D,
                            double tau, double rho, int64_t window, const uint8_t *block_mask,
                            int64_t block, int64_t n_units, const int64_t *units, double *dq,
                            double *dr, double *dk, double *dv)
{
    if (Hkv <= 0 || Hq % Hkv != 0 || D <= 0 || B <= 0 || L <= 0 || (block_mask && block <= 0))
        return 1;
    int64_t nb = block_mask ? (L + block - 1) / block : 0;
    int g = Hq / Hkv;
    int64_t total = units ? n_units : (int64_t)B * Hkv;
    size_t LD = (size_t)L * D;
    int bad = 0;
    for (int64_t u = 0; u < total && !bad; ++u) {
        int64_t b = units ? units[2 * u] : u / Hkv;
        int64_t hk = units ? units[2 * u + 1] : u % Hkv;
        size_t kvo = ((size_t)b * Hkv + (size_t)hk) * LD;
        double *dk_u = dk + (size_t)u * LD, *dv_u = dv + (size_t)u * LD;
        memset(dk_u, 0, sizeof(double) * LD);
        memset(dv_u, 0, sizeof(double) * LD);
        int64_t nrows = (int64_t)g * L;
        const uint8_t *mrow =
            block_mask ? block_mask + ((size_t)b * Hkv + (size_t)hk) * (size_t)(nb * nb) : NULL;
#pragma omp parallel
        {
            /* per-thread key-gradient sums, added into the unit in thread order */
            double *dk_t = (double *)calloc(LD, sizeof(double));
            double *dv_t = (double *)calloc(LD, sizeof(double));
            double *scr = (double *)malloc(sizeof(double) * 4 * (size_t)L);
            int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * (size_t)L);
            if (!dk_t || !dv_t || !scr || !keys) {
#pragma omp atomic write
                bad = 1;
            } else {
#pragma omp for schedule(static, 1) /* fixed row-to-thread map: deterministic sums */
                for (int64_t t = 0; t < nrows; ++t) {
                    int64_t hs = t / L, i = L - 1 - t % L; /* longest rows first */
                    int64_t h = hk * g + hs;
                    size_t qo = (((size_t)b * Hq + (size_t)h) * L + (size_t)i) * D;
                    size_t ro = (((size_t)u * g + (size_t)hs) * L + (size_t)i) * D;
                    for (int d = 0; d < D; ++d) {
                        dq[ro + d] = 0.0;
                        dr[ro + d] = 0.0;
                    }
                    int64_t n = prefill_keys(i, window, mrow, block, nb, keys);
                    row_backward(q, r, k, v, go, qo, kvo, keys, n, D, dtype, tau, rho, dq + ro,
                                 dr + ro, dk_t, dv_t, scr, scr + L, scr + 2 * (size_t)L,
                                 scr + 3 * (size_t)L);
                }
#pragma omp for ordered schedule(static, 1)
                for (int th = 0; th < omp_get_num_threads(); ++th) {
#pragma omp ordered
                    for (size_t e = 0; e < LD; ++e) {
                        dk_u[e] += dk_t[e];
                        dv_u[e] += dv_t[e];
                    }
                }
            }
            free(dk_t);
            free(dv_t);
            free(scr);
            free(keys);
        }
    }
    return bad ? 2 : 0;
}
