/*
 * tern_oracle.c -- plain f64 CPU reference for the SR4 ternary projection.
 *
 * TEST INFRASTRUCTURE ONLY (see tern_oracle.h).  Only the tests, the smoke
 * check and the benchmark's CPU-baseline leg load this library.
 *
 * Every function follows the definitions on the page "train_gpu.cu":
 *   - ternarisation: the glue kernel tg_tern_from_q (dead zone |q| < theta,
 *     otherwise the sign of q), with theta = SR4_THETA = 2 in the trainer;
 *   - W_eff: tg_apply_scale, W_eff[r, c] = scale[c] * tern[r, c] on a row-major
 *     [rows, cols] matrix, rows = input dim and cols = output dim (rows_of);
 *   - forward / input gradient: the projection is Y = X . W_eff, so its input
 *     gradient is dX = dY . W_eff^T (the trainer's fm_forward / fm_backward run
 *     these as GEMMs on W_eff);
 *   - gq: tg_gq, the gradient w.r.t. W_eff multiplied by scale[c];
 *   - sgrad: tg_scale_grad, sum over rows of grad[r, c] * tern[r, c], with the
 *     rows taken in ascending order and a double accumulator.
 * The 2-bit packed form is this library's own storage format for tern (the
 * page keeps tern as fp32); it is defined in tern_oracle.h.
 *
 * Compile with -ffp-contract=off so that no multiply-add is fused: each
 * product is rounded to double, then added, in the stated order.
 */
#include "tern_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

int oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}

/* ---- input widening: exact fp32 / bf16 -> double ---- */

static double widen_one(const void *src, int32_t dtype, int64_t i) {
    if (dtype == ORACLE_BF16) {
        /* a bf16 value is the upper half of the fp32 with the same bits */
        uint32_t u = (uint32_t)((const uint16_t *)src)[i] << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return (double)f;
    }
    return (double)((const float *)src)[i];
}

void oracle_widen(const void *src, int32_t dtype, int64_t n, double *dst) {
    for (int64_t i = 0; i < n; i++) dst[i] = widen_one(src, dtype, i);
}

/* ---- ternarisation (tg_tern_from_q) ---- */

int oracle_tern(const int8_t *q, int64_t n, int32_t theta, int8_t *tern) {
    if (theta < 1) return -1;
    for (int64_t i = 0; i < n; i++) {
        int v = q[i];
        int8_t t = 0;
        if (v >= theta) t = 1;
        else if (v <= -theta) t = -1;
        tern[i] = t;
    }
    return 0;
}

/* ---- 2-bit packing (this library's storage format) ---- */

int64_t oracle_packed_words(int64_t in, int64_t out) {
    return in * ((out + 15) / 16);
}

int oracle_pack(const int8_t *tern, int64_t in, int64_t out, uint32_t *packed) {
    int64_t wpr = (out + 15) / 16;
    for (int64_t r = 0; r < in; r++) {
        for (int64_t w = 0; w < wpr; w++) {
            uint32_t word = 0;
            for (int64_t j = 0; j < 16; j++) {
                int64_t c = w * 16 + j;
                uint32_t code = 0;
                if (c < out) {
                    int8_t t = tern[r * out + c];
                    if (t == 1) code = 1;        /* 01 */
                    else if (t == -1) code = 3;  /* 11 */
                    else if (t == 0) code = 0;   /* 00 */
                    else return -1;
                }
                word |= code << (2 * j);
            }
            packed[r * wpr + w] = word;
        }
    }
    return 0;
}

int oracle_unpack(const uint32_t *packed, int64_t in, int64_t out, int8_t *tern) {
    int64_t wpr = (out + 15) / 16;
    for (int64_t r = 0; r < in; r++) {
        for (int64_t w = 0; w < wpr; w++) {
            uint32_t word = packed[r * wpr + w];
            for (int64_t j = 0; j < 16; j++) {
                int64_t c = w * 16 + j;
                uint32_t code = (word >> (2 * j)) & 3u;
                if (c >= out) {
                    if (code != 0) return -1;
                    continue;
                }
                if (code == 0) tern[r * out + c] = 0;
                else if (code == 1) tern[r * out + c] = 1;
                else if (code == 3) tern[r * out + c] = -1;
                else return -1;
            }
        }
    }
    return 0;
}

/* ---- W_eff (tg_apply_scale), as double ---- */

static double *make_weff(const int8_t *q, int32_t theta, const float *scale,
                         int64_t in, int64_t out, int8_t **tern_out) {
    int64_t n = in * out;
    int8_t *tern = (int8_t *)malloc((size_t)(n > 0 ? n : 1));
    double *weff = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    if (!tern || !weff) { free(tern); free(weff); return NULL; }
    oracle_tern(q, n, theta, tern);
    for (int64_t r = 0; r < in; r++)
        for (int64_t c = 0; c < out; c++)
            weff[r * out + c] = (double)scale[c] * (double)tern[r * out + c];
    if (tern_out) *tern_out = tern; else free(tern);
    return weff;
}

/* ---- forward: Y = X . W_eff ---- */

int oracle_linear_fwd(const void *X, int32_t dtype, const int8_t *q, int32_t theta,
                      const float *scale, int64_t T, int64_t in, int64_t out,
                      const int64_t *rows, int64_t nrows, double *Y) {
    if (theta < 1) return -1;
    int64_t nr = rows ? nrows : T;
    if (rows)
        for (int64_t i = 0; i < nr; i++)
            if (rows[i] < 0 || rows[i] >= T) return -2;
    double *weff = make_weff(q, theta, scale, in, out, NULL);
    if (!weff) return -3;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < nr; i++) {
        int64_t t = rows ? rows[i] : i;
        double *y = Y + i * out;
        for (int64_t c = 0; c < out; c++) y[c] = 0.0;
        /* each y[c] accumulates r = 0, 1, ..., in-1 in order */
        for (int64_t r = 0; r < in; r++) {
            double x = widen_one(X, dtype, t * in + r);
            const double *w = weff + r * out;
            for (int64_t c = 0; c < out; c++) y[c] += x * w[c];
        }
    }
    free(weff);
    return 0;
}

/* ---- input gradient: dX = dY . W_eff^T ---- */

int oracle_linear_dx(const void *dY, int32_t dtype, const int8_t *q, int32_t theta,
                     const float *scale, int64_t T, int64_t in, int64_t out,
                     const int64_t *rows, int64_t nrows, double *dX) {
    if (theta < 1) return -1;
    int64_t nr = rows ? nrows : T;
    if (rows)
        for (int64_t i = 0; i < nr; i++)
            if (rows[i] < 0 || rows[i] >= T) return -2;
    double *weff = make_weff(q, theta, scale, in, out, NULL);
    if (!weff) return -3;
#pragma omp parallel
    {
        double *g = (double *)malloc((size_t)(out > 0 ? out : 1) * sizeof(double));
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < nr; i++) {
            int64_t t = rows ? rows[i] : i;
            for (int64_t c = 0; c < out; c++) g[c] = widen_one(dY, dtype, t * out + c);
            double *dx = dX + i * in;
            for (int64_t r = 0; r < in; r++) {
                /* dx[r] accumulates c = 0, 1, ..., out-1 in order */
                const double *w = weff + r * out;
                double s = 0.0;
                for (int64_t c = 0; c < out; c++) s += g[c] * w[c];
                dx[r] = s;
            }
        }
        free(g);
    }
    free(weff);
    return 0;
}

/* ---- weight side: G = X^T . dY, gq = G * scale, sgrad = column dot of G with tern ---- */

int oracle_linear_wgrad(const void *X, const void *dY, int32_t dtype, const int8_t *q,
                        int32_t theta, const float *scale, int64_t T, int64_t in,
                        int64_t out, const int64_t *cols, int64_t ncols,
                        double *G, double *gq, double *sgrad) {
    if (theta < 1) return -1;
    int64_t nc = cols ? ncols : out;
    if (cols)
        for (int64_t j = 0; j < nc; j++)
            if (cols[j] < 0 || cols[j] >= out) return -2;
    int64_t nn = in * nc;
    double *acc = (double *)malloc((size_t)(nn > 0 ? nn : 1) * sizeof(double));
    double *dys = (double *)malloc((size_t)(T * nc > 0 ? T * nc : 1) * sizeof(double));
    int8_t *tern = (int8_t *)malloc((size_t)(in * out > 0 ? in * out : 1));
    if (!acc || !dys || !tern) { free(acc); free(dys); free(tern); return -3; }
    oracle_tern(q, in * out, theta, tern);
    /* the selected columns of dY, widened */
    for (int64_t t = 0; t < T; t++)
        for (int64_t j = 0; j < nc; j++) {
            int64_t c = cols ? cols[j] : j;
            dys[t * nc + j] = widen_one(dY, dtype, t * out + c);
        }
    /* G[r, j]: each element accumulates t = 0, 1, ..., T-1 in order; threads
     * own disjoint blocks of rows r */
    const int64_t RB = 64;
    int64_t nblk = (in + RB - 1) / RB;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t b = 0; b < nblk; b++) {
        int64_t r0 = b * RB, r1 = r0 + RB < in ? r0 + RB : in;
        for (int64_t i = r0 * nc; i < r1 * nc; i++) acc[i] = 0.0;
        for (int64_t t = 0; t < T; t++) {
            const double *d = dys + t * nc;
            for (int64_t r = r0; r < r1; r++) {
                double x = widen_one(X, dtype, t * in + r);
                double *a = acc + r * nc;
                for (int64_t j = 0; j < nc; j++) a[j] += x * d[j];
            }
        }
    }
    for (int64_t r = 0; r < in; r++)
        for (int64_t j = 0; j < nc; j++) {
            int64_t c = cols ? cols[j] : j;
            if (G) G[r * nc + j] = acc[r * nc + j];
            gq[r * nc + j] = acc[r * nc + j] * (double)scale[c];
        }
    for (int64_t j = 0; j < nc; j++) {
        int64_t c = cols ? cols[j] : j;
        double s = 0.0;
        for (int64_t r = 0; r < in; r++) s += acc[r * nc + j] * (double)tern[r * out + c];
        sgrad[j] = s;
    }
    free(acc);
    free(dys);
    free(tern);
    return 0;
}

/* ---- SR4 health panel (page "train_gpu.cu", the sr4_panel fields) ----
 * Every field but churn depends on an element only through its value of q,
 * so the matrix is first reduced to a histogram over the 256 int8 values and
 * the fields are sums of bins: the class of a value by the threshold rule,
 * the rail (|v| equal to the clamp) and the dead zone (|v| below theta).
 * Churn needs the element's position: a second pass compares each element's
 * class with the previous classification.  The scale statistics run over the
 * columns in ascending order. */
int oracle_panel_add(const int8_t *q, int64_t in, int64_t out, int32_t theta, int32_t q_clamp,
                     const int8_t *prev_tern, const float *scale, int64_t counts[7],
                     double sstat[4]) {
    if (theta < 1) return -1;
    const int64_t n = in * out;
    int64_t bins[256];
    memset(bins, 0, sizeof bins);
    for (int64_t k = 0; k < n; k++) bins[(int)q[k] + 128]++;
    for (int v = -128; v <= 127; v++) {
        const int64_t h = bins[v + 128];
        const int mag = abs(v);
        counts[0] += h;                          /* total */
        if (v <= -theta) counts[1] += h;         /* class -1 */
        if (-theta < v && v < theta) counts[2] += h;   /* class 0 */
        if (v >= theta) counts[3] += h;          /* class +1 */
        if (mag == q_clamp) counts[4] += h;      /* on the rail */
        if (mag < theta) counts[5] += h;         /* in the dead zone */
    }
    if (prev_tern) {
        for (int64_t k = 0; k < n; k++) {
            const int8_t now = q[k] >= theta ? 1 : (q[k] <= -theta ? -1 : 0);
            counts[6] += prev_tern[k] != now;
        }
    }
    for (int64_t c = 0; c < out; c++) {
        const double sv = (double)scale[c];
        sstat[0] += 1.0;
        sstat[1] += sv;
        sstat[2] = sv < sstat[2] ? sv : sstat[2];
        sstat[3] = sv > sstat[3] ? sv : sstat[3];
    }
    return 0;
}

/* ---- scale step: AdamW on the per-column scale (textbook form, see header) ---- */

int oracle_scale_adamw(const double *sgrad, double *scale, double *m, double *v, int64_t out,
                       int32_t t, double lr, double scale_lr, double b1, double b2, double eps,
                       double wd) {
    if (t < 1) return -1;
    const double bc1 = 1.0 - pow(b1, (double)t), bc2 = 1.0 - pow(b2, (double)t);
    for (int64_t c = 0; c < out; c++) {
        const double g = sgrad[c] * scale_lr / lr;
        m[c] = b1 * m[c] + (1.0 - b1) * g;
        v[c] = b2 * v[c] + (1.0 - b2) * g * g;
        const double mhat = m[c] / bc1, vhat = v[c] / bc2;
        scale[c] -= lr * (mhat / (sqrt(vhat) + eps) + wd * scale[c]);
    }
    return 0;
}
