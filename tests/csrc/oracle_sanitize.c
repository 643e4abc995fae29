/* Driver of the CPU oracle and the input generator for a sanitizer build
 * (AddressSanitizer + UndefinedBehaviorSanitizer): every exported function on
 * small inputs, the sampled-row / sampled-column forms, zero sizes and the
 * error returns.  Exits 0 when every call returns what its header states;
 * the sanitizers abort on any out-of-bounds access or undefined behaviour.
 * Test infrastructure only. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "tern_oracle.h"

uint64_t synth_stream_seed(uint64_t base, uint64_t config_id, uint64_t proj_id, uint64_t tensor_id);
uint64_t synth_u64(uint64_t seed, uint64_t i);
void synth_normal_f32(uint64_t seed, int64_t n, double mean, double std, float *out);
void synth_normal_bf16(uint64_t seed, int64_t n, double mean, double std, uint16_t *out);
void synth_uniform_f32(uint64_t seed, int64_t n, double lo, double hi, float *out);
void synth_lognormal_f32(uint64_t seed, int64_t n, double mu, double sigma, float *out);
void synth_int8_uniform(uint64_t seed, int64_t n, int32_t lo, int32_t hi, int8_t *out);
void synth_int8_zero_or_pm(uint64_t seed, int64_t n, double p_zero, int32_t mag_lo, int32_t mag_hi,
                           int8_t *out);
void synth_f32_to_bf16(const float *src, int64_t n, uint16_t *out);
void synth_sample_indices(uint64_t seed, int64_t n, int64_t range, int64_t *out);

static int fails = 0;
#define CHECK(c)                                                    \
    do {                                                            \
        if (!(c)) {                                                 \
            fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
            fails++;                                                \
        }                                                           \
    } while (0)

/* exact-size heap buffers, so that the address sanitizer sees one element past
 * the end as an overflow */
static void *xalloc(size_t n) {
    void *p = malloc(n ? n : 1);
    if (!p) abort();
    memset(p, 0, n ? n : 1);
    return p;
}

static void one_shape(int64_t T, int64_t in, int64_t out, int bf) {
    const int64_t nx = T * in, ny = T * out, nw = in * out;
    float *Xf = xalloc(sizeof(float) * nx), *dYf = xalloc(sizeof(float) * ny);
    uint16_t *Xb = xalloc(2 * nx), *dYb = xalloc(2 * ny);
    int8_t *q = xalloc(nw), *tern = xalloc(nw), *back = xalloc(nw);
    float *scale = xalloc(sizeof(float) * out);
    uint64_t s = synth_stream_seed(1234, 77, (uint64_t)in, (uint64_t)out);
    synth_normal_f32(s, nx, 0.0, 1.0, Xf);
    synth_normal_f32(s + 1, ny, 0.0, 0.01, dYf);
    synth_normal_bf16(s + 2, nx, 0.0, 1.0, Xb);
    synth_normal_bf16(s + 3, ny, 0.0, 0.01, dYb);
    synth_int8_uniform(s + 4, nw, -7, 7, q);
    synth_uniform_f32(s + 5, out, 0.01, 0.1, scale);
    const void *X = bf ? (const void *)Xb : (const void *)Xf;
    const void *dY = bf ? (const void *)dYb : (const void *)dYf;
    const int32_t dt = bf ? ORACLE_BF16 : ORACLE_F32;

    CHECK(oracle_tern(q, nw, 2, tern) == 0);
    const int64_t words = oracle_packed_words(in, out);
    uint32_t *packed = xalloc(4 * (size_t)words);
    CHECK(oracle_pack(tern, in, out, packed) == 0);
    CHECK(oracle_unpack(packed, in, out, back) == 0);
    CHECK(memcmp(tern, back, (size_t)nw) == 0);

    double *Y = xalloc(sizeof(double) * ny), *dX = xalloc(sizeof(double) * nx);
    double *G = xalloc(sizeof(double) * nw), *gq = xalloc(sizeof(double) * nw);
    double *sg = xalloc(sizeof(double) * out);
    CHECK(oracle_linear_fwd(X, dt, q, 2, scale, T, in, out, NULL, 0, Y) == 0);
    CHECK(oracle_linear_dx(dY, dt, q, 2, scale, T, in, out, NULL, 0, dX) == 0);
    CHECK(oracle_linear_wgrad(X, dY, dt, q, 2, scale, T, in, out, NULL, 0, G, gq, sg) == 0);
    CHECK(oracle_linear_wgrad(X, dY, dt, q, 2, scale, T, in, out, NULL, 0, NULL, gq, sg) == 0);

    /* sampled rows and columns (the last index of each range included) */
    if (T > 0 && out > 0) {
        const int64_t nr = 3, nc = 2;
        int64_t rows[3], cols[2];
        synth_sample_indices(s + 6, nr - 1, T, rows);
        rows[nr - 1] = T - 1;
        synth_sample_indices(s + 7, nc - 1, out, cols);
        cols[nc - 1] = out - 1;
        double *Ys = xalloc(sizeof(double) * nr * out), *dXs = xalloc(sizeof(double) * nr * in);
        double *gqs = xalloc(sizeof(double) * in * nc), *sgs = xalloc(sizeof(double) * nc);
        CHECK(oracle_linear_fwd(X, dt, q, 2, scale, T, in, out, rows, nr, Ys) == 0);
        CHECK(oracle_linear_dx(dY, dt, q, 2, scale, T, in, out, rows, nr, dXs) == 0);
        CHECK(oracle_linear_wgrad(X, dY, dt, q, 2, scale, T, in, out, cols, nc, NULL, gqs, sgs) == 0);
        CHECK(memcmp(Ys + (nr - 1) * out, Y + (T - 1) * out, sizeof(double) * out) == 0);
        CHECK(sgs[nc - 1] == sg[out - 1]);
        /* an index outside the range is refused */
        rows[0] = T;
        CHECK(oracle_linear_fwd(X, dt, q, 2, scale, T, in, out, rows, nr, Ys) == -2);
        cols[0] = -1;
        CHECK(oracle_linear_wgrad(X, dY, dt, q, 2, scale, T, in, out, cols, nc, NULL, gqs, sgs) == -2);
        free(Ys); free(dXs); free(gqs); free(sgs);
    }
    CHECK(oracle_linear_fwd(X, dt, q, 0, scale, T, in, out, NULL, 0, Y) == -1);

    /* panel: with and without a previous classification */
    int64_t counts[7] = {0, 0, 0, 0, 0, 0, 0};
    double sstat[4] = {0.0, 0.0, HUGE_VAL, -HUGE_VAL};
    CHECK(oracle_panel_add(q, in, out, 2, 7, NULL, scale, counts, sstat) == 0);
    CHECK(oracle_panel_add(q, in, out, 2, 7, tern, scale, counts, sstat) == 0);
    CHECK(counts[0] == 2 * nw && counts[6] == 0);
    CHECK(oracle_panel_add(q, in, out, 0, 7, NULL, scale, counts, sstat) == -1);

    /* scale step */
    double *sgd = xalloc(sizeof(double) * out), *sc = xalloc(sizeof(double) * out);
    double *m = xalloc(sizeof(double) * out), *v = xalloc(sizeof(double) * out);
    for (int64_t c = 0; c < out; c++) { sgd[c] = sg[c]; sc[c] = scale[c]; }
    CHECK(oracle_scale_adamw(sgd, sc, m, v, out, 1, 1e-3, 1e-3, 0.9, 0.999, 1e-8, 0.0) == 0);
    CHECK(oracle_scale_adamw(sgd, sc, m, v, out, 0, 1e-3, 1e-3, 0.9, 0.999, 1e-8, 0.0) == -1);

    free(Xf); free(dYf); free(Xb); free(dYb); free(q); free(tern); free(back); free(scale);
    free(packed); free(Y); free(dX); free(G); free(gq); free(sg); free(sgd); free(sc); free(m); free(v);
}

int main(void) {
    /* the generator's remaining exports */
    float f[37], g[37];
    uint16_t b[37];
    int8_t z[37];
    int64_t idx[5];
    synth_lognormal_f32(5, 37, log(0.02), 0.5, f);
    synth_f32_to_bf16(f, 37, b);
    synth_int8_zero_or_pm(6, 37, 0.3, 1, 7, z);
    synth_sample_indices(7, 5, 11, idx);
    synth_uniform_f32(8, 37, -1.0, 1.0, g);
    for (int i = 0; i < 5; i++) CHECK(idx[i] >= 0 && idx[i] < 11);
    for (int i = 0; i < 37; i++) CHECK(z[i] == 0 || (abs(z[i]) >= 1 && abs(z[i]) <= 7));
    (void)synth_u64(9, 3);
    CHECK(oracle_set_num_threads(1) == 1 && oracle_num_threads() == 1);

    /* all int8 values through the threshold rule */
    int8_t all[256], t[256];
    for (int i = 0; i < 256; i++) all[i] = (int8_t)(i - 128);
    for (int th = 1; th <= 127; th += 21) CHECK(oracle_tern(all, 256, th, t) == 0);
    CHECK(oracle_tern(all, 256, 0, t) == -1);

    /* shapes: ragged words, a single element, zero sizes */
    const int64_t shapes[][3] = {{1, 1, 1}, {3, 5, 17}, {7, 8, 16}, {5, 24, 40}, {0, 8, 8}, {4, 0, 8},
                                 {4, 8, 0}, {2, 33, 31}};
    for (size_t k = 0; k < sizeof shapes / sizeof shapes[0]; k++)
        for (int bf = 0; bf < 2; bf++) one_shape(shapes[k][0], shapes[k][1], shapes[k][2], bf);
    if (fails) {
        fprintf(stderr, "%d checks failed\n", fails);
        return 1;
    }
    printf("oracle and generator clean under the sanitizers\n");
    return 0;
}
