/*
 * tern_oracle.h -- CPU reference ("oracle") for the SR4 ternary projection.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link or
 * call this code: it exists so that tests, the smoke check and the benchmark's
 * CPU-baseline leg can compare the HIP library against a plain, slow, obviously
 * correct computation.  It shares no code, header, table or helper with the HIP
 * library under ternary_weight_linear_tern_amd/csrc.
 *
 * Source of the method: the page "train_gpu.cu" (Foundry, cuda_kernels), its
 * header comment on the optimizer split (ternary projections with a
 * per-output-column scale, W_eff[r,c] = scale[c] * ternary(q)[r,c]) and its
 * "device glue kernels" section (tg_tern_from_q, tg_apply_scale, tg_gq,
 * tg_scale_grad).  The shape rule (rows = input dim, cols = output dim) is the
 * page's is_ternary_name / rows_of pair.
 *
 * Arithmetic: every floating-point input (fp32 or bf16 bits) is widened exactly
 * to double and every sum is accumulated in double in ascending index order.
 * Outputs are double.  Loops may be nested in any order that keeps each output
 * element's own summation order ascending, so results do not depend on the
 * number of OpenMP threads.
 *
 * Parity pins: every function here is pinned by the CPU tests (hand-derived
 * tables, a hand-packed word, brute force in pure Python on tiny shapes, the
 * +-1 sign-matrix special case against numpy's matmul, five-way bilinear
 * identities, finite differences of exactly linear functionals, and planted
 * mutants that the pins must catch).  No function is "parity unpinned".
 */
#ifndef TERN_ORACLE_H
#define TERN_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* storage types of floating-point inputs */
#define ORACLE_F32  0
#define ORACLE_BF16 1

/* tern[i] = +1 if q[i] >= theta, -1 if q[i] <= -theta, else 0.
 * Returns 0, or -1 if theta < 1 (the rule is only a sign-with-dead-zone for
 * theta >= 1). */
int oracle_tern(const int8_t *q, int64_t n, int32_t theta, int8_t *tern);

/* Number of u32 words of the 2-bit packed form of an [in, out] matrix:
 * in * ceil(out / 16). */
int64_t oracle_packed_words(int64_t in, int64_t out);

/* 2-bit packing of a row-major [in, out] ternary matrix.  Code of (r, c):
 * 0 -> 00, +1 -> 01, -1 -> 11, stored at bits 2*(c % 16) .. 2*(c % 16) + 1 of
 * word r * ceil(out/16) + c / 16 (least significant bits first).  Padding codes
 * of a partial last word are 00.  Returns 0, or -1 on a tern value outside
 * {-1, 0, +1}. */
int oracle_pack(const int8_t *tern, int64_t in, int64_t out, uint32_t *packed);

/* Inverse of oracle_pack.  Returns 0, or -1 if a reserved code (10) or a
 * nonzero padding code is found. */
int oracle_unpack(const uint32_t *packed, int64_t in, int64_t out, int8_t *tern);

/* Widen n stored values (fp32 or bf16 bits) to double, exactly. */
void oracle_widen(const void *src, int32_t dtype, int64_t n, double *dst);

/* Forward: Y[t, c] = sum_r X[t, r] * W_eff[r, c],  W_eff = scale[c] * tern(q)[r, c].
 * rows == NULL: all T token rows, Y is [T, out].
 * rows != NULL: Y is [nrows, out] holding token rows rows[0..nrows-1].
 * Returns 0, -1 on bad theta, -2 on a row index outside [0, T). */
int oracle_linear_fwd(const void *X, int32_t dtype, const int8_t *q, int32_t theta,
                      const float *scale, int64_t T, int64_t in, int64_t out,
                      const int64_t *rows, int64_t nrows, double *Y);

/* Input gradient: dX[t, r] = sum_c dY[t, c] * W_eff[r, c].
 * rows as in oracle_linear_fwd; dX is [T or nrows, in]. */
int oracle_linear_dx(const void *dY, int32_t dtype, const int8_t *q, int32_t theta,
                     const float *scale, int64_t T, int64_t in, int64_t out,
                     const int64_t *rows, int64_t nrows, double *dX);

/* Weight-side gradients for the output columns cols[0..ncols-1] (cols == NULL:
 * all out columns, ncols ignored):
 *   G[r, j]     = sum_t X[t, r] * dY[t, cols[j]]         (gradient w.r.t. W_eff)
 *   gq[r, j]    = G[r, j] * scale[cols[j]]                (gradient w.r.t. tern)
 *   sgrad[j]    = sum_r G[r, j] * tern[r, cols[j]]        (gradient w.r.t. scale)
 * G, gq are [in, ncols] row-major; G may be NULL.  Returns 0, -1 on bad theta,
 * -2 on a column index outside [0, out). */
int oracle_linear_wgrad(const void *X, const void *dY, int32_t dtype, const int8_t *q,
                        int32_t theta, const float *scale, int64_t T, int64_t in,
                        int64_t out, const int64_t *cols, int64_t ncols,
                        double *G, double *gq, double *sgrad);

/* SR4 health panel of one ternary matrix, added to running totals (page
 * "train_gpu.cu", sr4_panel and sr4_panel_compute).  For every element of q
 * [in, out]: its class under the threshold rule (negative, zero, positive),
 * rail (|q| == q_clamp), dead (|q| < theta), and, when prev_tern is not NULL,
 * churn (the class differs from prev_tern, the previous classification).  For
 * every column of scale [out]: its sum (double, ascending), minimum, maximum.
 *   counts[7] += {total, neg, zero, pos, rail, dead, churn}
 *   sstat[0] += out (columns), sstat[1] += sum, sstat[2] = min, sstat[3] = max
 *   (sstat[2], sstat[3] start at +/-HUGE_VAL for an empty panel).
 * Returns 0, or -1 if theta < 1. */
int oracle_panel_add(const int8_t *q, int64_t in, int64_t out, int32_t theta, int32_t q_clamp,
                     const int8_t *prev_tern, const float *scale, int64_t counts[7],
                     double sstat[4]);

/* The scale step that follows the scale gradient (page "train_gpu.cu": the
 * trainer multiplies sgrad by scale_lr / lr and calls its AdamW launcher on
 * the per-column scale, which forms bc1 = 1 - b1^t and bc2 = 1 - b2^t; the
 * update kernel's body is not on the page).  Textbook AdamW with decoupled
 * weight decay, in double, element by element:
 *   g = sgrad[c] * scale_lr / lr
 *   m[c] = b1 m[c] + (1 - b1) g;   v[c] = b2 v[c] + (1 - b2) g^2
 *   scale[c] -= lr ((m[c] / bc1) / (sqrt(v[c] / bc2) + eps) + wd scale[c])
 * scale, m, v (double) are updated in place.  Returns 0, or -1 if t < 1. */
int oracle_scale_adamw(const double *sgrad, double *scale, double *m, double *v, int64_t out,
                       int32_t t, double lr, double scale_lr, double b1, double b2, double eps,
                       double wd);

/* Threads the OpenMP build uses (1 without OpenMP). */
int oracle_num_threads(void);

/* Use n >= 1 threads from now on (results do not depend on it: every output
 * element keeps its own summation order); returns the new count. */
int oracle_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
