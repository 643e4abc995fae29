/*
 * tern.h -- C ABI of libtern, the MI355X (gfx950) forward and backward of the
 * SR4 ternary projection.
 *
 * The method (page "train_gpu.cu", Foundry cuda_kernels: header comment on the
 * optimizer split and the "device glue kernels" section):
 *   - a ternary projection keeps an int4 accumulator q (int8 storage) and a
 *     per-output-column fp32 scale;
 *   - tern = sign(q) where |q| >= theta, else 0 (tg_tern_from_q; the trainer
 *     uses theta = SR4_THETA = 2 and clamps q to +-SR4_Q_CLAMP = 7);
 *   - W_eff[r, c] = scale[c] * tern[r, c] on a row-major [in, out] matrix
 *     (tg_apply_scale; rows = input dim, cols = output dim per rows_of);
 *   - forward Y = X . W_eff; backward dX = dY . W_eff^T, the weight gradient
 *     G = X^T . dY, gq = G * scale[c] (tg_gq) and the scale gradient
 *     sgrad[c] = sum_r G[r, c] * tern[r, c] (tg_scale_grad).
 *
 * Conventions for every entry point:
 *   - All array pointers are DEVICE pointers owned by the caller: contiguous,
 *     row-major, 16-byte aligned.  The library allocates nothing, frees
 *     nothing, keeps no state between calls and never synchronises.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *     work is enqueued on it in order; results are ready when the caller's
 *     next synchronisation on that stream returns.
 *   - Inputs are only read; outputs are fully overwritten (nothing is
 *     accumulated into them).
 *   - Return value: TERN_OK (0) or a negative TERN_ERR_* code.  Arguments are
 *     validated before anything is enqueued; on an error nothing is enqueued.
 *     A device fault after a successful enqueue surfaces at the caller's next
 *     synchronisation, as for any HIP launch.
 *   - Shapes: T (tokens), in, out >= 0; in and out must be multiples of 8 so
 *     that every activation row starts 16-byte aligned.  Zero sizes are valid
 *     and give the mathematically right (possibly all-zero) outputs.
 *   - Outputs may not overlap inputs or each other (TERN_ERR_ALIAS).
 *   - Non-finite inputs give unspecified (but memory-safe) outputs.
 */
#ifndef TERN_H
#define TERN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types */
#define TERN_F32  0  /* IEEE binary32 */
#define TERN_BF16 1  /* bfloat16 (upper half of a binary32) */

/* status codes */
#define TERN_OK             0
#define TERN_ERR_NULL      -1  /* a required pointer is NULL */
#define TERN_ERR_SHAPE     -2  /* negative size, in or out not a multiple of 8, or too large */
#define TERN_ERR_THETA     -3  /* theta outside [1, 127] */
#define TERN_ERR_DTYPE     -4  /* unsupported element type combination */
#define TERN_ERR_ALIGN     -5  /* a pointer is not 16-byte aligned */
#define TERN_ERR_WORKSPACE -6  /* workspace missing or smaller than required */
#define TERN_ERR_ALIAS     -7  /* an output overlaps an input or another output */
#define TERN_ERR_HIP       -8  /* the HIP runtime refused a launch */
#define TERN_ERR_VALUE     -9  /* a scalar argument outside its range (optimizer step, learning rate) */
#define TERN_ERR_SCRATCH  -10  /* the sizes need more than the library's static scratch */

/* Number of uint32 words of a packed ternary handle for an [in, out] matrix
 * (0 if in or out is 0, -1 for negative sizes).  The caller allocates this
 * many words (4-byte aligned); tern_materialize fills all of them.  Layout:
 *   words [0, in*ceil(out/16)): the canonical 2-bit matrix (see
 *       tern_materialize);
 *   from word ceil(in*ceil(out/16) / 64) * 64: two fragment-ordered copies of
 *       the same codes, the forward operand (ceil(out/256) * ceil(in/32) * 512
 *       words) then the dX operand (ceil(in/256) * ceil(out/32) * 512 words),
 *       ordered for the loads of the GEMM kernels.  They carry no
 *       information beyond the canonical matrix. */
int64_t tern_packed_words(int64_t in, int64_t out);

/*
 * tern_materialize -- ternarise q and store it 2-bit packed.
 *   q           int8 [in, out], read only.  Any int8 value is accepted; the
 *               dead-zone rule is applied as is (the +-7 clamp belongs to the
 *               optimizer, not to this step).
 *   theta       dead-zone threshold, 1 <= theta <= 127 (the trainer uses 2).
 *   tern_packed handle of tern_packed_words(in, out) uint32 words, written.
 *               Canonical part: code of (r, c) 00 = 0, 01 = +1, 11 = -1 (10 is
 *               never written), at bits 2*(c % 16) .. 2*(c % 16)+1 of word
 *               r*ceil(out/16) + c/16, least significant bits first; padding
 *               codes of a partial last word are 00.  The fragment-ordered
 *               copies that follow are derived from it.  One handle serves the
 *               forward and the backward of the same step.
 * Errors: NULL, SHAPE, THETA, ALIGN, ALIAS, HIP.
 */
int tern_materialize(const int8_t *q, int64_t in, int64_t out, int32_t theta,
                     uint32_t *tern_packed, void *stream);

/*
 * tern_linear_fwd -- Y = X . W_eff with W_eff[r, c] = scale[c] * tern[r, c].
 *   X           [T, in] of act_dtype (TERN_F32 or TERN_BF16).
 *   tern_packed handle written by tern_materialize for these in, out.
 *   scale       fp32 [out].
 *   Y           [T, out] of y_dtype: TERN_F32, or TERN_BF16 (round to nearest
 *               even of the fp32 result) when act_dtype is TERN_BF16.
 * Arithmetic: products of X with +-1/0 accumulate in fp32 on the matrix cores;
 * the scale multiplies each fp32 column sum once.
 * Errors: NULL, SHAPE, DTYPE, ALIGN, ALIAS, HIP.
 */
int tern_linear_fwd(const void *X, int32_t act_dtype, const uint32_t *tern_packed,
                    const float *scale, int64_t T, int64_t in, int64_t out,
                    void *Y, int32_t y_dtype, void *stream);

/*
 * tern_linear_bwd_workspace_bytes -- device workspace (bytes) that
 * tern_linear_bwd and tern_linear_bwd_dw need for these sizes, with either
 * activation type (the larger of the two types' plans: the split of the
 * weight-gradient product over tokens depends on the element size).  Returns
 * 0 for invalid sizes.  The value depends only on its arguments.
 */
size_t tern_linear_bwd_workspace_bytes(int64_t T, int64_t in, int64_t out);

/*
 * tern_linear_bwd -- all gradients of the projection.
 *   X, dY       [T, in] and [T, out] of act_dtype (TERN_F32 or TERN_BF16).
 *   tern_packed, scale  as for tern_linear_fwd.
 *   dX          [T, in]  = dY . W_eff^T, dx_dtype must be TERN_F32.
 *   gq          fp32 [in, out] = (X^T . dY)[r, c] * scale[c].
 *   sgrad       fp32 [out]     = sum_r (X^T . dY)[r, c] * tern[r, c].
 *   workspace   device scratch of at least
 *               tern_linear_bwd_workspace_bytes(T, in, out) bytes
 *               (may be NULL when that is 0).  Its contents on entry are
 *               ignored and on return are unspecified.
 * Arithmetic: fp32 accumulation on the matrix cores.  With bf16 activations
 * the scale is folded into the bf16 B operand of the dX product as
 * +-bf16(scale[c]) (round to nearest even), since the scale sits on that
 * product's reduction index.  sgrad is summed in a fixed order (fp32 within a
 * row tile, then the row-tile partials in ascending order in f64, in eight
 * consecutive groups whose sums are added in ascending order), so repeated
 * calls on the same inputs give bitwise-identical results.
 * Errors: NULL, SHAPE, DTYPE, ALIGN, WORKSPACE, ALIAS, HIP.
 */
int tern_linear_bwd(const void *X, const void *dY, int32_t act_dtype,
                    const uint32_t *tern_packed, const float *scale,
                    int64_t T, int64_t in, int64_t out,
                    void *dX, int32_t dx_dtype, float *gq, float *sgrad,
                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * tern_linear_bwd_dx -- only the input gradient of tern_linear_bwd:
 *   dX [T, in] (TERN_F32) = dY . W_eff^T.  Same argument rules; no workspace.
 * Errors: NULL, SHAPE, DTYPE, ALIGN, ALIAS, HIP.
 */
int tern_linear_bwd_dx(const void *dY, int32_t act_dtype, const uint32_t *tern_packed,
                       const float *scale, int64_t T, int64_t in, int64_t out,
                       void *dX, int32_t dx_dtype, void *stream);

/*
 * tern_linear_bwd_dw -- only the weight-side gradients of tern_linear_bwd:
 *   gq [in, out] and sgrad [out] as defined there, with the same workspace
 *   (tern_linear_bwd_workspace_bytes).  tern_linear_bwd is exactly
 *   tern_linear_bwd_dx followed by tern_linear_bwd_dw on the same stream.
 * Errors: NULL, SHAPE, DTYPE, ALIGN, WORKSPACE, ALIAS, HIP.
 */
int tern_linear_bwd_dw(const void *X, const void *dY, int32_t act_dtype,
                       const uint32_t *tern_packed, const float *scale,
                       int64_t T, int64_t in, int64_t out,
                       float *gq, float *sgrad, void *workspace, size_t workspace_bytes,
                       void *stream);

/*
 * tern_linear_bwd_noalloc -- tern_linear_bwd without a workspace argument, for
 * callers that cannot allocate device memory (code under graph capture, tight
 * serving loops, harnesses that forbid allocation).  Same arguments, results
 * and errors as tern_linear_bwd, minus the workspace.  The backward's scratch
 * (sgrad partial table, split partial products of G) lives in a static device
 * array of 64 MiB that the library holds on each GPU it runs on until the
 * process ends; where the usual plan needs more, the weight-gradient product
 * is split over fewer token ranges (the results then differ from
 * tern_linear_bwd's by fp32 rounding only).  The call allocates nothing: no
 * hipMalloc, hipFree or allocating library routine.  Its first call on a
 * device looks up that device's array (make it outside a graph capture).
 * Calls on one GPU share the array, so calls that overlap in time on one GPU
 * (on different streams, or from different threads) race; calls in one
 * stream's order do not.  No part of the array needs to start at zero.
 * Errors: as tern_linear_bwd, plus SCRATCH when even the smallest plan needs
 *   more than 64 MiB (in / 256 * out * 4 bytes of sgrad partials, that is
 *   in * out above 4 Gi elements), HIP.
 */
int tern_linear_bwd_noalloc(const void *X, const void *dY, int32_t act_dtype,
                            const uint32_t *tern_packed, const float *scale,
                            int64_t T, int64_t in, int64_t out,
                            void *dX, int32_t dx_dtype, float *gq, float *sgrad, void *stream);

/*
 * Accumulating variants of the backward.  dX += adds one projection's input
 * gradient to a buffer that already holds others (an input feeding several
 * projections).  gq, sgrad += alpha * ... sums weight-side gradients over
 * micro-batches: the page's trainer averages the gradients of B > 1 sequences,
 * which alpha = 1/B expresses.
 *
 * tern_linear_bwd_dx_acc -- dX [T, in] (fp32, read and written) +=
 *   dY . W_eff^T, with the same arithmetic as tern_linear_bwd_dx; the sum is
 *   added to the old value in fp32.  Same argument rules; no workspace.  With
 *   T, in or out 0 nothing is added.
 *   Errors: NULL, SHAPE, DTYPE, ALIGN, ALIAS, HIP.
 *
 * tern_linear_bwd_acc_workspace_bytes -- device workspace (bytes) that
 *   tern_linear_bwd_dw_acc needs with either activation type (at least that
 *   of tern_linear_bwd: G always goes through the workspace here).  0 for
 *   invalid sizes.
 *
 * tern_linear_bwd_dw_acc -- with G = X^T . dY as in tern_linear_bwd:
 *   gq[r, c] += alpha * (G[r, c] * scale[c])   (fp32, read and written),
 *   sgrad[c] += alpha * sum_r G[r, c] * tern[r, c]   (the sum in the same
 *   fixed order, added to the old value in f64, then rounded to fp32).
 *   workspace: at least tern_linear_bwd_acc_workspace_bytes(...) bytes.
 *   alpha: any float (1 adds, 1/B averages B micro-batches).  With T = 0
 *   nothing is added.
 *   Errors: NULL, SHAPE, DTYPE, ALIGN, WORKSPACE, ALIAS, HIP.
 */
int tern_linear_bwd_dx_acc(const void *dY, int32_t act_dtype, const uint32_t *tern_packed,
                           const float *scale, int64_t T, int64_t in, int64_t out,
                           float *dX, void *stream);
size_t tern_linear_bwd_acc_workspace_bytes(int64_t T, int64_t in, int64_t out);
int tern_linear_bwd_dw_acc(const void *X, const void *dY, int32_t act_dtype,
                           const uint32_t *tern_packed, const float *scale,
                           int64_t T, int64_t in, int64_t out, float alpha,
                           float *gq, float *sgrad, void *workspace, size_t workspace_bytes,
                           void *stream);

/*
 * tern_scale_adamw -- the step of the per-column scale that follows its
 * gradient (page "train_gpu.cu": the trainer multiplies sgrad by
 * scale_lr / lr, then runs its AdamW launcher on the scale with the step's
 * bias corrections bc1 = 1 - b1^step, bc2 = 1 - b2^step; its hyper-parameters
 * are b1 0.9, b2 0.999, eps 1e-8, weight decay 0).  The update kernel's body
 * is not on the page; this is textbook AdamW with decoupled weight decay, in
 * fp32, per column c < out:
 *   g = sgrad[c] * (scale_lr / lr)
 *   m[c] = b1 m[c] + (1 - b1) g;   v[c] = b2 v[c] + (1 - b2) g^2
 *   scale[c] -= lr ((m[c] / bc1) / (sqrt(v[c] / bc2) + eps) + wd scale[c])
 * sgrad [out] is read; scale, m, v [out] (fp32, device, 4-byte aligned) are
 * updated in place; m = v = 0 before the first step (step = 1).
 * Errors: NULL, SHAPE (out < 0 or too large), VALUE (step < 1, lr or
 *   scale_lr not positive and finite), ALIGN, ALIAS, HIP.
 */
int tern_scale_adamw(const float *sgrad, float *scale, float *m, float *v, int64_t out,
                     int32_t step, float lr, float scale_lr, float b1, float b2, float eps,
                     float wd, void *stream);

/*
 * Projections that read one input.  nvg_train.rs (lin_fwd_shared) runs up to
 * four linears that read the same x off one staging pass of x, and the
 * trainer's attention projections read one input.  Here such a group is one
 * projection over the concatenated columns, W_group = [W_1 | W_2 | ...] of
 * [in, out_1 + ... + out_n]: one materialize, one forward (Y_group [T, sum out]
 * holds each Y_i as a column slice), one backward whose dX is the sum of the
 * projections' input gradients, and gq / sgrad as column slices.  Each
 * output column keeps its own summation order, so a Y_i slice equals the Y of
 * projection i alone bit for bit.
 *
 * tern_group_gather -- q_group[r, off_i + c] = q[i][r, c] and
 *   scale_group[off_i + c] = scale[i][c], with off_i = out[0] + ... +
 *   out[i-1].  q, scale, out: host arrays of n entries (1 <= n <= 8) holding
 *   device pointers to row-major int8 [in, out[i]] and fp32 [out[i]].
 *   q_group: device int8 [in, sum out]; scale_group: device fp32 [sum out].
 *   Then tern_materialize(q_group, in, sum out, ...) builds the group's
 *   handle.  Errors: NULL, SHAPE (n outside [1, 8], a negative size or a
 *   total above the limits), ALIAS (an output overlapping an input or the
 *   other output), HIP.
 */
int tern_group_gather(const int8_t *const *q, const float *const *scale, const int64_t *out,
                      int32_t n, int64_t in, int8_t *q_group, float *scale_group, void *stream);

/*
 * SR4 health panel (page "train_gpu.cu": the sr4_panel struct and
 * sr4_panel_compute, which the trainer runs on the host after a step).  Here
 * the counts are taken on the device into a caller-owned accumulator, one
 * ternary matrix per tern_panel_add call:
 *   total        elements counted;
 *   neg, zero, pos  elements whose ternary value (threshold rule with theta)
 *                is -1, 0, +1;
 *   rail         elements with |q| == q_clamp (the page's SR4_Q_CLAMP, 7);
 *   dead         elements with |q| < theta (equal to zero by definition);
 *   churn        elements whose ternary value differs from the one in
 *                prev_packed (the previous step's handle), over churn_total
 *                elements compared (calls with prev_packed NULL add none);
 *   scale_count, scale_sum, scale_min, scale_max  over the scale columns.
 * The page's fractions of these counts come from tern_panel_fractions.
 * Integer counts are exact; the scale sum is a fixed-order f64 sum per call,
 * so repeated runs give identical panels.
 *
 * tern_panel_reset -- zero the accumulator (min +inf, max -inf).
 * tern_panel_add -- add one matrix: q int8 [in, out], scale fp32 [out],
 *   prev_packed a handle of tern_materialize for the same in, out (its
 *   canonical part is read) or NULL.  theta in [1, 127], q_clamp in
 *   [0, 128].  panel is device memory, 8-byte aligned, written in stream
 *   order (calls on one stream accumulate; calls on different streams must
 *   not overlap on one panel: the class counts are added atomically, but
 *   total, the derived zero / dead and the scale statistics are updated by
 *   one thread at the end of each call).
 * Errors: NULL, SHAPE, THETA (theta or q_clamp out of range), ALIGN, ALIAS,
 *   HIP.
 */
typedef struct tern_panel {
    uint64_t total, neg, zero, pos, rail, dead;
    uint64_t churn, churn_total;
    uint64_t scale_count;
    double scale_sum, scale_min, scale_max;
} tern_panel_t;
int tern_panel_reset(tern_panel_t *panel, void *stream);
int tern_panel_add(const int8_t *q, int64_t in, int64_t out, int32_t theta, int32_t q_clamp,
                   const uint32_t *prev_packed, const float *scale, tern_panel_t *panel,
                   void *stream);

/*
 * tern_panel_fractions -- the page's panel fractions (sr4_panel_compute's
 * pct_neg, pct_zero, pct_pos, rail_pct, dead_pct, churn, and the scale mean)
 * of an accumulator.  A HOST function: panel is a host copy of the device
 * accumulator (copied after the adds have completed), out a host struct.
 *   pct_neg, pct_zero, pct_pos, rail, dead = the count / total (0 when total
 *   is 0); churn = churn / total when every counted element was compared
 *   with a previous handle (churn_total == total > 0), else 0, as the page
 *   reports churn only when a previous snapshot exists; scale_mean =
 *   scale_sum / scale_count (0 when no column was counted).
 * Errors: NULL.
 */
typedef struct tern_panel_fractions {
    double pct_neg, pct_zero, pct_pos, rail, dead, churn, scale_mean;
} tern_panel_fractions_t;
int tern_panel_fractions(const tern_panel_t *panel, tern_panel_fractions_t *out);

/*
 * The projections of one layer, one launch per product.  The page's trainer
 * launches every projection's kernels in turn (its own note: launch-bound).
 * Here the tiles of all projections of one product (and, for the weight
 * gradient, their splits over tokens) form one work list that a persistent
 * grid walks: small projections fill the chip together, and a layer step is
 * four launches (materialize, forward, dX, dW) plus the dW finish.  Each call
 * computes exactly what the single-projection call computes for every
 * projection (forward and dX bitwise alike; gq and sgrad to fp32 rounding,
 * since the split over tokens is planned for the layer).  Projections the
 * grouped kernels do not take (fp32 activations, in or out below 32 for the
 * forward / dX reduction, a dX whose scale is carried as two bf16 terms, in
 * or out below 256 for dW, empty sizes) run through the single-projection
 * path within the same call.
 *
 * tern_proj_t describes one projection: its sizes and the device buffers of
 * the calls that use them (members a call does not use may be NULL):
 *   in, out       sizes (multiples of 8); all projections share T;
 *   q             int8 [in, out]           (tern_layer_materialize)
 *   tern_packed   handle of tern_packed_words(in, out) words (written by
 *                 tern_layer_materialize, read by the other calls)
 *   scale         fp32 [out]
 *   X             [T, in]   act_dtype      (forward, dW)
 *   dY            [T, out]  act_dtype      (dX, dW)
 *   Y             [T, out]  y_dtype        (forward)
 *   dX            fp32 [T, in]             (dX)
 *   gq, sgrad     fp32 [in, out], [out]    (dW)
 * Inputs may be shared between projections (one X for several); no output
 * may overlap any input or any other output of the call (TERN_ERR_ALIAS).
 * n: 1 to 8 projections (TERN_ERR_SHAPE otherwise); the array is host
 * memory, read during the call only.
 */
typedef struct tern_proj {
    int64_t in, out;
    const int8_t *q;
    uint32_t *tern_packed;
    const float *scale;
    const void *X;
    const void *dY;
    void *Y;
    float *dX;
    float *gq;
    float *sgrad;
} tern_proj_t;

/* tern_layer_materialize -- tern_materialize of every projection (q ->
 * tern_packed), one launch.  Errors: NULL, SHAPE, THETA, ALIGN, ALIAS, HIP. */
int tern_layer_materialize(const tern_proj_t *projs, int32_t n, int32_t theta, void *stream);

/* tern_layer_fwd -- tern_linear_fwd of every projection (Y = X . W_eff).
 * Errors: NULL, SHAPE, DTYPE, ALIGN, ALIAS, HIP. */
int tern_layer_fwd(const tern_proj_t *projs, int32_t n, int64_t T, int32_t act_dtype, int32_t y_dtype,
                   void *stream);

/* tern_layer_bwd_dx -- tern_linear_bwd_dx of every projection (dX = dY .
 * W_eff^T, fp32).  Errors: NULL, SHAPE, DTYPE, ALIGN, ALIAS, HIP. */
int tern_layer_bwd_dx(const tern_proj_t *projs, int32_t n, int64_t T, int32_t act_dtype, void *stream);

/* tern_layer_bwd_dw_workspace_bytes -- workspace of tern_layer_bwd_dw for
 * these projections and T, with either activation type (0 for invalid
 * sizes; only in and out of each projection are read). */
size_t tern_layer_bwd_dw_workspace_bytes(const tern_proj_t *projs, int32_t n, int64_t T);

/* tern_layer_bwd_dw -- tern_linear_bwd_dw of every projection (gq, sgrad),
 * sgrad in the same fixed order per projection, bitwise repeatable.
 * workspace: at least tern_layer_bwd_dw_workspace_bytes(projs, n, T) bytes.
 * Errors: NULL, SHAPE, DTYPE, ALIGN, WORKSPACE, ALIAS, HIP. */
int tern_layer_bwd_dw(const tern_proj_t *projs, int32_t n, int64_t T, int32_t act_dtype, void *workspace,
                      size_t workspace_bytes, void *stream);

/*
 * Graphs of library calls.  The page's trainer launches every glue kernel and
 * GEMM of a step separately and notes that it is launch-bound; a caller can
 * instead record any sequence of the calls above (for example materialize,
 * forward and backward of all six projections of a layer) once and replay it
 * as one launch.
 *
 * tern_graph_begin -- start recording the work that this thread enqueues on
 *   `stream`, which must be a created stream (not NULL, the legacy default
 *   stream).  Until tern_graph_end, the entry points above validate their
 *   arguments as usual but only record their kernels: nothing runs.  The
 *   library records no memset, copy, allocation or synchronisation.
 * tern_graph_end -- stop recording on `stream` and instantiate the graph;
 *   *graph receives an opaque handle owned by the caller.  Buffers are
 *   recorded by address: each replay reads and writes the same device
 *   memory, with the contents it holds when the replay runs.  On failure
 *   *graph is NULL.
 * tern_graph_launch -- enqueue one replay on `stream` (any stream of the
 *   device the graph was recorded on), ordered like a kernel launch.
 * tern_graph_destroy -- release the handle (NULL is accepted); replays
 *   already enqueued complete normally.
 * The handle holds host-side graph objects, no device memory of its own.
 * Errors: NULL (stream, graph or handle missing), HIP (the runtime refused the
 *   capture, e.g. a stream that is already recording or a capture that a
 *   synchronising call invalidated, or the instantiation or launch).
 */
typedef struct tern_graph_s *tern_graph_t;
int tern_graph_begin(void *stream);
int tern_graph_end(void *stream, tern_graph_t *graph);
int tern_graph_launch(tern_graph_t graph, void *stream);
int tern_graph_destroy(tern_graph_t graph);

/* Human-readable name of a status code (static string, never NULL). */
const char *tern_status_str(int status);

/* Library version string (static). */
const char *tern_version(void);

#ifdef __cplusplus
}
#endif
#endif /* TERN_H */
