// tern_layer.cpp -- the projections of one layer (one token count T) with one
// launch per product: all materializes, all forwards, all input gradients,
// all weight gradients (declared in include/tern.h, tern_layer_*).
//
// The page's trainer runs every projection's kernels one after another and is
// launch-bound; here the work items of all projections of one product (output
// tiles: 512 x 128 for the forward and dX, 256 x 256 times the splits over
// tokens for dW) form one item space
// that a persistent grid walks, so small projections fill the chip together
// and pay one launch.  A projection that the grouped kernels do not take
// (fp32 activations, a reduction shorter than 32, a dX whose scale is carried
// as two bf16 terms, a dW side below 256, empty sizes) runs through the
// single-projection path inside the same call.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "../../include/tern.h"
#include "tern_kernels.h"
#include "tern_plan.h"

using namespace tern;

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }
size_t esize(int32_t dt) { return dt == TERN_BF16 ? 2 : 4; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
int hip_status(hipError_t e) { return e == hipSuccess ? TERN_OK : TERN_ERR_HIP; }
size_t al256(size_t x) { return (x + 255) & ~size_t(255); }

struct Span {
    const void *p;
    size_t n;
};

// Does any output span overlap another output span or an input span?
bool spans_alias(const Span *outs, int nout, const Span *ins, int nin) {
    for (int i = 0; i < nout; i++) {
        for (int j = i + 1; j < nout; j++)
            if (ranges_overlap(outs[i].p, outs[i].n, outs[j].p, outs[j].n)) return true;
        for (int j = 0; j < nin; j++)
            if (ranges_overlap(outs[i].p, outs[i].n, ins[j].p, ins[j].n)) return true;
    }
    return false;
}

// Common checks of a layer call: the count, the array, every projection's
// sizes.
int check_layer(const tern_proj_t *p, int32_t n, int64_t T) {
    if (n < 1 || n > kMaxGroup) return TERN_ERR_SHAPE;
    if (!p) return TERN_ERR_NULL;
    for (int i = 0; i < n; i++) {
        const int rc = validate_shape(T, p[i].in, p[i].out);
        if (rc) return rc;
    }
    return TERN_OK;
}

// Problem order of a group: longest reduction first, so that the longest
// items start in the first round of the persistent grid.
void order_by_k(int *idx, int m, const int64_t *k) {
    std::stable_sort(idx, idx + m, [&](int a, int b) { return k[a] > k[b]; });
}

// Fill ga.start from the problems' item counts; false if they do not fit.
bool finish_group(GroupArgs &ga) {
    int64_t total = 0;
    for (int i = 0; i < ga.n; i++) {
        ga.start[i] = (int)total;
        total += (int64_t)ga.p[i].tiles_m * ga.p[i].tiles_n * ga.p[i].splits;
        if (total > (int64_t(1) << 30)) return false;
    }
    ga.start[ga.n] = (int)total;
    return true;
}

// Workspace layout of the weight-gradient products of a layer: per
// projection, its sgrad partial table and (split over tokens) its partial
// products, each 256-byte aligned, projections one after another.
struct LayerDw {
    bool grouped[kMaxGroup];
    int64_t kps = 0, splits = 1;
    size_t part_off[kMaxGroup], ws_off[kMaxGroup];
    int64_t part_rows[kMaxGroup];
    BwdLayout single[kMaxGroup];
    size_t total = 0;
};

bool dw_groupable(const tern_proj_t &q, int64_t T, bool bf) {
    return bf && T > 0 && q.in >= 256 && q.out >= 256;
}

LayerDw plan_layer_dw(const tern_proj_t *p, int n, int64_t T, bool bf) {
    LayerDw L;
    int64_t tiles = 0, sum_io = 0;
    for (int i = 0; i < n; i++) {
        L.grouped[i] = dw_groupable(p[i], T, bf);
        if (L.grouped[i]) {
            tiles += cdiv(p[i].in, 256) * cdiv(p[i].out, 256);
            sum_io += p[i].in * p[i].out;
        }
    }
    if (tiles > 0) {
        L.kps = plan_layer_dw_splits(T, tiles, sum_io, bf);
        L.splits = cdiv(T, L.kps);
    }
    size_t off = 0;
    for (int i = 0; i < n; i++) {
        L.part_off[i] = L.ws_off[i] = off;
        L.part_rows[i] = 0;
        if (L.grouped[i]) {
            L.part_rows[i] = L.splits > 1 ? cdiv(p[i].in, kReduceRows) : cdiv(p[i].in, 256);
            const size_t pb = al256(size_t(L.part_rows[i]) * size_t(p[i].out) * 4);
            L.ws_off[i] = off + pb;
            off += pb + (L.splits > 1 ? al256(size_t(L.splits) * size_t(p[i].in) * size_t(p[i].out) * 4) : 0);
        } else {
            L.single[i] = plan_bwd(T, p[i].in, p[i].out, bf);
            off += al256(L.single[i].total);
        }
    }
    L.total = off;
    return L;
}

}  // namespace

extern "C" {

int tern_layer_materialize(const tern_proj_t *p, int32_t n, int32_t theta, void *stream) {
    if (n < 1 || n > kMaxGroup) return TERN_ERR_SHAPE;
    if (!p) return TERN_ERR_NULL;
    if (theta < 1 || theta > 127) return TERN_ERR_THETA;
    Span outs[kMaxGroup], ins[kMaxGroup];
    for (int i = 0; i < n; i++) {
        const tern_proj_t &q = p[i];
        if (q.in < 0 || q.out < 0 || q.in > kMaxInOut || q.out > kMaxInOut) return TERN_ERR_SHAPE;
        const size_t qb = (size_t)q.in * (size_t)q.out, pb = (size_t)tern_packed_words(q.in, q.out) * 4;
        if (qb && (!q.q || !q.tern_packed)) return TERN_ERR_NULL;
        if (qb && !aligned4(q.tern_packed)) return TERN_ERR_ALIGN;
        outs[i] = {q.tern_packed, qb ? pb : 0};
        ins[i] = {q.q, qb};
    }
    if (spans_alias(outs, n, ins, n)) return TERN_ERR_ALIAS;
    MatOneHost m[kMaxGroup];
    int k = 0;
    for (int i = 0; i < n; i++) {
        if ((size_t)p[i].in * (size_t)p[i].out == 0) continue;
        m[k++] = {p[i].q, p[i].tern_packed, p[i].in, p[i].out, p[i].out % 16 == 0 && aligned16(p[i].q)};
    }
    if (k == 0) return TERN_OK;
    return hip_status(launch_materialize_group(m, k, theta, (hipStream_t)stream));
}

int tern_layer_fwd(const tern_proj_t *p, int32_t n, int64_t T, int32_t act_dtype, int32_t y_dtype, void *stream) {
    int rc = check_layer(p, n, T);
    if (rc) return rc;
    if (act_dtype != TERN_F32 && act_dtype != TERN_BF16) return TERN_ERR_DTYPE;
    if (!(y_dtype == TERN_F32 || (y_dtype == TERN_BF16 && act_dtype == TERN_BF16))) return TERN_ERR_DTYPE;
    Span outs[kMaxGroup], ins[3 * kMaxGroup];
    for (int i = 0; i < n; i++) {
        const tern_proj_t &q = p[i];
        const size_t xb = (size_t)T * q.in * esize(act_dtype), yb = (size_t)T * q.out * esize(y_dtype);
        const size_t pb = (size_t)tern_packed_words(q.in, q.out) * 4, sb = (size_t)q.out * 4;
        if ((xb && !q.X) || (pb && !q.tern_packed) || (sb && !q.scale) || (yb && !q.Y)) return TERN_ERR_NULL;
        if ((xb && !aligned16(q.X)) || (sb && !aligned16(q.scale)) || (yb && !aligned16(q.Y)) ||
            (pb && !aligned4(q.tern_packed)))
            return TERN_ERR_ALIGN;
        outs[i] = {q.Y, yb};
        ins[3 * i] = {q.X, xb};
        ins[3 * i + 1] = {q.tern_packed, pb};
        ins[3 * i + 2] = {q.scale, sb};
    }
    if (spans_alias(outs, n, ins, 3 * n)) return TERN_ERR_ALIAS;
    hipStream_t st = (hipStream_t)stream;
    const bool bf = act_dtype == TERN_BF16;
    int idx[kMaxGroup], m = 0;
    int64_t kk[kMaxGroup];
    for (int i = 0; i < n; i++) {
        kk[i] = p[i].in;
        if (bf && T > 0 && p[i].out > 0 && p[i].in >= 32) idx[m++] = i;
    }
    order_by_k(idx, m, kk);
    GroupArgs ga{};
    ga.n = m;
    for (int j = 0; j < m; j++) {
        const tern_proj_t &q = p[idx[j]];
        GemmArgs &a = ga.p[j];
        a.act0 = q.X;
        a.packed = q.tern_packed;
        a.frag = q.tern_packed + packed_layout(q.in, q.out).fwd_off;
        a.scale = q.scale;
        a.out_ptr = q.Y;
        a.M = (int)q.out; a.N = (int)T; a.K = (int)q.in;
        a.splits = 1; a.kps = (int)q.in;
        a.in = (int)q.in; a.out = (int)q.out; a.wpr = (int)cdiv(q.out, 16); a.T = (int)T;
        a.y_bf16 = y_dtype == TERN_BF16;
        a.nch = (int)cdiv(q.in, kFragChunk);
    }
    if (m > 0) {
        if (!rd_items(ga)) return TERN_ERR_SHAPE;
        rc = hip_status(launch_gemm_group(MODE_FWD, ga, st));
        if (rc) return rc;
    }
    // the projections the grouped kernel does not take, one by one
    bool done[kMaxGroup] = {};
    for (int j = 0; j < m; j++) done[idx[j]] = true;
    for (int i = 0; i < n && rc == TERN_OK; i++)
        if (!done[i])
            rc = tern_linear_fwd(p[i].X, act_dtype, p[i].tern_packed, p[i].scale, T, p[i].in, p[i].out, p[i].Y,
                                 y_dtype, stream);
    return rc;
}

int tern_layer_bwd_dx(const tern_proj_t *p, int32_t n, int64_t T, int32_t act_dtype, void *stream) {
    int rc = check_layer(p, n, T);
    if (rc) return rc;
    if (act_dtype != TERN_F32 && act_dtype != TERN_BF16) return TERN_ERR_DTYPE;
    Span outs[kMaxGroup], ins[3 * kMaxGroup];
    for (int i = 0; i < n; i++) {
        const tern_proj_t &q = p[i];
        const size_t gb = (size_t)T * q.out * esize(act_dtype), db = (size_t)T * q.in * 4;
        const size_t pb = (size_t)tern_packed_words(q.in, q.out) * 4, sb = (size_t)q.out * 4;
        if ((gb && !q.dY) || (pb && !q.tern_packed) || (sb && !q.scale) || (db && !q.dX)) return TERN_ERR_NULL;
        if ((gb && !aligned16(q.dY)) || (sb && !aligned16(q.scale)) || (db && !aligned16(q.dX)) ||
            (pb && !aligned4(q.tern_packed)))
            return TERN_ERR_ALIGN;
        outs[i] = {q.dX, db};
        ins[3 * i] = {q.dY, gb};
        ins[3 * i + 1] = {q.tern_packed, pb};
        ins[3 * i + 2] = {q.scale, sb};
    }
    if (spans_alias(outs, n, ins, 3 * n)) return TERN_ERR_ALIAS;
    hipStream_t st = (hipStream_t)stream;
    const bool bf = act_dtype == TERN_BF16;
    int idx[kMaxGroup], m = 0;
    int64_t kk[kMaxGroup];
    for (int i = 0; i < n; i++) {
        kk[i] = p[i].out;
        if (bf && T > 0 && p[i].in > 0 && p[i].out >= 32 && !dx_exact_scale(T, p[i].in, p[i].out)) idx[m++] = i;
    }
    order_by_k(idx, m, kk);
    GroupArgs ga{};
    ga.n = m;
    for (int j = 0; j < m; j++) {
        const tern_proj_t &q = p[idx[j]];
        GemmArgs &a = ga.p[j];
        a.act0 = q.dY;
        a.packed = q.tern_packed;
        a.frag = q.tern_packed + packed_layout(q.in, q.out).dx_off;
        a.scale = q.scale;
        a.out_ptr = q.dX;
        a.M = (int)q.in; a.N = (int)T; a.K = (int)q.out;
        a.splits = 1; a.kps = (int)q.out;
        a.in = (int)q.in; a.out = (int)q.out; a.wpr = (int)cdiv(q.out, 16); a.T = (int)T;
        a.nch = (int)cdiv(q.out, kFragChunk);
    }
    if (m > 0) {
        if (!rd_items(ga)) return TERN_ERR_SHAPE;
        rc = hip_status(launch_gemm_group(MODE_DX, ga, st));
        if (rc) return rc;
    }
    bool done[kMaxGroup] = {};
    for (int j = 0; j < m; j++) done[idx[j]] = true;
    for (int i = 0; i < n && rc == TERN_OK; i++)
        if (!done[i])
            rc = tern_linear_bwd_dx(p[i].dY, act_dtype, p[i].tern_packed, p[i].scale, T, p[i].in, p[i].out, p[i].dX,
                                    TERN_F32, stream);
    return rc;
}

size_t tern_layer_bwd_dw_workspace_bytes(const tern_proj_t *p, int32_t n, int64_t T) {
    if (check_layer(p, n, T) != TERN_OK) return 0;
    // either activation type: the larger of the two layouts
    const size_t a = plan_layer_dw(p, n, T, true).total, b = plan_layer_dw(p, n, T, false).total;
    return a > b ? a : b;
}

int tern_layer_bwd_dw(const tern_proj_t *p, int32_t n, int64_t T, int32_t act_dtype, void *workspace,
                      size_t workspace_bytes, void *stream) {
    int rc = check_layer(p, n, T);
    if (rc) return rc;
    if (act_dtype != TERN_F32 && act_dtype != TERN_BF16) return TERN_ERR_DTYPE;
    const bool bf = act_dtype == TERN_BF16;
    const LayerDw L = plan_layer_dw(p, n, T, bf);
    Span outs[3 * kMaxGroup + 1], ins[4 * kMaxGroup];
    for (int i = 0; i < n; i++) {
        const tern_proj_t &q = p[i];
        const size_t es = esize(act_dtype);
        const size_t xb = (size_t)T * q.in * es, gb = (size_t)T * q.out * es;
        const size_t pb = (size_t)tern_packed_words(q.in, q.out) * 4, sb = (size_t)q.out * 4;
        const size_t qb = (size_t)q.in * q.out * 4;
        if ((xb && !q.X) || (gb && !q.dY) || (pb && !q.tern_packed) || (sb && !q.scale) || (qb && !q.gq) ||
            (sb && !q.sgrad))
            return TERN_ERR_NULL;
        if ((xb && !aligned16(q.X)) || (gb && !aligned16(q.dY)) || (sb && !aligned16(q.scale)) ||
            (qb && !aligned16(q.gq)) || (sb && !aligned16(q.sgrad)) || (pb && !aligned4(q.tern_packed)))
            return TERN_ERR_ALIGN;
        outs[2 * i] = {q.gq, qb};
        outs[2 * i + 1] = {q.sgrad, sb};
        ins[4 * i] = {q.X, xb};
        ins[4 * i + 1] = {q.dY, gb};
        ins[4 * i + 2] = {q.tern_packed, pb};
        ins[4 * i + 3] = {q.scale, sb};
    }
    if (L.total && !workspace) return TERN_ERR_WORKSPACE;
    if (workspace_bytes < L.total) return TERN_ERR_WORKSPACE;
    if (L.total && !aligned16(workspace)) return TERN_ERR_ALIGN;
    outs[2 * n] = {workspace, L.total};
    if (spans_alias(outs, 2 * n + 1, ins, 4 * n)) return TERN_ERR_ALIAS;
    hipStream_t st = (hipStream_t)stream;
    char *ws = (char *)workspace;
    int idx[kMaxGroup], m = 0;
    int64_t kk[kMaxGroup];
    for (int i = 0; i < n; i++) {
        kk[i] = p[i].in * p[i].out;   // same K (T) for all: larger products first
        if (L.grouped[i]) idx[m++] = i;
    }
    order_by_k(idx, m, kk);
    GroupArgs ga{};
    ga.n = m;
    DwFinishHost fin[kMaxGroup];
    for (int j = 0; j < m; j++) {
        const int i = idx[j];
        const tern_proj_t &q = p[i];
        GemmArgs &a = ga.p[j];
        float *part = (float *)(ws + L.part_off[i]);
        float *split_ws = (float *)(ws + L.ws_off[i]);
        a.act0 = q.X;
        a.act1 = q.dY;
        a.packed = q.tern_packed;
        a.frag = q.tern_packed + packed_layout(q.in, q.out).fwd_off;
        a.scale = q.scale;
        a.out_ptr = L.splits > 1 ? (void *)split_ws : (void *)q.gq;
        a.part = part;
        a.M = (int)q.in; a.N = (int)q.out; a.K = (int)T;
        a.tiles_m = (int)cdiv(q.in, 256); a.tiles_n = (int)cdiv(q.out, 256);
        a.splits = (int)L.splits; a.kps = (int)L.kps;
        a.in = (int)q.in; a.out = (int)q.out; a.wpr = (int)cdiv(q.out, 16); a.T = (int)T;
        GemmPlan pl;
        pl.mode = MODE_DW; pl.tile = TILE_256; pl.grid = 1; pl.splits = L.splits;
        rc = check_gemm_args(pl, a);
        if (rc) return rc;
        fin[j] = {split_ws, q.scale, q.tern_packed, q.gq, part, q.sgrad, q.in, q.out, L.splits, L.part_rows[i]};
    }
    if (m > 0) {
        if (!finish_group(ga)) return TERN_ERR_SHAPE;
        rc = hip_status(launch_gemm_group(MODE_DW, ga, st));
        if (rc == TERN_OK) rc = hip_status(launch_dw_finish_group(fin, m, st));
        if (rc) return rc;
    }
    for (int i = 0; i < n && rc == TERN_OK; i++)
        if (!L.grouped[i])
            rc = enqueue_dw(p[i].X, p[i].dY, bf, p[i].tern_packed, p[i].scale, T, p[i].in, p[i].out, p[i].gq,
                            p[i].sgrad, ws + L.part_off[i], L.single[i], st, false, 1.0f);
    return rc;
}

}  // extern "C"
