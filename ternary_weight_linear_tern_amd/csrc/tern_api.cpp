// tern_api.cpp -- the C ABI of libtern (declared in include/tern.h).
//
// Each entry point validates its arguments (HIP-free checks from tern_plan),
// plans the launches and enqueues them on the caller's stream.  Nothing here
// allocates device memory, synchronises or keeps state; the graph calls at the
// end hold host-side graph objects in a handle the caller owns.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <new>

#include "../../include/tern.h"
#include "tern_kernels.h"
#include "tern_plan.h"

using namespace tern;

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }
size_t esize(int32_t dt) { return dt == TERN_BF16 ? 2 : 4; }
bool act_ok(int32_t dt) { return dt == TERN_F32 || dt == TERN_BF16; }

int hip_status(hipError_t e) { return e == hipSuccess ? TERN_OK : TERN_ERR_HIP; }

struct Buf {
    const void *p;
    size_t n;
};

// Any output overlapping any other listed buffer?
bool any_alias(const Buf *outs, int nout, const Buf *ins, int nin) {
    for (int i = 0; i < nout; i++) {
        for (int j = i + 1; j < nout; j++)
            if (ranges_overlap(outs[i].p, outs[i].n, outs[j].p, outs[j].n)) return true;
        for (int j = 0; j < nin; j++)
            if (ranges_overlap(outs[i].p, outs[i].n, ins[j].p, ins[j].n)) return true;
    }
    return false;
}

}  // namespace

extern "C" {

const char *tern_version(void) { return "libtern 0.1 (gfx950)"; }

const char *tern_status_str(int status) {
    switch (status) {
        case TERN_OK: return "ok";
        case TERN_ERR_NULL: return "null pointer";
        case TERN_ERR_SHAPE: return "invalid shape (negative, in/out not a multiple of 8, or too large)";
        case TERN_ERR_THETA: return "theta outside [1, 127]";
        case TERN_ERR_DTYPE: return "unsupported element type";
        case TERN_ERR_ALIGN: return "pointer not 16-byte aligned";
        case TERN_ERR_WORKSPACE: return "workspace missing or too small";
        case TERN_ERR_ALIAS: return "output overlaps an input or another output";
        case TERN_ERR_HIP: return "HIP launch failed";
        case TERN_ERR_VALUE: return "scalar argument out of range (optimizer step or learning rate)";
        case TERN_ERR_SCRATCH: return "sizes need more than the library's static scratch (64 MiB)";
        default: return "unknown status";
    }
}

int64_t tern_packed_words(int64_t in, int64_t out) {
    if (in < 0 || out < 0) return -1;
    return packed_layout(in, out).total;
}

int tern_materialize(const int8_t *q, int64_t in, int64_t out, int32_t theta, uint32_t *tern_packed,
                     void *stream) {
    if (in < 0 || out < 0 || in > kMaxInOut || out > kMaxInOut) return TERN_ERR_SHAPE;
    if (theta < 1 || theta > 127) return TERN_ERR_THETA;
    if (in == 0 || out == 0) return TERN_OK;
    if (!q || !tern_packed) return TERN_ERR_NULL;
    if (!aligned4(tern_packed)) return TERN_ERR_ALIGN;
    const size_t qb = (size_t)in * (size_t)out;
    const size_t pb = (size_t)tern_packed_words(in, out) * 4;
    if (ranges_overlap(q, qb, tern_packed, pb)) return TERN_ERR_ALIAS;
    // the 16-byte vector path needs every row of q 16-byte aligned
    const bool vec = out % 16 == 0 && aligned16(q);
    return hip_status(launch_materialize(q, in, out, theta, vec, tern_packed, (hipStream_t)stream));
}

int tern_linear_fwd(const void *X, int32_t act_dtype, const uint32_t *tern_packed, const float *scale,
                    int64_t T, int64_t in, int64_t out, void *Y, int32_t y_dtype, void *stream) {
    int rc = validate_shape(T, in, out);
    if (rc) return rc;
    if (!act_ok(act_dtype)) return TERN_ERR_DTYPE;
    if (!(y_dtype == TERN_F32 || (y_dtype == TERN_BF16 && act_dtype == TERN_BF16))) return TERN_ERR_DTYPE;
    const size_t xb = (size_t)T * in * esize(act_dtype);
    const size_t yb = (size_t)T * out * esize(y_dtype);
    const size_t pb = (size_t)tern_packed_words(in, out) * 4;
    const size_t sb = (size_t)out * 4;
    if ((xb && !X) || (pb && !tern_packed) || (sb && !scale) || (yb && !Y)) return TERN_ERR_NULL;
    if ((xb && !aligned16(X)) || (sb && !aligned16(scale)) || (yb && !aligned16(Y)) ||
        (pb && !aligned4(tern_packed)))
        return TERN_ERR_ALIGN;
    const Buf outs[] = {{Y, yb}};
    const Buf ins[] = {{X, xb}, {tern_packed, pb}, {scale, sb}};
    if (any_alias(outs, 1, ins, 3)) return TERN_ERR_ALIAS;
    hipStream_t st = (hipStream_t)stream;
    if (yb == 0) return TERN_OK;
    if (in == 0) return hip_status(launch_zero(Y, yb, st));  // empty sum

    const bool bf = act_dtype == TERN_BF16;
    GemmPlan p = plan_gemm(MODE_FWD, T, in, out, bf);
    GemmArgs a{};
    a.act0 = X;
    a.packed = tern_packed;
    a.scale = scale;
    a.out_ptr = Y;
    a.M = (int)p.M; a.N = (int)p.N; a.K = (int)p.K;
    a.tiles_m = (int)p.tiles_m; a.tiles_n = (int)p.tiles_n;
    a.splits = (int)p.splits; a.kps = (int)p.k_per_split;
    a.in = (int)in; a.out = (int)out; a.wpr = (int)((out + 15) / 16); a.T = (int)T;
    a.y_bf16 = y_dtype == TERN_BF16;
    a.frag = tern_packed + packed_layout(in, out).fwd_off;
    a.nch = (int)((in + kFragChunk - 1) / kFragChunk);
    rc = check_gemm_args(p, a);
    if (rc) return rc;
    return hip_status(launch_gemm(p, bf, a, st));
}

size_t tern_linear_bwd_workspace_bytes(int64_t T, int64_t in, int64_t out) {
    return bwd_workspace_bytes(T, in, out, false);
}

}  // extern "C"

namespace tern {

int check_bwd(const void *X, const void *dY, int32_t act_dtype, const uint32_t *tern_packed,
              const float *scale, int64_t T, int64_t in, int64_t out, void *dX, int32_t dx_dtype,
              float *gq, float *sgrad, void *workspace, size_t workspace_bytes, bool want_dx,
              bool want_dw, bool acc, BwdLayout &L, size_t ws_limit, bool check_ws) {
    int rc = validate_shape(T, in, out);
    if (rc) return rc;
    if (!act_ok(act_dtype) || (want_dx && dx_dtype != TERN_F32)) return TERN_ERR_DTYPE;
    const bool bf = act_dtype == TERN_BF16;
    const size_t es = esize(act_dtype);
    const size_t xb = want_dw ? (size_t)T * in * es : 0, dyb = (size_t)T * out * es;
    const size_t pb = (size_t)tern_packed_words(in, out) * 4;
    const size_t sb = (size_t)out * 4;
    const size_t dxb = want_dx ? (size_t)T * in * 4 : 0;
    const size_t gqb = want_dw ? (size_t)in * out * 4 : 0, sgb = want_dw ? (size_t)out * 4 : 0;
    L = plan_bwd(T, in, out, bf, acc, ws_limit);
    const size_t wsb = want_dw && check_ws ? L.total : 0;
    if ((xb && !X) || (dyb && !dY) || (pb && !tern_packed) || (sb && !scale) || (dxb && !dX) ||
        (gqb && !gq) || (sgb && !sgrad))
        return TERN_ERR_NULL;
    if (wsb && !workspace) return TERN_ERR_WORKSPACE;
    if (workspace_bytes < wsb) return TERN_ERR_WORKSPACE;
    if ((xb && !aligned16(X)) || (dyb && !aligned16(dY)) || (sb && !aligned16(scale)) ||
        (dxb && !aligned16(dX)) || (gqb && !aligned16(gq)) || (sgb && !aligned16(sgrad)) ||
        (pb && !aligned4(tern_packed)) || (wsb && !aligned16(workspace)))
        return TERN_ERR_ALIGN;
    const Buf outs[] = {{dX, dxb}, {gq, gqb}, {sgrad, sgb}, {workspace, wsb}};
    const Buf ins[] = {{X, xb}, {dY, dyb}, {tern_packed, pb}, {scale, sb}};
    if (any_alias(outs, 4, ins, 4)) return TERN_ERR_ALIAS;
    return TERN_OK;
}

namespace {

GemmArgs args_for(const GemmPlan &p, const uint32_t *tern_packed, const float *scale, int64_t T,
                  int64_t in, int64_t out) {
    GemmArgs a{};
    a.packed = tern_packed;
    a.scale = scale;
    a.M = (int)p.M; a.N = (int)p.N; a.K = (int)p.K;
    a.tiles_m = (int)p.tiles_m; a.tiles_n = (int)p.tiles_n;
    a.splits = (int)p.splits; a.kps = (int)p.k_per_split;
    a.in = (int)in; a.out = (int)out; a.wpr = (int)((out + 15) / 16); a.T = (int)T;
    return a;
}

// host check, then the launch
int checked_launch(const GemmPlan &p, bool bf, const GemmArgs &a, hipStream_t st) {
    const int rc = check_gemm_args(p, a);
    if (rc) return rc;
    return hip_status(launch_gemm(p, bf, a, st));
}

}  // namespace

int enqueue_dx(const void *dY, bool bf, const uint32_t *tern_packed, const float *scale, int64_t T,
               int64_t in, int64_t out, void *dX, const BwdLayout &L, hipStream_t st, bool acc) {
    const size_t dxb = (size_t)T * in * 4;
    if (dxb == 0) return TERN_OK;
    if (out == 0) return acc ? TERN_OK : hip_status(launch_zero(dX, dxb, st));  // empty sum
    GemmArgs a = args_for(L.dx, tern_packed, scale, T, in, out);
    a.acc = acc;
    a.exact_scale = bf && dx_exact_scale(T, in, out);
    a.frag = tern_packed + packed_layout(in, out).dx_off;
    a.nch = (int)((out + kFragChunk - 1) / kFragChunk);
    a.act0 = dY;
    a.out_ptr = dX;
    return checked_launch(L.dx, bf, a, st);
}

int enqueue_dw(const void *X, const void *dY, bool bf, const uint32_t *tern_packed, const float *scale,
               int64_t T, int64_t in, int64_t out, float *gq, float *sgrad, void *workspace,
               const BwdLayout &L, hipStream_t st, bool acc, float alpha) {
    if (acc && (T == 0 || in == 0 || out == 0)) return TERN_OK;   // nothing to add
    if (T == 0 || in == 0 || out == 0) {
        // G is an empty sum (T == 0) or empty: gq = 0 and sgrad = 0 where they exist
        hipError_t e = hipSuccess;
        if ((size_t)in * out) e = launch_zero(gq, (size_t)in * out * 4, st);
        if (e == hipSuccess && out) e = launch_zero(sgrad, (size_t)out * 4, st);
        return hip_status(e);
    }
    if (!workspace) return TERN_ERR_WORKSPACE;   // the partial table (and split partials) live there
    float *part = (float *)((char *)workspace + L.part_off);
    GemmArgs a = args_for(L.dw, tern_packed, scale, T, in, out);
    a.frag = tern_packed + packed_layout(in, out).fwd_off;   // tern codes for the sgrad partials
    a.act0 = X;
    a.act1 = dY;
    a.part = part;
    a.acc = acc;
    int rc;
    if (L.dw.splits > 1 || acc) {
        float *ws = (float *)((char *)workspace + L.ws_off);
        a.out_ptr = ws;
        rc = checked_launch(L.dw, bf, a, st);
        if (rc == TERN_OK)
            rc = hip_status(
                launch_dw_reduce(ws, (int)L.dw.splits, scale, tern_packed, in, out, gq, part, acc, alpha, st));
    } else {
        a.out_ptr = gq;
        rc = checked_launch(L.dw, bf, a, st);
    }
    if (rc == TERN_OK) rc = hip_status(launch_sgrad_reduce(part, L.part_rows, out, sgrad, acc, alpha, st));
    return rc;
}

}  // namespace tern

extern "C" {

int tern_linear_bwd(const void *X, const void *dY, int32_t act_dtype, const uint32_t *tern_packed,
                    const float *scale, int64_t T, int64_t in, int64_t out, void *dX, int32_t dx_dtype,
                    float *gq, float *sgrad, void *workspace, size_t workspace_bytes, void *stream) {
    BwdLayout L;
    int rc = check_bwd(X, dY, act_dtype, tern_packed, scale, T, in, out, dX, dx_dtype, gq, sgrad,
                       workspace, workspace_bytes, true, true, false, L, ~size_t(0), true);
    if (rc) return rc;
    const bool bf = act_dtype == TERN_BF16;
    hipStream_t st = (hipStream_t)stream;
    rc = enqueue_dx(dY, bf, tern_packed, scale, T, in, out, dX, L, st, false);
    if (rc == TERN_OK)
        rc = enqueue_dw(X, dY, bf, tern_packed, scale, T, in, out, gq, sgrad, workspace, L, st, false, 1.0f);
    return rc;
}

int tern_linear_bwd_dx(const void *dY, int32_t act_dtype, const uint32_t *tern_packed, const float *scale,
                       int64_t T, int64_t in, int64_t out, void *dX, int32_t dx_dtype, void *stream) {
    BwdLayout L;
    int rc = check_bwd(nullptr, dY, act_dtype, tern_packed, scale, T, in, out, dX, dx_dtype, nullptr,
                       nullptr, nullptr, 0, true, false, false, L, ~size_t(0), true);
    if (rc) return rc;
    return enqueue_dx(dY, act_dtype == TERN_BF16, tern_packed, scale, T, in, out, dX, L, (hipStream_t)stream,
                      false);
}

int tern_linear_bwd_dw(const void *X, const void *dY, int32_t act_dtype, const uint32_t *tern_packed,
                       const float *scale, int64_t T, int64_t in, int64_t out, float *gq, float *sgrad,
                       void *workspace, size_t workspace_bytes, void *stream) {
    BwdLayout L;
    int rc = check_bwd(X, dY, act_dtype, tern_packed, scale, T, in, out, nullptr, TERN_F32, gq, sgrad,
                       workspace, workspace_bytes, false, true, false, L, ~size_t(0), true);
    if (rc) return rc;
    return enqueue_dw(X, dY, act_dtype == TERN_BF16, tern_packed, scale, T, in, out, gq, sgrad, workspace, L,
                      (hipStream_t)stream, false, 1.0f);
}

// ---- accumulating variants

size_t tern_linear_bwd_acc_workspace_bytes(int64_t T, int64_t in, int64_t out) {
    return bwd_workspace_bytes(T, in, out, true);
}

int tern_linear_bwd_dx_acc(const void *dY, int32_t act_dtype, const uint32_t *tern_packed, const float *scale,
                           int64_t T, int64_t in, int64_t out, float *dX, void *stream) {
    BwdLayout L;
    int rc = check_bwd(nullptr, dY, act_dtype, tern_packed, scale, T, in, out, dX, TERN_F32, nullptr, nullptr,
                       nullptr, 0, true, false, false, L, ~size_t(0), true);
    if (rc) return rc;
    return enqueue_dx(dY, act_dtype == TERN_BF16, tern_packed, scale, T, in, out, dX, L, (hipStream_t)stream,
                      true);
}

int tern_linear_bwd_dw_acc(const void *X, const void *dY, int32_t act_dtype, const uint32_t *tern_packed,
                           const float *scale, int64_t T, int64_t in, int64_t out, float alpha, float *gq,
                           float *sgrad, void *workspace, size_t workspace_bytes, void *stream) {
    BwdLayout L;
    int rc = check_bwd(X, dY, act_dtype, tern_packed, scale, T, in, out, nullptr, TERN_F32, gq, sgrad, workspace,
                       workspace_bytes, false, true, true, L, ~size_t(0), true);
    if (rc) return rc;
    return enqueue_dw(X, dY, act_dtype == TERN_BF16, tern_packed, scale, T, in, out, gq, sgrad, workspace, L,
                      (hipStream_t)stream, true, alpha);
}

// ---- the panel's fractions (host arithmetic on a host copy of the accumulator)

int tern_panel_fractions(const tern_panel_t *panel, tern_panel_fractions_t *out) {
    if (!panel || !out) return TERN_ERR_NULL;
    const double total = (double)panel->total;
    auto frac = [&](uint64_t n) { return panel->total ? (double)n / total : 0.0; };
    out->pct_neg = frac(panel->neg);
    out->pct_zero = frac(panel->zero);
    out->pct_pos = frac(panel->pos);
    out->rail = frac(panel->rail);
    out->dead = frac(panel->dead);
    // churn is a fraction only when every counted element had a previous code
    out->churn = (panel->total && panel->churn_total == panel->total) ? frac(panel->churn) : 0.0;
    out->scale_mean = panel->scale_count ? panel->scale_sum / (double)panel->scale_count : 0.0;
    return TERN_OK;
}

// ---- graphs of library calls: stream capture, instantiation, replay

struct tern_graph_s {
    hipGraph_t graph;
    hipGraphExec_t exec;
};

int tern_graph_begin(void *stream) {
    if (!stream) return TERN_ERR_NULL;
    // thread-local mode: calls of other threads are not recorded and cannot
    // invalidate this capture
    return hip_status(hipStreamBeginCapture((hipStream_t)stream, hipStreamCaptureModeThreadLocal));
}

int tern_graph_end(void *stream, tern_graph_t *graph) {
    if (!graph) return TERN_ERR_NULL;
    *graph = nullptr;
    if (!stream) return TERN_ERR_NULL;
    hipGraph_t g = nullptr;
    if (hipStreamEndCapture((hipStream_t)stream, &g) != hipSuccess || !g) {
        if (g) (void)hipGraphDestroy(g);
        return TERN_ERR_HIP;
    }
    hipGraphExec_t x = nullptr;
    if (hipGraphInstantiate(&x, g, nullptr, nullptr, 0) != hipSuccess) {
        (void)hipGraphDestroy(g);
        return TERN_ERR_HIP;
    }
    tern_graph_s *h = new (std::nothrow) tern_graph_s{g, x};
    if (!h) {
        (void)hipGraphExecDestroy(x);
        (void)hipGraphDestroy(g);
        return TERN_ERR_HIP;
    }
    *graph = h;
    return TERN_OK;
}

int tern_graph_launch(tern_graph_t graph, void *stream) {
    if (!graph) return TERN_ERR_NULL;
    return hip_status(hipGraphLaunch(graph->exec, (hipStream_t)stream));
}

int tern_graph_destroy(tern_graph_t graph) {
    if (!graph) return TERN_OK;
    const hipError_t e1 = hipGraphExecDestroy(graph->exec);
    const hipError_t e2 = hipGraphDestroy(graph->graph);
    delete graph;
    return e1 == hipSuccess && e2 == hipSuccess ? TERN_OK : TERN_ERR_HIP;
}

}  // extern "C"
