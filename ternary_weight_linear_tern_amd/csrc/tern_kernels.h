// tern_kernels.h -- internal launchers of the gfx950 kernels (not part of the
// C ABI; tern_api.cpp is the only caller).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>

#include "tern_plan.h"

namespace tern {

hipError_t launch_gemm(const GemmPlan &p, bool bf16, const GemmArgs &a, hipStream_t st);
// One persistent launch over the items of several problems of one mode (bf16
// activations; forward / dX on 512 x 128 tiles, the accumulating dX and dW on
// 256 x 256 tiles, whatever tiles_m / tiles_n the problems carry; each
// problem's arguments complete and checked, forward / dX with K >= 32, dW with
// M, N >= 256).
hipError_t launch_gemm_group(int mode, const GroupArgs &ga, hipStream_t st);
// The whole packed handle (canonical words, padding, both fragment-ordered
// copies; see PackedLayout) from q in one launch.
hipError_t launch_materialize(const int8_t *q, int64_t in, int64_t out, int theta, bool vec,
                              uint32_t *packed, hipStream_t st);
// acc: gq += alpha * G * scale instead of gq = G * scale
hipError_t launch_dw_reduce(const float *ws, int splits, const float *scale, const uint32_t *packed,
                            int64_t in, int64_t out, float *gq, float *part, bool acc, float alpha,
                            hipStream_t st);
// acc: sgrad += alpha * (sum of the partials) instead of sgrad = the sum
hipError_t launch_sgrad_reduce(const float *part, int64_t nparts, int64_t out, float *sgrad, bool acc, float alpha,
                               hipStream_t st);
hipError_t launch_zero(void *p, size_t bytes, hipStream_t st);

// Several handles in one launch (n <= kMaxGroup matrices; vec: the 16-byte
// path, which needs out % 16 == 0 and q 16-byte aligned).
struct MatOneHost {
    const int8_t *q;
    uint32_t *packed;
    int64_t in, out;
    bool vec;
};
hipError_t launch_materialize_group(const MatOneHost *m, int n, int theta, hipStream_t st);

// The dW finish of several projections in two launches: the split-K reduce of
// those with splits > 1 (gq = G * scale and the 4-row sgrad partials), then
// the fixed-order sgrad sum of all (nparts rows of partials each).
struct DwFinishHost {
    const float *ws;
    const float *scale;
    const uint32_t *packed;
    float *gq, *part, *sgrad;
    int64_t in, out, splits, nparts;
};
hipError_t launch_dw_finish_group(const DwFinishHost *f, int n, hipStream_t st);

// Backward pieces shared by the entry points (tern_api.cpp, tern_noalloc.hip).
// check_bwd validates the arguments of a backward call (want_dx / want_dw
// select the parts) and plans it with a workspace of at most ws_limit bytes;
// check_ws false leaves the workspace pointer and size out of the checks (the
// caller supplies the workspace itself).  The enqueue functions return a
// TERN_* status.
int check_bwd(const void *X, const void *dY, int32_t act_dtype, const uint32_t *tern_packed,
              const float *scale, int64_t T, int64_t in, int64_t out, void *dX, int32_t dx_dtype,
              float *gq, float *sgrad, void *workspace, size_t workspace_bytes, bool want_dx,
              bool want_dw, bool acc, BwdLayout &L, size_t ws_limit, bool check_ws);
int enqueue_dx(const void *dY, bool bf, const uint32_t *tern_packed, const float *scale, int64_t T,
               int64_t in, int64_t out, void *dX, const BwdLayout &L, hipStream_t st, bool acc);
// acc: gq += alpha * G * scale and sgrad += alpha * sum_r G * tern; G then
// always goes through the workspace (L planned with acc).
int enqueue_dw(const void *X, const void *dY, bool bf, const uint32_t *tern_packed, const float *scale,
               int64_t T, int64_t in, int64_t out, float *gq, float *sgrad, void *workspace,
               const BwdLayout &L, hipStream_t st, bool acc, float alpha);

}  // namespace tern
