// tern_kernels.h -- internal launchers of the gfx950 kernels (not part of the
// C ABI; tern_api.cpp is the only caller).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>

#include "tern_plan.h"

namespace tern {

// Kernel arguments of the three MFMA GEMMs (see tern_plan.h for M, N, K).
struct GemmArgs {
    const void *act0;        // FWD: X, DX: dY, DW: X
    const void *act1;        // DW: dY
    const uint32_t *packed;  // tern, 2-bit packed [in][wpr]
    const uint32_t *frag;    // FWD / DX: this product's fragment-ordered copy of tern
    const float *scale;      // [out]
    void *out_ptr;           // FWD: Y, DX: dX, DW: gq (1 split) or split partials
    float *part;             // DW with 1 split: sgrad partials [tiles_m][out]
    int M, N, K;
    int tiles_m, tiles_n, splits, kps;
    int in, out, wpr, T;
    int y_bf16;
    int nch;                 // FWD / DX: chunks of 32 K per tile in the fragment copy
    int acc;                 // DX: add to the existing dX; DW: raw G into out_ptr even with one split
};

hipError_t launch_gemm(const GemmPlan &p, bool bf16, const GemmArgs &a, hipStream_t st);
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

}  // namespace tern
