// tern_optim.hip -- the per-column scale step (C ABI in include/tern.h).
//
// The trainer on the page "train_gpu.cu" follows the scale gradient with
// sgrad *= scale_lr / lr and its AdamW launcher on the scale (bias
// corrections 1 - b1^t and 1 - b2^t formed on the host).  The update itself is
// textbook AdamW with decoupled weight decay: one thread per column, fp32.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "../../include/tern.h"
#include "tern_plan.h"

namespace tern {
namespace odev {

__global__ __launch_bounds__(256) void scale_adamw_kernel(const float *__restrict__ sgrad, float *__restrict__ scale,
                                                          float *__restrict__ m, float *__restrict__ v, int64_t out,
                                                          float k, float lr, float b1, float b2, float eps, float wd,
                                                          float bc1, float bc2) {
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= out) return;
    const float g = sgrad[c] * k;
    const float mm = b1 * m[c] + (1.0f - b1) * g;
    const float vv = b2 * v[c] + (1.0f - b2) * g * g;
    m[c] = mm;
    v[c] = vv;
    const float s = scale[c];
    scale[c] = s - lr * ((mm / bc1) / (sqrtf(vv / bc2) + eps) + wd * s);
}

}  // namespace odev
}  // namespace tern

using namespace tern;

extern "C" {

int tern_scale_adamw(const float *sgrad, float *scale, float *m, float *v, int64_t out, int32_t step, float lr,
                     float scale_lr, float b1, float b2, float eps, float wd, void *stream) {
    if (out < 0 || out > kMaxInOut) return TERN_ERR_SHAPE;
    if (step < 1 || !(lr > 0.0f) || !isfinite(lr) || !(scale_lr > 0.0f) || !isfinite(scale_lr))
        return TERN_ERR_VALUE;
    if (out == 0) return TERN_OK;
    if (!sgrad || !scale || !m || !v) return TERN_ERR_NULL;
    if (((uintptr_t)sgrad | (uintptr_t)scale | (uintptr_t)m | (uintptr_t)v) & 3u) return TERN_ERR_ALIGN;
    const size_t b = (size_t)out * 4;
    if (ranges_overlap(scale, b, m, b) || ranges_overlap(scale, b, v, b) || ranges_overlap(m, b, v, b) ||
        ranges_overlap(sgrad, b, scale, b) || ranges_overlap(sgrad, b, m, b) || ranges_overlap(sgrad, b, v, b))
        return TERN_ERR_ALIAS;
    // the page's host-side scalars: gradient factor and bias corrections in fp32
    const float k = scale_lr / lr;
    const float bc1 = 1.0f - powf(b1, (float)step), bc2 = 1.0f - powf(b2, (float)step);
    hipLaunchKernelGGL(odev::scale_adamw_kernel, dim3((unsigned)((out + 255) / 256)), dim3(256), 0,
                       (hipStream_t)stream, sgrad, scale, m, v, out, k, lr, b1, b2, eps, wd, bc1, bc2);
    return hipGetLastError() == hipSuccess ? TERN_OK : TERN_ERR_HIP;
}

}  // extern "C"
