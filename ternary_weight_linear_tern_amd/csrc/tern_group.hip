// tern_group.hip -- gather of projections that read one input into one
// projection over their concatenated columns (C ABI in include/tern.h).
//
// A group of linears with a shared input (nvg_train.rs, lin_fwd_shared; the
// trainer's attention projections) becomes W_group = [W_1 | W_2 | ...]: this
// kernel writes the group's q and scale from the members' buffers, and the
// single-projection entry points do the rest.  Each thread writes one 16-byte
// span of a q_group row (or the ragged end of one), finding each byte's member
// from the column offsets (one 16-byte copy when the widths allow it); a second
// grid dimension copies the scales.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tern.h"
#include "tern_plan.h"

namespace tern {
namespace gdev {

constexpr int kMaxGroup = 8;

struct GroupSrc {
    const int8_t *q[kMaxGroup];
    const float *scale[kMaxGroup];
    int64_t off[kMaxGroup + 1];   // column offsets; off[n] = total columns
    int n;
};

// VEC: every member's width is a multiple of 16 and every q is 16-byte
// aligned, so a 16-byte span of a q_group row lies in one member and moves
// with one load and one store.
template <bool VEC>
__global__ __launch_bounds__(256) void group_gather_kernel(GroupSrc s, int64_t in, int8_t *__restrict__ qg,
                                                           float *__restrict__ sg) {
    const int64_t total = s.off[s.n];
    if (blockIdx.y == 1) {   // scales
        for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < total; c += (int64_t)gridDim.x * 256) {
            int i = 0;
            while (i + 1 < s.n && c >= s.off[i + 1]) i++;
            sg[c] = s.scale[i][c - s.off[i]];
        }
        return;
    }
    const int64_t spans = (total + 15) / 16, n16 = in * spans;
    for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < n16; t += (int64_t)gridDim.x * 256) {
        const int64_t r = t / spans, c0 = (t - r * spans) * 16;
        int i = 0;
        while (i + 1 < s.n && c0 >= s.off[i + 1]) i++;
        int8_t *dst = qg + r * total + c0;
        if constexpr (VEC) {
            const int64_t w = s.off[i + 1] - s.off[i];
            *(uint4 *)dst = *(const uint4 *)(s.q[i] + r * w + (c0 - s.off[i]));
            continue;
        }
        for (int j = 0; j < 16 && c0 + j < total; j++) {
            const int64_t c = c0 + j;
            while (i + 1 < s.n && c >= s.off[i + 1]) i++;
            const int64_t w = s.off[i + 1] - s.off[i];
            dst[j] = s.q[i][r * w + (c - s.off[i])];
        }
    }
}

}  // namespace gdev
}  // namespace tern

using namespace tern;

extern "C" {

int tern_group_gather(const int8_t *const *q, const float *const *scale, const int64_t *out, int32_t n,
                      int64_t in, int8_t *q_group, float *scale_group, void *stream) {
    if (n < 1 || n > gdev::kMaxGroup || in < 0 || in > kMaxInOut) return TERN_ERR_SHAPE;
    if (!q || !scale || !out) return TERN_ERR_NULL;
    gdev::GroupSrc s{};
    s.n = n;
    s.off[0] = 0;
    for (int i = 0; i < n; i++) {
        if (out[i] < 0) return TERN_ERR_SHAPE;
        s.off[i + 1] = s.off[i] + out[i];
        if (s.off[i + 1] > kMaxInOut) return TERN_ERR_SHAPE;
        s.q[i] = q[i];
        s.scale[i] = scale[i];
        if ((in * out[i] && !q[i]) || (out[i] && !scale[i])) return TERN_ERR_NULL;
    }
    const int64_t total = s.off[n];
    const size_t qb = (size_t)in * (size_t)total, sb = (size_t)total * 4;
    if ((qb && !q_group) || (sb && !scale_group)) return TERN_ERR_NULL;
    if (ranges_overlap(q_group, qb, scale_group, sb)) return TERN_ERR_ALIAS;
    for (int i = 0; i < n; i++) {
        const size_t qi = (size_t)in * (size_t)out[i], si = (size_t)out[i] * 4;
        if (ranges_overlap(q_group, qb, q[i], qi) || ranges_overlap(q_group, qb, scale[i], si) ||
            ranges_overlap(scale_group, sb, q[i], qi) || ranges_overlap(scale_group, sb, scale[i], si))
            return TERN_ERR_ALIAS;
    }
    if (total == 0) return TERN_OK;
    const int64_t n16 = in * ((total + 15) / 16);
    int64_t blocks = (n16 > total ? n16 : total) / 256 + 1;
    if (blocks > 4096) blocks = 4096;
    bool vec = ((uintptr_t)q_group & 15u) == 0;
    for (int i = 0; i < n; i++) vec = vec && out[i] % 16 == 0 && ((uintptr_t)q[i] & 15u) == 0;
    if (vec)
        hipLaunchKernelGGL(gdev::group_gather_kernel<true>, dim3((unsigned)blocks, 2), dim3(256), 0,
                           (hipStream_t)stream, s, in, q_group, scale_group);
    else
        hipLaunchKernelGGL(gdev::group_gather_kernel<false>, dim3((unsigned)blocks, 2), dim3(256), 0,
                           (hipStream_t)stream, s, in, q_group, scale_group);
    return hipGetLastError() == hipSuccess ? TERN_OK : TERN_ERR_HIP;
}

}  // extern "C"
