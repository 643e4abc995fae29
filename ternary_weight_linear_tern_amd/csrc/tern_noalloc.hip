// tern_noalloc.hip -- the backward of the ternary projection for callers that
// cannot allocate device memory (code under graph capture, tight serving
// loops, harnesses that forbid allocation): tern_linear_bwd_noalloc takes no
// workspace and keeps the backward's scratch (the sgrad partial table and the
// split-over-tokens partial products of the weight gradient) in a static
// device array of kNoallocScratchBytes instead.
//
// Each GPU the library runs on holds its own copy of the array until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it names a stand-in, not device memory): the array's device address is
// taken once per device with hipGetSymbolAddress, with that device current, on
// the entry point's first call there, and that address is what the kernels get.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/tern.h"
#include "tern_kernels.h"
#include "tern_plan.h"

namespace {

constexpr size_t kNoallocScratchBytes = size_t(64) << 20;   // 64 MiB per device
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) char scratch[kNoallocScratchBytes];

namespace {

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's copy of the array (looked up once per
// device, with the device current).
int scratch_of_current_device(void **ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TERN_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return TERN_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return TERN_OK;
}

}  // namespace

extern "C" int tern_linear_bwd_noalloc(const void *X, const void *dY, int32_t act_dtype,
                                       const uint32_t *tern_packed, const float *scale, int64_t T,
                                       int64_t in, int64_t out, void *dX, int32_t dx_dtype, float *gq,
                                       float *sgrad, void *stream) {
    using namespace tern;
    // the arguments, with the plan limited to the static array (fewer
    // splits of the weight-gradient product over tokens where needed)
    BwdLayout L;
    int rc = check_bwd(X, dY, act_dtype, tern_packed, scale, T, in, out, dX, dx_dtype, gq, sgrad, nullptr, 0,
                       true, true, false, L, kNoallocScratchBytes, false);
    if (rc) return rc;
    if (L.total > kNoallocScratchBytes) return TERN_ERR_SCRATCH;
    void *ws = nullptr;
    if (L.total > 0) {
        rc = scratch_of_current_device(&ws);
        if (rc) return rc;
        // no caller buffer can lie inside a library array, but check anyway
        const size_t es = act_dtype == TERN_BF16 ? 2 : 4;
        const void *bufs[] = {X, dY, tern_packed, scale, dX, gq, sgrad};
        const size_t sizes[] = {(size_t)T * in * es, (size_t)T * out * es,
                                (size_t)tern_packed_words(in, out) * 4, (size_t)out * 4, (size_t)T * in * 4,
                                (size_t)in * out * 4, (size_t)out * 4};
        for (int i = 0; i < 7; i++)
            if (ranges_overlap(ws, L.total, bufs[i], sizes[i])) return TERN_ERR_ALIAS;
    }
    const bool bf = act_dtype == TERN_BF16;
    hipStream_t st = (hipStream_t)stream;
    rc = enqueue_dx(dY, bf, tern_packed, scale, T, in, out, dX, L, st, false);
    if (rc == TERN_OK) rc = enqueue_dw(X, dY, bf, tern_packed, scale, T, in, out, gq, sgrad, ws, L, st, false, 1.0f);
    return rc;
}
