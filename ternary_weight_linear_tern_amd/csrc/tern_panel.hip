// tern_panel.hip -- the SR4 health panel on gfx950 (C ABI in include/tern.h).
//
// The page "train_gpu.cu" (sr4_panel, sr4_panel_compute) copies q and scale
// to the host after a step and counts there: the ternary class of every
// element under the threshold rule, rail (|q| at the clamp), dead (|q| below
// theta), churn against the previous classification, and the scale's mean,
// minimum and maximum.  Here one kernel counts a matrix on the device, one
// thread per 16 elements of a row (the span of one packed word), so the
// classes and the churn against the previous handle's canonical word are
// popcounts of 2-bit codes; block sums go to the accumulator with integer
// atomics, which are exact in any order.  A one-block kernel adds the scale
// statistics in a fixed order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tern.h"
#include "tern_plan.h"

namespace tern {
namespace pdev {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ void panel_reset_kernel(tern_panel_t *p) {
    if (threadIdx.x == 0 && blockIdx.x == 0) {
        p->total = p->neg = p->zero = p->pos = p->rail = p->dead = 0;
        p->churn = p->churn_total = p->scale_count = 0;
        p->scale_sum = 0.0;
        p->scale_min = __builtin_inf();
        p->scale_max = -__builtin_inf();
    }
}

// Sum of v over the block (PANEL_NT threads), valid in every thread: lanes
// within each wave, then the waves' sums in ascending order.
constexpr int PANEL_NT = 1024;
__device__ __forceinline__ uint64_t block_sum(uint64_t v, uint64_t *red) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    uint64_t s = 0;
#pragma unroll
    for (int w = 0; w < PANEL_NT / 64; w++) s += red[w];
    return s;
}

// Counts of one matrix that need its elements: nonzero +1 and -1 codes, rail
// (|q| == clamp) and churn against the previous handle's canonical words.
// total, zero (= dead) and churn_total follow from in * out and these, and
// panel_scale_kernel adds them once the counts are in.  Every block adds its
// sums with a few integer atomics, exact in any order.
template <bool VEC>
__global__ __launch_bounds__(PANEL_NT) void panel_count_kernel(const int8_t *__restrict__ q, int64_t out,
                                                               int64_t wpr, int64_t nwords, int theta, int clamp,
                                                               const uint32_t *__restrict__ prev,
                                                               tern_panel_t *__restrict__ p) {
    __shared__ uint64_t red[PANEL_NT / 64];
    uint32_t neg = 0, pos = 0, rail = 0, churn = 0;
    // word index -> (row, word column): a 32-bit division when the indices fit
    // (a 64-bit one is a long software sequence)
    const bool narrow = nwords <= 0xFFFFFFFFll;
#pragma unroll 4
    for (int64_t i = (int64_t)blockIdx.x * PANEL_NT + threadIdx.x; i < nwords; i += (int64_t)gridDim.x * PANEL_NT) {
        const int64_t r = narrow ? (int64_t)((uint32_t)i / (uint32_t)wpr) : i / wpr, wc = i - r * wpr;
        const int8_t *row = q + r * out + wc * 16;
        const int nc = out - wc * 16 < 16 ? (int)(out - wc * 16) : 16;
        int8_t b[16];
        if constexpr (VEC) {
            const u32x4 v = *(const u32x4 *)row;
#pragma unroll
            for (int j = 0; j < 16; j++) b[j] = (int8_t)((v[j >> 2] >> (8 * (j & 3))) & 0xFFu);
        } else {
#pragma unroll
            for (int j = 0; j < 16; j++) b[j] = j < nc ? row[j] : (int8_t)0;
        }
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < 16; j++) {
            // elements past a ragged row end are 0 here: code 00 (theta >= 1),
            // and left out of the rail count (a clamp of 0 would match them)
            const int v = b[j];
            const uint32_t code = v >= theta ? 1u : (v <= -theta ? 3u : 0u);
            word |= code << (2 * j);
            rail += (v == clamp || v == -clamp) && j < nc;
        }
        // code 01 = +1, 11 = -1 (bit 0: nonzero, bit 1: negative)
        pos += (uint32_t)__builtin_popcount(word & ~(word >> 1) & 0x55555555u);
        neg += (uint32_t)__builtin_popcount(word & (word >> 1) & 0x55555555u);
        if (prev) {
            const uint32_t d = word ^ prev[i];   // padding codes are 00 in both
            churn += (uint32_t)__builtin_popcount((d | (d >> 1)) & 0x55555555u);
        }
    }
    const uint64_t s_neg = block_sum(neg, red);
    const uint64_t s_pos = block_sum(pos, red);
    const uint64_t s_rail = block_sum(rail, red);
    const uint64_t s_churn = prev ? block_sum(churn, red) : 0;
    if (threadIdx.x == 0) {
        if (s_neg) atomicAdd((unsigned long long *)&p->neg, (unsigned long long)s_neg);
        if (s_pos) atomicAdd((unsigned long long *)&p->pos, (unsigned long long)s_pos);
        if (s_rail) atomicAdd((unsigned long long *)&p->rail, (unsigned long long)s_rail);
        if (s_churn) atomicAdd((unsigned long long *)&p->churn, (unsigned long long)s_churn);
    }
}

// One block: thread t sums columns t, t + 256, ... in f64 (ascending), then a
// fixed tree over the threads; thread 0 adds the result to the accumulator.
__global__ __launch_bounds__(256) void panel_scale_kernel(const float *__restrict__ scale, int64_t out,
                                                          int64_t elems, int compared,
                                                          tern_panel_t *__restrict__ p) {
    __shared__ double ssum[256];
    __shared__ float smin[256], smax[256];
    const int t = threadIdx.x;
    double s = 0.0;
    float mn = __builtin_inff(), mx = -__builtin_inff();
    for (int64_t c = t; c < out; c += 256) {
        const float v = scale[c];
        s += (double)v;
        mn = v < mn ? v : mn;
        mx = v > mx ? v : mx;
    }
    ssum[t] = s;
    smin[t] = mn;
    smax[t] = mx;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
        if (t < h) {
            ssum[t] += ssum[t + h];
            smin[t] = smin[t + h] < smin[t] ? smin[t + h] : smin[t];
            smax[t] = smax[t + h] > smax[t] ? smax[t + h] : smax[t];
        }
        __syncthreads();
    }
    if (t == 0) {
        // the matrix's element count, and the classes that follow from it
        // (the counts of this matrix are in: same stream, earlier kernel)
        p->total += (uint64_t)elems;
        if (compared) p->churn_total += (uint64_t)elems;
        p->zero = p->total - p->neg - p->pos;
        p->dead = p->zero;   // |q| < theta is exactly the zero class
        p->scale_count += (uint64_t)out;
        p->scale_sum += ssum[0];
        if ((double)smin[0] < p->scale_min) p->scale_min = (double)smin[0];
        if ((double)smax[0] > p->scale_max) p->scale_max = (double)smax[0];
    }
}

}  // namespace pdev
}  // namespace tern

using namespace tern;

extern "C" {

int tern_panel_reset(tern_panel_t *panel, void *stream) {
    if (!panel) return TERN_ERR_NULL;
    if (((uintptr_t)panel & 7u) != 0) return TERN_ERR_ALIGN;
    hipLaunchKernelGGL(pdev::panel_reset_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, panel);
    return hipGetLastError() == hipSuccess ? TERN_OK : TERN_ERR_HIP;
}

int tern_panel_add(const int8_t *q, int64_t in, int64_t out, int32_t theta, int32_t q_clamp,
                   const uint32_t *prev_packed, const float *scale, tern_panel_t *panel, void *stream) {
    if (in < 0 || out < 0 || in > kMaxInOut || out > kMaxInOut) return TERN_ERR_SHAPE;
    if (theta < 1 || theta > 127 || q_clamp < 0 || q_clamp > 128) return TERN_ERR_THETA;
    const size_t qb = (size_t)in * (size_t)out, sb = (size_t)out * 4, pb = sizeof(tern_panel_t);
    const size_t hb = prev_packed ? (size_t)in * (size_t)((out + 15) / 16) * 4 : 0;
    if (!panel || (qb && !q) || (sb && !scale)) return TERN_ERR_NULL;
    if (((uintptr_t)panel & 7u) != 0 || ((uintptr_t)scale & 3u) != 0 || ((uintptr_t)prev_packed & 3u) != 0)
        return TERN_ERR_ALIGN;
    if (ranges_overlap(panel, pb, q, qb) || ranges_overlap(panel, pb, scale, sb) ||
        ranges_overlap(panel, pb, prev_packed, hb))
        return TERN_ERR_ALIAS;
    hipStream_t st = (hipStream_t)stream;
    const int64_t wpr = (out + 15) / 16, nwords = in * wpr;
    if (nwords > 0) {
        // every block adds its sums to the same 64-bit fields, and those
        // atomics serialise at one L2 channel (about 8 ns each): 128 blocks
        // of 1024 threads (two waves per SIMD), each streaming many words
        int64_t blocks = (nwords + pdev::PANEL_NT - 1) / pdev::PANEL_NT;
        if (blocks > 128) blocks = 128;
        const bool vec = out % 16 == 0 && ((uintptr_t)q & 15u) == 0;
        if (vec)
            hipLaunchKernelGGL(pdev::panel_count_kernel<true>, dim3((unsigned)blocks), dim3(pdev::PANEL_NT), 0, st,
                               q, out, wpr, nwords, (int)theta, (int)q_clamp, prev_packed, panel);
        else
            hipLaunchKernelGGL(pdev::panel_count_kernel<false>, dim3((unsigned)blocks), dim3(pdev::PANEL_NT), 0, st,
                               q, out, wpr, nwords, (int)theta, (int)q_clamp, prev_packed, panel);
        if (hipGetLastError() != hipSuccess) return TERN_ERR_HIP;
    }
    if (out > 0) {
        hipLaunchKernelGGL(pdev::panel_scale_kernel, dim3(1), dim3(256), 0, st, scale, out, in * out,
                           prev_packed ? 1 : 0, panel);
        if (hipGetLastError() != hipSuccess) return TERN_ERR_HIP;
    }
    return TERN_OK;
}

}  // extern "C"
