// tern_kernels.hip -- gfx950 (MI355X) kernels of the SR4 ternary projection.
//
// The method (page "train_gpu.cu", "device glue kernels" section and the
// optimizer-split header comment): tern = sign(q) outside the dead zone
// |q| < theta (tg_tern_from_q), W_eff[r, c] = scale[c] * tern[r, c]
// (tg_apply_scale, rows = input dim), Y = X . W_eff, dX = dY . W_eff^T,
// G = X^T . dY, gq = G * scale[c] (tg_gq), sgrad[c] = sum_r G[r, c] tern[r, c]
// (tg_scale_grad).
//
// Design on CDNA4 (not a translation of the page's K80 kernels, which
// materialise W_eff in fp32 and call cuBLAS):
//   * tern is stored 2-bit packed (16 codes per u32) and is never expanded in
//     HBM.  The GEMMs read the packed words, decode them in registers and stage
//     the bf16 (or fp32) operand tile in LDS.
//   * Forward: the scale multiplies the fp32 column sums in the epilogue.
//     dX: the scale sits on the reduction index, so it is folded into the
//     decoded operand as +-bf16(scale[c]) (fp32 path: exact +-scale[c]).
//     dW: the epilogue writes gq = G * scale[c] and reduces G * tern over the
//     tile's rows in a fixed order into per-row-tile partials; a second kernel
//     sums the partials in ascending row-tile order (deterministic sgrad).
//   * One GEMM template: 256 threads = 4 wave64s in 2 x 2, each wave owning a
//     (BM/2) x (BN/2) block of 32x32 MFMA tiles (v_mfma_f32_32x32x16_bf16, or
//     v_mfma_f32_32x32x2_f32 for fp32).  Operands are staged through
//     double-buffered LDS tiles whose rows are 128 bytes of K plus 16 bytes of
//     padding (conflict-free 16-byte reads for the MFMA fragments).  Global
//     reads use buffer loads whose out-of-range lanes return zero, which handles
//     ragged M, N and K edges without branches in the loads.
//   * The workgroup -> tile map sends consecutive tiles to the same XCD (the
//     hardware deals workgroups round-robin over the 8 XCDs) and walks tiles in
//     groups of 8 along M, so tiles resident on one XCD share operand panels in
//     that XCD's L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tern_kernels.h"

namespace tern {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int NT = 256;               // threads per workgroup
constexpr int RC = 9;                 // 16-byte chunks per LDS row: 8 of K data + 1 pad
constexpr uint32_t OOB = 0x80000000u;  // buffer offset that is always out of range

// Buffer resource over [p, p + 2 GiB): offsets >= 0x7FFFFFFF read as zero.
// Word 3 selects the 32-bit data format required by untyped buffer loads.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, 0x7FFFFFFF, 0x00020000);
}
__device__ __forceinline__ u32x4 bload128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t bload32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

// 2-bit code -> ternary value: 01 -> +1, 11 -> -1, 00 and the unused 10 -> 0.
__device__ __forceinline__ float code_to_f32(uint32_t code) {
    return (float)((int)(code & 1u) * (1 - (int)(code & 2u)));
}

// Two 2-bit codes held at bits 0-1 and 16-17 of xs -> two bf16 values in one
// dword, through a byte lookup with v_perm: selector bytes [c0, c0+4, c1, c1+4]
// pick the low byte from 0x80008000 (bytes 00 80 00 80) and the high byte from
// 0xBF803F00 (bytes 00 3F 80 BF), giving 0x0000, 0x3F80 (+1), 0x8000 (-0, the
// unused code) or 0xBF80 (-1).
__device__ __forceinline__ uint32_t tern_pair_bf16(uint32_t xs) {
    uint32_t sel = xs * 0x0101u + 0x04000400u;
    return __builtin_amdgcn_perm(0xBF803F00u, 0x80008000u, sel);
}

// Pair of consecutive-column codes (bits 0-3 of `nib`) times a pair of bf16
// scale bits `s2`: code 01 keeps the scale, 11 flips its sign bit, 00 gives 0.
__device__ __forceinline__ uint32_t scaled_pair_bf16(uint32_t w, int sh, uint32_t s2) {
    uint32_t xs = ((w >> sh) & 3u) | (((w >> (sh + 2)) & 3u) << 16);
    uint32_t nzm = (xs & 0x00010001u) * 0xFFFFu;
    uint32_t sgm = (xs & 0x00020002u) << 14;
    return (s2 & nzm) ^ sgm;
}

template <int BM_>
struct Geo {
    static constexpr int BM = BM_, BN = BM_;
    static constexpr int WM = 2, WN = 2;
    static constexpr int TM = BM / WM, TN = BN / WN;
    static constexpr int FM = TM / 32, FN = TN / 32;
    static constexpr int ROWS = BM + BN;  // LDS rows per buffer (A rows, then B rows)
};

// Workgroup -> (tile_m, tile_n, split).
__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int &tm, int &tn, int &sp) {
    const int nb = gridDim.x, b = blockIdx.x;
    int L = b;
    if ((nb & 7) == 0) L = (b & 7) * (nb >> 3) + (b >> 3);
    const int tiles = tiles_m * tiles_n;
    sp = L / tiles;
    const int t = L - sp * tiles;
    constexpr int GM = 8;
    const int group = t / (GM * tiles_n);
    const int first = group * GM;
    const int gs = min(tiles_m - first, GM);
    const int within = t - group * GM * tiles_n;
    tm = first + within % gs;
    tn = within / gs;
}

// ---------------------------------------------------------------------------
// Operand stagers.  Each fetches one K step of its tile into registers
// (fetch), then writes it to an LDS buffer as K-contiguous rows (commit).
// ---------------------------------------------------------------------------

// Rows of a row-major matrix whose K dimension is contiguous: X or dY as the
// N-side operand of the forward and dX products.  16-byte chunks copied as is.
template <bool BF, int R>
struct StageDirect {
    static constexpr int CH = R * 8 / NT;
    const char *base;   // row 0 of the tile
    int kbytes;         // bytes of K per row
    uint32_t off[CH];
    u32x4 v[CH];

    __device__ __forceinline__ void init(const void *p, int64_t ld_bytes, int rows_valid, int kb) {
        base = (const char *)p;
        kbytes = kb;
        const int tid = threadIdx.x;
#pragma unroll
        for (int i = 0; i < CH; i++) {
            const int cid = tid + NT * i, row = cid >> 3, ch = cid & 7;
            off[i] = row < rows_valid ? (uint32_t)(row * ld_bytes + ch * 16) : OOB;
        }
    }
    __device__ __forceinline__ void fetch(int kbyte0) {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + kbyte0);
        const bool kin = kbyte0 + (int)(threadIdx.x & 7) * 16 < kbytes;
#pragma unroll
        for (int i = 0; i < CH; i++) v[i] = bload128(rs, kin ? off[i] : OOB);
    }
    __device__ __forceinline__ void commit(u32x4 *sm) const {
        const int tid = threadIdx.x;
#pragma unroll
        for (int i = 0; i < CH; i++) {
            const int cid = tid + NT * i;
            sm[(cid >> 3) * RC + (cid & 7)] = v[i];
        }
    }
};

// Tokens-major activations read as the transposed operand of the dW product:
// source S[k][m] (k = token, m = feature), tile of BK tokens x R features.
// bf16: each unit is an 8 x 8 block transposed in registers with v_perm;
// fp32: a 4 x 4 block.
template <bool BF, int R>
struct StageTrans {
    static constexpr int KR = BF ? 8 : 4;      // k rows per unit
    static constexpr int MC = BF ? 8 : 4;      // m columns per unit (16 bytes)
    static constexpr int UNITS = 8 * (R / MC); // BK / KR == 8 for both types
    static constexpr int UPT = UNITS >= NT ? UNITS / NT : 1;
    const char *base;   // element (k = 0, m = tile's m0)
    int64_t ld;         // bytes per token row
    uint32_t coff[UPT]; // byte offset of the unit's 16-byte column chunk, or OOB
    u32x4 v[UPT][KR];

    __device__ __forceinline__ void init(const void *p, int64_t ld_bytes, int cols_valid) {
        base = (const char *)p;
        ld = ld_bytes;
        const int tid = threadIdx.x;
#pragma unroll
        for (int i = 0; i < UPT; i++) {
            const int u = tid + NT * i, mg = u >> 3;
            const bool act = u < UNITS;
            coff[i] = (act && mg * MC < cols_valid) ? (uint32_t)(mg * 16) : OOB;
        }
    }
    // k0: first token of this step, relative to base; krem: tokens left in range
    __device__ __forceinline__ void fetch(int64_t k0, int krem) {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + k0 * ld);
        const int kg = threadIdx.x & 7;
#pragma unroll
        for (int i = 0; i < UPT; i++) {
#pragma unroll
            for (int j = 0; j < KR; j++) {
                const int kr = kg * KR + j;
                const uint32_t o = (kr < krem && coff[i] != OOB) ? (uint32_t)(kr * ld) + coff[i] : OOB;
                v[i][j] = bload128(rs, o);
            }
        }
    }
    __device__ __forceinline__ void commit(u32x4 *sm) const {
        const int tid = threadIdx.x;
#pragma unroll
        for (int i = 0; i < UPT; i++) {
            const int u = tid + NT * i;
            if (u >= UNITS) continue;
            const int kg = u & 7, mg = u >> 3;
            if constexpr (BF) {
#pragma unroll
                for (int e = 0; e < 8; e++) {
                    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
                    u32x4 o;
                    o.x = __builtin_amdgcn_perm(v[i][1][e >> 1], v[i][0][e >> 1], sel);
                    o.y = __builtin_amdgcn_perm(v[i][3][e >> 1], v[i][2][e >> 1], sel);
                    o.z = __builtin_amdgcn_perm(v[i][5][e >> 1], v[i][4][e >> 1], sel);
                    o.w = __builtin_amdgcn_perm(v[i][7][e >> 1], v[i][6][e >> 1], sel);
                    sm[(mg * 8 + e) * RC + kg] = o;
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    u32x4 o;
                    o.x = v[i][0][e];
                    o.y = v[i][1][e];
                    o.z = v[i][2][e];
                    o.w = v[i][3][e];
                    sm[(mg * 4 + e) * RC + kg] = o;
                }
            }
        }
    }
};

// Forward weight operand: rows m = output columns c, K = input rows r.  The
// packed words hold 16 consecutive c of one r, so each unit reads KR words
// (KR consecutive r) of one 8-column half word and transposes while decoding.
template <bool BF, int R>
struct StageTernT {
    static constexpr int KR = BF ? 8 : 4;
    static constexpr int UNITS = 8 * (R / 8);
    static constexpr int UPT = UNITS >= NT ? UNITS / NT : 1;
    const char *base;   // word (r = 0, c = tile's m0)
    int64_t ldw;        // bytes per packed row
    uint32_t coff[UPT];
    uint32_t w[UPT][KR];

    __device__ __forceinline__ void init(const uint32_t *p, int64_t wpr, int words_valid) {
        base = (const char *)p;
        ldw = wpr * 4;
        const int tid = threadIdx.x;
#pragma unroll
        for (int i = 0; i < UPT; i++) {
            const int u = tid + NT * i, cg = u >> 3;
            const bool act = u < UNITS;
            coff[i] = (act && (cg >> 1) < words_valid) ? (uint32_t)((cg >> 1) * 4) : OOB;
        }
    }
    __device__ __forceinline__ void fetch(int64_t k0, int krem) {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + k0 * ldw);
        const int kg = threadIdx.x & 7;
#pragma unroll
        for (int i = 0; i < UPT; i++) {
#pragma unroll
            for (int j = 0; j < KR; j++) {
                const int kr = kg * KR + j;
                const uint32_t o = (kr < krem && coff[i] != OOB) ? (uint32_t)(kr * ldw) + coff[i] : OOB;
                w[i][j] = bload32(rs, o);
            }
        }
    }
    __device__ __forceinline__ void commit(u32x4 *sm) const {
        const int tid = threadIdx.x;
#pragma unroll
        for (int i = 0; i < UPT; i++) {
            const int u = tid + NT * i;
            if (u >= UNITS) continue;
            const int kg = u & 7, cg = u >> 3, half = cg & 1;
            if constexpr (BF) {
                // y[d]: this half word of rows 2d (low 16 bits) and 2d + 1 (high)
                const uint32_t hsel = half ? 0x07060302u : 0x05040100u;
                uint32_t y[4];
#pragma unroll
                for (int d = 0; d < 4; d++) y[d] = __builtin_amdgcn_perm(w[i][2 * d + 1], w[i][2 * d], hsel);
#pragma unroll
                for (int e = 0; e < 8; e++) {
                    u32x4 o;
                    o.x = tern_pair_bf16((y[0] >> (2 * e)) & 0x00030003u);
                    o.y = tern_pair_bf16((y[1] >> (2 * e)) & 0x00030003u);
                    o.z = tern_pair_bf16((y[2] >> (2 * e)) & 0x00030003u);
                    o.w = tern_pair_bf16((y[3] >> (2 * e)) & 0x00030003u);
                    sm[(cg * 8 + e) * RC + kg] = o;
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; e++) {
                    const int sh = 2 * (8 * half + e);
                    f32x4 o;
                    o.x = code_to_f32((w[i][0] >> sh) & 3u);
                    o.y = code_to_f32((w[i][1] >> sh) & 3u);
                    o.z = code_to_f32((w[i][2] >> sh) & 3u);
                    o.w = code_to_f32((w[i][3] >> sh) & 3u);
                    sm[(cg * 8 + e) * RC + kg] = __builtin_bit_cast(u32x4, o);
                }
            }
        }
    }
};

// dX weight operand: rows m = input rows r, K = output columns c (contiguous in
// the packed words), values tern * scale[c].  Each unit is one packed word
// (16 consecutive c of one r); the unit's K quarter is fixed per thread, so the
// 16 scales are loaded (and rounded to bf16) once per K step.
template <bool BF, int R>
struct StageTernS {
    static constexpr int WPK = BF ? 4 : 2;   // packed words per row per K step
    static constexpr int UNITS = R * WPK;
    static constexpr int UPT = UNITS >= NT ? UNITS / NT : 1;
    const char *base;   // word (r = tile's m0, c = 0)
    const float *scale;
    int64_t wpr;
    int out;
    uint32_t roff[UPT];
    uint32_t w[UPT];
    f32x4 s[4];

    __device__ __forceinline__ void init(const uint32_t *p, int64_t wpr_, int rows_valid,
                                         const float *sc, int out_) {
        base = (const char *)p;
        wpr = wpr_;
        scale = sc;
        out = out_;
        const int tid = threadIdx.x;
#pragma unroll
        for (int i = 0; i < UPT; i++) {
            const int u = tid + NT * i, row = u / WPK;
            const bool act = u < UNITS;
            roff[i] = (act && row < rows_valid) ? (uint32_t)(row * wpr * 4) : OOB;
        }
    }
    // k0: first output column of this K step (multiple of 16)
    __device__ __forceinline__ void fetch(int k0) {
        const int wq = threadIdx.x % WPK;
        const int wcol = (k0 >> 4) + wq;
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + (int64_t)(k0 >> 4) * 4);
        const bool win = wcol < wpr;
#pragma unroll
        for (int i = 0; i < UPT; i++) w[i] = bload32(rs, (win && roff[i] != OOB) ? roff[i] + wq * 4 : OOB);
        const int c0 = k0 + 16 * wq;
        const __amdgpu_buffer_rsrc_t rsc = make_rsrc(scale + c0);
#pragma unroll
        for (int q = 0; q < 4; q++)
            s[q] = __builtin_bit_cast(f32x4, bload128(rsc, (c0 + 4 * q < out) ? (uint32_t)(16 * q) : OOB));
    }
    __device__ __forceinline__ void commit(u32x4 *sm) const {
        const int tid = threadIdx.x;
        const int wq = tid % WPK;
        if constexpr (BF) {
            uint32_t s2[8];
#pragma unroll
            for (int q = 0; q < 4; q++) {
                f32x2 a = {s[q].x, s[q].y}, b = {s[q].z, s[q].w};
                s2[2 * q] = __builtin_bit_cast(uint32_t, __builtin_convertvector(a, bf16x2));
                s2[2 * q + 1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(b, bf16x2));
            }
#pragma unroll
            for (int i = 0; i < UPT; i++) {
                const int u = tid + NT * i;
                if (u >= UNITS) continue;
                const int row = u / WPK;
                u32x4 o0, o1;
                o0.x = scaled_pair_bf16(w[i], 0, s2[0]);
                o0.y = scaled_pair_bf16(w[i], 4, s2[1]);
                o0.z = scaled_pair_bf16(w[i], 8, s2[2]);
                o0.w = scaled_pair_bf16(w[i], 12, s2[3]);
                o1.x = scaled_pair_bf16(w[i], 16, s2[4]);
                o1.y = scaled_pair_bf16(w[i], 20, s2[5]);
                o1.z = scaled_pair_bf16(w[i], 24, s2[6]);
                o1.w = scaled_pair_bf16(w[i], 28, s2[7]);
                sm[row * RC + 2 * wq] = o0;
                sm[row * RC + 2 * wq + 1] = o1;
            }
        } else {
#pragma unroll
            for (int i = 0; i < UPT; i++) {
                const int u = tid + NT * i;
                if (u >= UNITS) continue;
                const int row = u / WPK;
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    f32x4 o;
                    o.x = code_to_f32((w[i] >> (8 * q)) & 3u) * s[q].x;
                    o.y = code_to_f32((w[i] >> (8 * q + 2)) & 3u) * s[q].y;
                    o.z = code_to_f32((w[i] >> (8 * q + 4)) & 3u) * s[q].z;
                    o.w = code_to_f32((w[i] >> (8 * q + 6)) & 3u) * s[q].w;
                    sm[row * RC + 4 * wq + q] = __builtin_bit_cast(u32x4, o);
                }
            }
        }
    }
};

// ---------------------------------------------------------------------------
// MFMA over one staged K step.  Fragment layout of the 32x32 MFMAs: lane l
// supplies row (l % 32) of A and column (l % 32) of B; bf16 lanes hold 8
// consecutive K, lanes 0-31 the first 8 and lanes 32-63 the next 8.  For fp32
// (K = 2 per instruction) lane half h of step j carries K index 16 h + j, the
// same for both operands, so each lane reads 4 steps with one 16-byte load.
// ---------------------------------------------------------------------------
template <bool BF, int BM>
__device__ __forceinline__ void mma_step(const u32x4 *smA, const u32x4 *smB,
                                         f32x16 (&acc)[Geo<BM>::FM][Geo<BM>::FN],
                                         int arow, int brow, int h) {
    using G = Geo<BM>;
    if constexpr (BF) {
#pragma unroll
        for (int kk = 0; kk < 4; kk++) {
            u32x4 a[G::FM], b[G::FN];
#pragma unroll
            for (int fm = 0; fm < G::FM; fm++) a[fm] = smA[(arow + fm * 32) * RC + 2 * kk + h];
#pragma unroll
            for (int fn = 0; fn < G::FN; fn++) b[fn] = smB[(brow + fn * 32) * RC + 2 * kk + h];
#pragma unroll
            for (int fm = 0; fm < G::FM; fm++)
#pragma unroll
                for (int fn = 0; fn < G::FN; fn++)
                    acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, a[fm]), __builtin_bit_cast(bf16x8, b[fn]),
                        acc[fm][fn], 0, 0, 0);
        }
    } else {
#pragma unroll
        for (int q = 0; q < 4; q++) {
            f32x4 a[G::FM], b[G::FN];
#pragma unroll
            for (int fm = 0; fm < G::FM; fm++)
                a[fm] = __builtin_bit_cast(f32x4, smA[(arow + fm * 32) * RC + 4 * h + q]);
#pragma unroll
            for (int fn = 0; fn < G::FN; fn++)
                b[fn] = __builtin_bit_cast(f32x4, smB[(brow + fn * 32) * RC + 4 * h + q]);
#pragma unroll
            for (int e = 0; e < 4; e++)
#pragma unroll
                for (int fm = 0; fm < G::FM; fm++)
#pragma unroll
                    for (int fn = 0; fn < G::FN; fn++)
                        acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[fm][e], b[fn][e],
                                                                           acc[fm][fn], 0, 0, 0);
        }
    }
}

// ---------------------------------------------------------------------------
// The GEMM kernel: MODE_FWD, MODE_DX or MODE_DW (see tern_plan.h for M, N, K).
// ---------------------------------------------------------------------------
template <bool BF, int MODE, int BM>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_kernel(GemmArgs g) {
    using G = Geo<BM>;
    constexpr int BK = BF ? 64 : 32;
    constexpr int ES = BF ? 2 : 4;
    __shared__ u32x4 smem[2 * G::ROWS * RC];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / G::WN, wn = wave % G::WN;
    const int l32 = lane & 31, h = lane >> 5;

    int tm, tn, sp;
    tile_coords(g.tiles_m, g.tiles_n, tm, tn, sp);
    const int m0 = tm * BM, n0 = tn * G::BN;
    const int64_t kbeg = (int64_t)sp * g.kps;
    const int64_t kend = min((int64_t)g.K, kbeg + g.kps);
    const int nk = (int)((kend - kbeg + BK - 1) / BK);

    // A side (rows m) and B side (rows n) stagers for this mode
    using SA = typename std::conditional<
        MODE == MODE_FWD, StageTernT<BF, BM>,
        typename std::conditional<MODE == MODE_DX, StageTernS<BF, BM>, StageTrans<BF, BM>>::type>::type;
    using SB = typename std::conditional<MODE == MODE_DW, StageTrans<BF, G::BN>,
                                         StageDirect<BF, G::BN>>::type;
    SA sa;
    SB sb;
    const int mvalid = g.M - m0, nvalid = g.N - n0;
    if constexpr (MODE == MODE_FWD) {
        // A: packed tern words of columns [m0, m0 + BM); B: X rows [n0, n0 + BN)
        sa.init(g.packed + m0 / 16, g.wpr, (int)(g.wpr - m0 / 16));
        sb.init((const char *)g.act0 + (int64_t)n0 * g.in * ES, (int64_t)g.in * ES, nvalid, g.in * ES);
    } else if constexpr (MODE == MODE_DX) {
        sa.init(g.packed + (int64_t)m0 * g.wpr, g.wpr, mvalid, g.scale, g.out);
        sb.init((const char *)g.act0 + (int64_t)n0 * g.out * ES, (int64_t)g.out * ES, nvalid, g.out * ES);
    } else {
        sa.init((const char *)g.act0 + kbeg * g.in * ES + (int64_t)m0 * ES, (int64_t)g.in * ES, mvalid);
        sb.init((const char *)g.act1 + kbeg * g.out * ES + (int64_t)n0 * ES, (int64_t)g.out * ES, nvalid);
    }

    auto fetch = [&](int it) {
        const int64_t k0 = (int64_t)it * BK;  // relative to kbeg
        const int krem = (int)min<int64_t>(BK, kend - kbeg - k0);
        if constexpr (MODE == MODE_FWD) {
            sa.fetch(k0, krem);
            sb.fetch((int)(k0 * ES));
        } else if constexpr (MODE == MODE_DX) {
            sa.fetch((int)k0);
            sb.fetch((int)(k0 * ES));
        } else {
            sa.fetch(k0, krem);
            sb.fetch(k0, krem);
        }
    };
    auto commit = [&](int buf) {
        sa.commit(smem + buf * G::ROWS * RC);
        sb.commit(smem + (buf * G::ROWS + BM) * RC);
    };

    f32x16 acc[G::FM][G::FN];
#pragma unroll
    for (int fm = 0; fm < G::FM; fm++)
#pragma unroll
        for (int fn = 0; fn < G::FN; fn++)
#pragma unroll
            for (int i = 0; i < 16; i++) acc[fm][fn][i] = 0.0f;

    fetch(0);
    commit(0);
    __syncthreads();
    const int arow = wm * G::TM + l32, brow = BM + wn * G::TN + l32;
    for (int it = 0; it < nk; it++) {
        const int cur = it & 1;
        const bool more = it + 1 < nk;
        if (more) fetch(it + 1);
        const u32x4 *sm = smem + cur * G::ROWS * RC;
        mma_step<BF, BM>(sm, sm, acc, arow, brow, h);
        if (more) commit(cur ^ 1);
        __syncthreads();
    }

    // ---- epilogues.  acc[fm][fn][i] is C[m][n] with
    //   m = m0 + wm*TM + fm*32 + 8*(i/4) + 4*h + i%4,  n = n0 + wn*TN + fn*32 + l32
    const int mw = m0 + wm * G::TM, nw = n0 + wn * G::TN;
    if constexpr (MODE == MODE_FWD || MODE == MODE_DX) {
        // output stored [n][m]: token-major rows of Y (m = c) or dX (m = r)
        const int ldo = (MODE == MODE_FWD) ? g.out : g.in;
#pragma unroll
        for (int fm = 0; fm < G::FM; fm++) {
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int m = mw + fm * 32 + 8 * q + 4 * h;
                if (m >= g.M) continue;
                f32x4 sc = {1.0f, 1.0f, 1.0f, 1.0f};
                if constexpr (MODE == MODE_FWD) sc = *(const f32x4 *)(g.scale + m);
#pragma unroll
                for (int fn = 0; fn < G::FN; fn++) {
                    const int n = nw + fn * 32 + l32;
                    if (n >= g.N) continue;
                    f32x4 v = {acc[fm][fn][4 * q], acc[fm][fn][4 * q + 1], acc[fm][fn][4 * q + 2],
                               acc[fm][fn][4 * q + 3]};
                    if constexpr (MODE == MODE_FWD) v = v * sc;
                    const int64_t o = (int64_t)n * ldo + m;
                    if (MODE == MODE_FWD && g.y_bf16) {
                        f32x2 a = {v.x, v.y}, b = {v.z, v.w};
                        u32x2 pk = {__builtin_bit_cast(uint32_t, __builtin_convertvector(a, bf16x2)),
                                    __builtin_bit_cast(uint32_t, __builtin_convertvector(b, bf16x2))};
                        *(u32x2 *)((uint16_t *)g.out_ptr + o) = pk;
                    } else {
                        *(f32x4 *)((float *)g.out_ptr + o) = v;
                    }
                }
            }
        }
    } else {
        // MODE_DW: C[m][n] = G[r][c] (m = r < in, n = c < out)
        float *dst = (float *)g.out_ptr;
        if (g.splits > 1) {
            dst += (int64_t)sp * g.M * g.N;
#pragma unroll
            for (int fm = 0; fm < G::FM; fm++)
#pragma unroll
                for (int i = 0; i < 16; i++) {
                    const int m = mw + fm * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
                    if (m >= g.M) continue;
#pragma unroll
                    for (int fn = 0; fn < G::FN; fn++) {
                        const int n = nw + fn * 32 + l32;
                        if (n < g.N) dst[(int64_t)m * g.N + n] = acc[fm][fn][i];
                    }
                }
            return;
        }
        float sc[G::FN], ps[G::FN];
#pragma unroll
        for (int fn = 0; fn < G::FN; fn++) {
            const int n = nw + fn * 32 + l32;
            sc[fn] = n < g.N ? g.scale[n] : 0.0f;
            ps[fn] = 0.0f;
        }
#pragma unroll
        for (int fm = 0; fm < G::FM; fm++)
#pragma unroll
            for (int i = 0; i < 16; i++) {
                const int m = mw + fm * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
                if (m >= g.M) continue;
#pragma unroll
                for (int fn = 0; fn < G::FN; fn++) {
                    const int n = nw + fn * 32 + l32;
                    if (n >= g.N) continue;
                    const float gv = acc[fm][fn][i];
                    dst[(int64_t)m * g.N + n] = gv * sc[fn];
                    const uint32_t word = g.packed[(int64_t)m * g.wpr + (n >> 4)];
                    ps[fn] += gv * code_to_f32((word >> (2 * (n & 15))) & 3u);
                }
            }
        // lanes l and l + 32 hold the two row halves of each column
#pragma unroll
        for (int fn = 0; fn < G::FN; fn++) ps[fn] += __shfl_xor(ps[fn], 32);
        float *red = (float *)smem;  // [WM][BN]; the main loop ended with a barrier
        if (h == 0) {
#pragma unroll
            for (int fn = 0; fn < G::FN; fn++) red[wm * G::BN + wn * G::TN + fn * 32 + l32] = ps[fn];
        }
        __syncthreads();
        if (tid < G::BN && n0 + tid < g.N) {
            float v = red[tid];
#pragma unroll
            for (int w2 = 1; w2 < G::WM; w2++) v += red[w2 * G::BN + tid];
            g.part[(int64_t)tm * g.N + n0 + tid] = v;
        }
    }
}

// ---------------------------------------------------------------------------
// Small kernels
// ---------------------------------------------------------------------------

// Ternarise and pack: one thread per packed word (16 codes of one row).
template <bool VEC>
__global__ __launch_bounds__(256) void materialize_kernel(const int8_t *__restrict__ q, int64_t out,
                                                          int64_t wpr, int theta,
                                                          uint32_t *__restrict__ packed, int64_t nwords) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= nwords) return;
    const int64_t r = i / wpr, wc = i - r * wpr;
    const int8_t *row = q + r * out + wc * 16;
    uint32_t word = 0;
    if constexpr (VEC) {
        const u32x4 v = *(const u32x4 *)row;
#pragma unroll
        for (int j = 0; j < 16; j++) {
            const int b = (int)(int8_t)((v[j >> 2] >> (8 * (j & 3))) & 0xFFu);
            const uint32_t code = b >= theta ? 1u : (b <= -theta ? 3u : 0u);
            word |= code << (2 * j);
        }
    } else {
        const int64_t nc = out - wc * 16;
#pragma unroll
        for (int j = 0; j < 16; j++) {
            if (j < nc) {
                const int b = row[j];
                const uint32_t code = b >= theta ? 1u : (b <= -theta ? 3u : 0u);
                word |= code << (2 * j);
            }
        }
    }
    packed[i] = word;
}

// Split-K finish of dW: G = sum over splits (ascending), gq = G * scale, and
// the sgrad partial of a block of kReduceRows rows (ascending r).
__global__ __launch_bounds__(256) void dw_reduce_kernel(const float *__restrict__ ws, int splits,
                                                        const float *__restrict__ scale,
                                                        const uint32_t *__restrict__ packed, int in,
                                                        int out, int64_t wpr, float *__restrict__ gq,
                                                        float *__restrict__ part) {
    const int c = blockIdx.x * 256 + threadIdx.x;
    if (c >= out) return;
    const int r0 = blockIdx.y * 64;
    const int r1 = min(in, r0 + 64);
    const float s = scale[c];
    const int64_t plane = (int64_t)in * out;
    float p = 0.0f;
    for (int r = r0; r < r1; r++) {
        const int64_t o = (int64_t)r * out + c;
        float gv = 0.0f;
        for (int k = 0; k < splits; k++) gv += ws[k * plane + o];
        gq[o] = gv * s;
        const uint32_t word = packed[(int64_t)r * wpr + (c >> 4)];
        p += gv * code_to_f32((word >> (2 * (c & 15))) & 3u);
    }
    part[(int64_t)blockIdx.y * out + c] = p;
}

// sgrad[c] = sum of the partials in ascending row-block order, in f64.
__global__ __launch_bounds__(256) void sgrad_reduce_kernel(const float *__restrict__ part, int nparts,
                                                           int out, float *__restrict__ sgrad) {
    const int c = blockIdx.x * 256 + threadIdx.x;
    if (c >= out) return;
    double a = 0.0;
    for (int p = 0; p < nparts; p++) a += (double)part[(int64_t)p * out + c];
    sgrad[c] = (float)a;
}

// Zero fill in 16-byte units.
__global__ __launch_bounds__(256) void zero16_kernel(u32x4 *__restrict__ p, int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) p[i] = z;
}

}  // namespace dev

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------

namespace {
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

template <bool BF, int MODE>
hipError_t launch_mode(const GemmPlan &p, const GemmArgs &a, hipStream_t st) {
    const dim3 grid((unsigned)p.grid), block(dev::NT);
    switch (p.tile) {
        case TILE_256: hipLaunchKernelGGL((dev::gemm_kernel<BF, MODE, 256>), grid, block, 0, st, a); break;
        case TILE_128: hipLaunchKernelGGL((dev::gemm_kernel<BF, MODE, 128>), grid, block, 0, st, a); break;
        default: hipLaunchKernelGGL((dev::gemm_kernel<BF, MODE, 64>), grid, block, 0, st, a); break;
    }
    return hipGetLastError();
}
}  // namespace

hipError_t launch_gemm(const GemmPlan &p, bool bf16, const GemmArgs &a, hipStream_t st) {
    if (p.grid <= 0) return hipSuccess;
    if (bf16) {
        if (p.mode == MODE_FWD) return launch_mode<true, MODE_FWD>(p, a, st);
        if (p.mode == MODE_DX) return launch_mode<true, MODE_DX>(p, a, st);
        return launch_mode<true, MODE_DW>(p, a, st);
    }
    if (p.mode == MODE_FWD) return launch_mode<false, MODE_FWD>(p, a, st);
    if (p.mode == MODE_DX) return launch_mode<false, MODE_DX>(p, a, st);
    return launch_mode<false, MODE_DW>(p, a, st);
}

hipError_t launch_materialize(const int8_t *q, int64_t in, int64_t out, int theta, bool vec,
                              uint32_t *packed, hipStream_t st) {
    const int64_t wpr = cdiv(out, 16);
    const int64_t nwords = in * wpr;
    if (nwords <= 0) return hipSuccess;
    const dim3 grid((unsigned)cdiv(nwords, 256)), block(256);
    if (vec)
        hipLaunchKernelGGL((dev::materialize_kernel<true>), grid, block, 0, st, q, out, wpr, theta, packed, nwords);
    else
        hipLaunchKernelGGL((dev::materialize_kernel<false>), grid, block, 0, st, q, out, wpr, theta, packed, nwords);
    return hipGetLastError();
}

hipError_t launch_dw_reduce(const float *ws, int splits, const float *scale, const uint32_t *packed,
                            int64_t in, int64_t out, float *gq, float *part, hipStream_t st) {
    const dim3 grid((unsigned)cdiv(out, 256), (unsigned)cdiv(in, kReduceRows)), block(256);
    hipLaunchKernelGGL(dev::dw_reduce_kernel, grid, block, 0, st, ws, splits, scale, packed, (int)in,
                       (int)out, cdiv(out, 16), gq, part);
    return hipGetLastError();
}

hipError_t launch_sgrad_reduce(const float *part, int64_t nparts, int64_t out, float *sgrad, hipStream_t st) {
    if (out <= 0) return hipSuccess;
    const dim3 grid((unsigned)cdiv(out, 256)), block(256);
    hipLaunchKernelGGL(dev::sgrad_reduce_kernel, grid, block, 0, st, part, (int)nparts, (int)out, sgrad);
    return hipGetLastError();
}

hipError_t launch_zero(void *p, size_t bytes, hipStream_t st) {
    if (bytes == 0) return hipSuccess;
    const int64_t n16 = (int64_t)(bytes / 16);
    int64_t blocks = cdiv(n16, 256);
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(dev::zero16_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (dev::u32x4 *)p, n16);
    return hipGetLastError();
}

}  // namespace tern
