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
//     HBM.  The GEMMs read the packed words (or a fragment-ordered copy of
//     them) and decode them in registers: the generic kernel below stages the
//     decoded bf16 (or fp32) operand tile in LDS, the persistent forward / dX
//     kernel decodes straight into MFMA operand registers.
//   * Forward: the scale multiplies the fp32 column sums in the epilogue.
//     dX: the scale sits on the reduction index, so it is folded into the
//     decoded operand as +-bf16(scale[c]) (fp32 path: exact +-scale[c]).
//     dW: the epilogue writes gq = G * scale[c] and reduces G * tern over the
//     tile's rows in a fixed order into per-row-tile partials; a second kernel
//     sums the partials in ascending row-tile order (deterministic sgrad).
//   * One generic GEMM template (fp32, tiles below 256 x 256, and the bf16
//     cases the persistent kernels do not take: K < 32, a dW side below 256,
//     the two-term dX scale): 256 threads = 4 wave64s in 2 x 2, each wave
//     owning a
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
//   * The bf16 products with full tiles run persistent kernels over a group
//     of problems (all projections of a layer), walked statically or in
//     balanced classes of workgroups (group_item, tern_plan.h):
//     - gemm_rd_kernel (forward, dX): 512 x 128 tiles (output columns x
//       tokens); the four waves, side by side along the columns, stream the
//       tile's 128 activation rows through one shared ring of four LDS
//       stages, each loading a quarter, with one workgroup barrier per chunk;
//       each wave decodes the fp4 fragment copy of tern in registers, runs
//       the MFMAs with the activations as A (the tile lands transposed in the
//       accumulators) and stores whole lines straight from them;
//     - gemm_dw_kernel (dW, 256 x 256 tiles): two shared 64-token stages of X and dY with
//       transposing LDS reads, one barrier per stage, and 4-byte L2 warm-up
//       loads for the chunk three beyond each refill.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

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
// The same with a record count of n bytes (offsets >= n read as zero).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_n(const void *p, uint32_t n) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)n, 0x00020000);
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
// Operand stagers.  Each fetches one K step of its tile into one of two
// register sets (fetch<S>), then writes it to an LDS buffer as K-contiguous
// rows, one output chunk at a time (commit<S>(j), j < NOUT), so the writes can
// be spread between the MFMAs of the step being computed.
// ---------------------------------------------------------------------------

// Rows of a row-major matrix whose K dimension is contiguous: X or dY as the
// N-side operand of the forward and dX products.  16-byte chunks copied as is.
template <bool BF, int R>
struct StageDirect {
    static constexpr int CH = R * 8 / NT;
    static constexpr int NOUT = CH;
    const char *base;   // row 0 of the tile
    int kbytes;         // bytes of K per row
    uint32_t off[CH];
    u32x4 v[2][CH];

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
    // kbyte0: byte offset of this K step within a row
    template <int S>
    __device__ __forceinline__ void fetch(int kbyte0) {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + kbyte0);
        const bool kin = kbyte0 + (int)(threadIdx.x & 7) * 16 < kbytes;
#pragma unroll
        for (int i = 0; i < CH; i++) v[S][i] = bload128(rs, kin ? off[i] : OOB);
    }
    template <int S>
    __device__ __forceinline__ void commit(int j, u32x4 *sm) const {
        const int cid = (int)threadIdx.x + NT * j;
        sm[(cid >> 3) * RC + (cid & 7)] = v[S][j];
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
    static constexpr int NOUT = UPT * MC;      // one LDS chunk per m column
    const char *base;   // element (k = 0, m = tile's m0)
    int64_t ld;         // bytes per token row
    uint32_t coff[UPT]; // byte offset of the unit's 16-byte column chunk, or OOB
    u32x4 v[2][UPT][KR];

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
    template <int S>
    __device__ __forceinline__ void fetch(int64_t k0, int krem) {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + k0 * ld);
        const int kg = threadIdx.x & 7;
#pragma unroll
        for (int i = 0; i < UPT; i++) {
#pragma unroll
            for (int j = 0; j < KR; j++) {
                const int kr = kg * KR + j;
                const uint32_t o = (kr < krem && coff[i] != OOB) ? (uint32_t)(kr * ld) + coff[i] : OOB;
                v[S][i][j] = bload128(rs, o);
            }
        }
    }
    template <int S>
    __device__ __forceinline__ void commit(int jo, u32x4 *sm) const {
        const int i = jo / MC, e = jo % MC;
        const int u = (int)threadIdx.x + NT * i;
        if constexpr (UNITS < NT) {
            if (u >= UNITS) return;
        }
        const int kg = u & 7, mg = u >> 3;
        u32x4 o;
        if constexpr (BF) {
            const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
            o.x = __builtin_amdgcn_perm(v[S][i][1][e >> 1], v[S][i][0][e >> 1], sel);
            o.y = __builtin_amdgcn_perm(v[S][i][3][e >> 1], v[S][i][2][e >> 1], sel);
            o.z = __builtin_amdgcn_perm(v[S][i][5][e >> 1], v[S][i][4][e >> 1], sel);
            o.w = __builtin_amdgcn_perm(v[S][i][7][e >> 1], v[S][i][6][e >> 1], sel);
        } else {
            o.x = v[S][i][0][e];
            o.y = v[S][i][1][e];
            o.z = v[S][i][2][e];
            o.w = v[S][i][3][e];
        }
        sm[(mg * MC + e) * RC + kg] = o;
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
    static constexpr int NOUT = UPT * 8;       // one LDS chunk per column of the half word
    const char *base;   // word (r = 0, c = tile's m0)
    int64_t ldw;        // bytes per packed row
    uint32_t coff[UPT];
    uint32_t w[2][UPT][KR];

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
    template <int S>
    __device__ __forceinline__ void fetch(int64_t k0, int krem) {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + k0 * ldw);
        const int kg = threadIdx.x & 7;
#pragma unroll
        for (int i = 0; i < UPT; i++) {
#pragma unroll
            for (int j = 0; j < KR; j++) {
                const int kr = kg * KR + j;
                const uint32_t o = (kr < krem && coff[i] != OOB) ? (uint32_t)(kr * ldw) + coff[i] : OOB;
                w[S][i][j] = bload32(rs, o);
            }
        }
    }
    template <int S>
    __device__ __forceinline__ void commit(int jo, u32x4 *sm) const {
        const int i = jo / 8, e = jo % 8;
        const int u = (int)threadIdx.x + NT * i;
        if constexpr (UNITS < NT) {
            if (u >= UNITS) return;
        }
        const int kg = u & 7, cg = u >> 3, half = cg & 1;
        u32x4 o;
        if constexpr (BF) {
            // y_d: this half word of rows 2d (low 16 bits) and 2d + 1 (high)
            const uint32_t hsel = half ? 0x07060302u : 0x05040100u;
            const uint32_t y0 = __builtin_amdgcn_perm(w[S][i][1], w[S][i][0], hsel);
            const uint32_t y1 = __builtin_amdgcn_perm(w[S][i][3], w[S][i][2], hsel);
            const uint32_t y2 = __builtin_amdgcn_perm(w[S][i][5], w[S][i][4], hsel);
            const uint32_t y3 = __builtin_amdgcn_perm(w[S][i][7], w[S][i][6], hsel);
            o.x = tern_pair_bf16((y0 >> (2 * e)) & 0x00030003u);
            o.y = tern_pair_bf16((y1 >> (2 * e)) & 0x00030003u);
            o.z = tern_pair_bf16((y2 >> (2 * e)) & 0x00030003u);
            o.w = tern_pair_bf16((y3 >> (2 * e)) & 0x00030003u);
        } else {
            const int sh = 2 * (8 * half + e);
            f32x4 f;
            f.x = code_to_f32((w[S][i][0] >> sh) & 3u);
            f.y = code_to_f32((w[S][i][1] >> sh) & 3u);
            f.z = code_to_f32((w[S][i][2] >> sh) & 3u);
            f.w = code_to_f32((w[S][i][3] >> sh) & 3u);
            o = __builtin_bit_cast(u32x4, f);
        }
        sm[(cg * 8 + e) * RC + kg] = o;
    }
};

// dX weight operand: rows m = input rows r, K = output columns c (contiguous in
// the packed words), values tern * scale[c].  Each unit is one packed word
// (16 consecutive c of one r); the unit's K quarter is fixed per thread, so the
// 16 scales are loaded (and rounded to bf16) once per K step.  bf16: a step of
// the first pass over K uses hi = bf16(scale), a step of the second pass (exact
// scale) lo = bf16(scale - hi), so the two passes together carry the scale to
// about 16 significant bits.
template <bool BF, int R>
struct StageTernS {
    static constexpr int WPK = BF ? 4 : 2;   // packed words per row per K step
    static constexpr int UNITS = R * WPK;
    static constexpr int UPT = UNITS >= NT ? UNITS / NT : 1;
    static constexpr int CPU_ = BF ? 2 : 4;  // LDS chunks per unit
    static constexpr int NOUT = UPT * CPU_;
    const char *base;   // word (r = tile's m0, c = 0)
    const float *scale;
    int64_t wpr;
    int out;
    uint32_t roff[UPT];
    uint32_t w[2][UPT];
    f32x4 s[2][4];
    bool lo[2];         // register set S holds a second-pass (scale - hi) step

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
    // k0: first output column of this K step (multiple of 16); second: the
    // step belongs to the second pass over K
    template <int S>
    __device__ __forceinline__ void fetch(int k0, bool second = false) {
        lo[S] = second;
        const int wq = threadIdx.x % WPK;
        const int wcol = (k0 >> 4) + wq;
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + (int64_t)(k0 >> 4) * 4);
        const bool win = wcol < wpr;
#pragma unroll
        for (int i = 0; i < UPT; i++) w[S][i] = bload32(rs, (win && roff[i] != OOB) ? roff[i] + wq * 4 : OOB);
        const int c0 = k0 + 16 * wq;
        const __amdgpu_buffer_rsrc_t rsc = make_rsrc(scale + c0);
#pragma unroll
        for (int q = 0; q < 4; q++)
            s[S][q] = __builtin_bit_cast(f32x4, bload128(rsc, (c0 + 4 * q < out) ? (uint32_t)(16 * q) : OOB));
    }
    template <int S>
    __device__ __forceinline__ void commit(int jo, u32x4 *sm) const {
        const int i = jo / CPU_, c = jo % CPU_;
        const int u = (int)threadIdx.x + NT * i;
        if constexpr (UNITS < NT) {
            if (u >= UNITS) return;
        }
        const int wq = (int)threadIdx.x % WPK, row = u / WPK;
        u32x4 o;
        if constexpr (BF) {
            // two pairs of bf16 scales per f32x4 of scales
            uint32_t s2[4];
#pragma unroll
            for (int q = 0; q < 2; q++) {
                f32x4 sq = s[S][2 * c + q];
                if (lo[S]) {
                    // the part of the scale that bf16 rounding dropped
                    const f32x2 a0 = {sq.x, sq.y}, b0 = {sq.z, sq.w};
                    const f32x2 ah = __builtin_convertvector(__builtin_convertvector(a0, bf16x2), f32x2);
                    const f32x2 bh = __builtin_convertvector(__builtin_convertvector(b0, bf16x2), f32x2);
                    sq = f32x4{sq.x - ah.x, sq.y - ah.y, sq.z - bh.x, sq.w - bh.y};
                }
                f32x2 a = {sq.x, sq.y}, b = {sq.z, sq.w};
                s2[2 * q] = __builtin_bit_cast(uint32_t, __builtin_convertvector(a, bf16x2));
                s2[2 * q + 1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(b, bf16x2));
            }
            o.x = scaled_pair_bf16(w[S][i], 16 * c + 0, s2[0]);
            o.y = scaled_pair_bf16(w[S][i], 16 * c + 4, s2[1]);
            o.z = scaled_pair_bf16(w[S][i], 16 * c + 8, s2[2]);
            o.w = scaled_pair_bf16(w[S][i], 16 * c + 12, s2[3]);
            sm[row * RC + 2 * wq + c] = o;
        } else {
            const f32x4 sq = s[S][c];
            f32x4 f;
            f.x = code_to_f32((w[S][i] >> (8 * c)) & 3u) * sq.x;
            f.y = code_to_f32((w[S][i] >> (8 * c + 2)) & 3u) * sq.y;
            f.z = code_to_f32((w[S][i] >> (8 * c + 4)) & 3u) * sq.z;
            f.w = code_to_f32((w[S][i] >> (8 * c + 6)) & 3u) * sq.w;
            sm[row * RC + 4 * wq + c] = __builtin_bit_cast(u32x4, f);
        }
    }
};

// ---------------------------------------------------------------------------
// MFMA over one quarter of a staged K step (K = 16 bf16 or 8 fp32).  Fragment
// layout of the 32x32 MFMAs: lane l supplies row (l % 32) of A and column
// (l % 32) of B; bf16 lanes hold 8 consecutive K, lanes 0-31 the first 8 and
// lanes 32-63 the next 8.  For fp32 (K = 2 per instruction) lane half h of
// instruction j carries K index 16 h + j, the same for both operands, so a lane
// reads 4 instructions' operands with one 16-byte load.
// ---------------------------------------------------------------------------
template <bool BF, int BM>
__device__ __forceinline__ void mma_quarter(const u32x4 *sm, f32x16 (&acc)[Geo<BM>::FM][Geo<BM>::FN],
                                            int arow, int brow, int h, int kk) {
    using G = Geo<BM>;
    const int ch = BF ? 2 * kk + h : 4 * h + kk;
    u32x4 a[G::FM], b[G::FN];
#pragma unroll
    for (int fm = 0; fm < G::FM; fm++) a[fm] = sm[(arow + fm * 32) * RC + ch];
#pragma unroll
    for (int fn = 0; fn < G::FN; fn++) b[fn] = sm[(brow + fn * 32) * RC + ch];
    if constexpr (BF) {
#pragma unroll
        for (int fm = 0; fm < G::FM; fm++)
#pragma unroll
            for (int fn = 0; fn < G::FN; fn++)
                acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, a[fm]), __builtin_bit_cast(bf16x8, b[fn]), acc[fm][fn], 0, 0, 0);
    } else {
#pragma unroll
        for (int e = 0; e < 4; e++)
#pragma unroll
            for (int fm = 0; fm < G::FM; fm++)
#pragma unroll
                for (int fn = 0; fn < G::FN; fn++)
                    acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                        __builtin_bit_cast(f32x4, a[fm])[e], __builtin_bit_cast(f32x4, b[fn])[e], acc[fm][fn],
                        0, 0, 0);
    }
}

// ---------------------------------------------------------------------------
// The GEMM kernel: MODE_FWD, MODE_DX or MODE_DW (see tern_plan.h for M, N, K).
//
// Main loop (two LDS buffers, two register sets), iteration it:
//   issue the global loads of K step it + 2 into register set it % 2;
//   for each K quarter: MFMAs on LDS buffer it % 2, interleaved with the
//   decode and LDS writes of K step it + 1 (register set (it + 1) % 2) into
//   LDS buffer (it + 1) % 2;
//   barrier.
// Steps at or past the end load nothing (out-of-range offsets read zero) and
// their LDS buffer is never read, so the loop body has no branches.
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
    // dX with bf16 activations and the exact scale: the K steps run twice,
    // the second time with the scale's bf16 remainder (steps past the last
    // load nothing)
    const int passes = (MODE == MODE_DX && BF && g.exact_scale) ? 2 : 1;
    const int nsteps = passes * nk;

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
    const int64_t klen = kend - kbeg;

    auto fetch = [&](auto set_c, int it_all) {
        constexpr int S = decltype(set_c)::value;
        const bool second = it_all >= nk && it_all < nsteps;
        const int it = it_all < nsteps ? it_all - (second ? nk : 0) : nk;   // nk: past the end
        const int64_t k0 = (int64_t)it * BK;  // relative to kbeg
        const int krem = (int)max<int64_t>(-1, min<int64_t>(BK, klen - k0));
        if constexpr (MODE == MODE_FWD) {
            sa.template fetch<S>(k0, krem);
            sb.template fetch<S>((int)(k0 * ES));
        } else if constexpr (MODE == MODE_DX) {
            sa.template fetch<S>((int)k0, second);
            sb.template fetch<S>((int)(k0 * ES));
        } else {
            sa.template fetch<S>(k0, krem);
            sb.template fetch<S>(k0, krem);
        }
    };
    // commit the outputs of quarter p (of 4) of register set S into LDS buffer `buf`
    auto commit_part = [&](auto set_c, int buf, int p) {
        constexpr int S = decltype(set_c)::value;
        u32x4 *smA = smem + buf * G::ROWS * RC;
        u32x4 *smB = smem + (buf * G::ROWS + BM) * RC;
#pragma unroll
        for (int j = 0; j < SA::NOUT; j++)
            if (j % 4 == p) sa.template commit<S>(j, smA);
#pragma unroll
        for (int j = 0; j < SB::NOUT; j++)
            if (j % 4 == p) sb.template commit<S>(j, smB);
    };

    f32x16 acc[G::FM][G::FN];
#pragma unroll
    for (int fm = 0; fm < G::FM; fm++)
#pragma unroll
        for (int fn = 0; fn < G::FN; fn++)
#pragma unroll
            for (int i = 0; i < 16; i++) acc[fm][fn][i] = 0.0f;

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    const int arow = wm * G::TM + l32, brow = BM + wn * G::TN + l32;

    if constexpr (MODE != MODE_DW) {
        // two register sets: loads run two K steps ahead of the MFMAs
        fetch(I0{}, 0);
        fetch(I1{}, 1);
#pragma unroll
        for (int p = 0; p < 4; p++) commit_part(I0{}, 0, p);
        __syncthreads();

        // one pipelined K step: compute on LDS buffer CUR, stage register set
        // 1 - CUR (step it + 1) into the other buffer, refill register set CUR
        // with step it + 2
        auto body = [&](auto cur_c, int it) {
            constexpr int CUR = decltype(cur_c)::value;
            fetch(std::integral_constant<int, CUR>{}, it + 2);
            const u32x4 *sm = smem + CUR * G::ROWS * RC;
#pragma unroll
            for (int kk = 0; kk < 4; kk++) {
                mma_quarter<BF, BM>(sm, acc, arow, brow, h, kk);
                commit_part(std::integral_constant<int, 1 - CUR>{}, 1 - CUR, kk);
            }
            __syncthreads();
        };
        // pairs of steps keep the register sets static; an odd count runs one
        // extra step on an all-zero buffer, which adds nothing
        for (int it = 0; it < nsteps; it += 2) {
            body(I0{}, it);
            body(I1{}, it + 1);
        }
    } else {
        // dW: both operands are transposed while staging, which needs twice
        // the registers per step; one register set, one step ahead
        fetch(I0{}, 0);
#pragma unroll
        for (int p = 0; p < 4; p++) commit_part(I0{}, 0, p);
        __syncthreads();
        for (int it = 0; it < nk; it++) {
            const int cur = it & 1;
            fetch(I0{}, it + 1);
            const u32x4 *sm = smem + cur * G::ROWS * RC;
#pragma unroll
            for (int kk = 0; kk < 4; kk++) mma_quarter<BF, BM>(sm, acc, arow, brow, h, kk);
#pragma unroll
            for (int p = 0; p < 4; p++) commit_part(I0{}, cur ^ 1, p);
            __syncthreads();
        }
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
                    if (MODE == MODE_DX && g.acc) v += *(const f32x4 *)((const float *)g.out_ptr + o);
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
        if (g.splits > 1 || g.acc) {   // raw G of this split (sp = 0 with one split)
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
// dW GEMM (bf16, 256 x 256 tiles, persistent, split-K): G[r][c] = sum over
// tokens t of X[t][r] dY[t][c].  Both operands are token-major.  They stream
// into two LDS stages in chunks of 64 tokens with direct-to-LDS buffer loads
// (across tile and split boundaries), and the MFMA fragments come from
// ds_read_b64_tr_b16 transposing reads.  One barrier per chunk, before the
// chunk's last K quarter: past it no wave reads the chunk's stage any more, so
// the refill with the chunk after the next one starts there.  Its X half goes
// out during the last quarter's MFMAs and its dY half during the next chunk's
// first quarter, one load per two MFMAs: a CU's 64 refill loads need about as
// many address-unit cycles as two quarters of MFMAs, and packed into one
// quarter they stalled the waves' issue (4 % slower dW).  The next barrier
// waits for both halves.
// Epilogue, one split: gq = G * scale[c], and the tile's per-column sum of
// G * tern over its 256 rows (fixed order) into the partial table; several
// splits: the split's raw G, summed by dw_reduce_kernel.
// ---------------------------------------------------------------------------

typedef short v4i16 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

constexpr int W_KC = 64;                 // tokens per chunk
constexpr int W_NST = 2;                 // LDS stages
constexpr int W_Q = W_KC / 16;           // MFMA K quarters per chunk
constexpr int W_DR = W_KC / 8;           // DMA instructions per wave per operand and chunk
constexpr int W_OP = W_KC * 512;         // one operand of a stage: W_KC tokens x 256 features
constexpr int W_STAGE = 2 * W_OP;
__shared__ __attribute__((aligned(16))) char w_lds[W_NST * W_STAGE];
__shared__ float w_red[2 * 256];         // cross-wave sgrad partials of a tile

// 16 bytes per lane to LDS at lds + IMM + 16 lane from voff + soff + IMM; the
// immediate moves both addresses and is covered by the range check.
template <int IMM>
__device__ __forceinline__ void dma16_imm(__amdgpu_buffer_rsrc_t rs, void *lds, uint32_t voff, int soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void *)lds, 16, voff, soff, IMM, 0);
}

__device__ __forceinline__ void wait_vm0() {
    // vmcnt(0), leave expcnt and lgkmcnt at their maxima
    __builtin_amdgcn_s_waitcnt(0x0F70);
}

// Item j of this workgroup in the walk of a group of problems (group_item).
__device__ __forceinline__ bool g_item(const GroupArgs &ga, int j, int &pi, int &tm, int &tn, int &sp) {
    return group_item(ga, (int)gridDim.x, (int)blockIdx.x, j, pi, tm, tn, sp);
}

// DMA of one chunk of a token-major operand: W_KC token rows x 256 features
// (512 bytes).  Wave w, instruction i (< W_DR) writes rows 2 (W_DR w + i) and
// + 1; lane l fills physical chunk l % 32 of row (l / 32) with the logical chunk
// (l % 32) ^ (4 (row % 4)), which puts the four token rows of a transposing read
// in four different 64-byte quarters of a 256-byte window.  Four instructions
// share one M0: the immediate offset 1024 (i % 4) moves the LDS destination and
// the global address alike, so the lane offsets are stored less 1024 (i % 4)
// (which needs 2 rows of a token-major operand to span 1024 bytes: M, N >= 256).
// The resource's record count ends at the item's last token row, so rows past
// it (ragged or padding chunks, or no item at all) read as zero.
struct DmaTok {
    uint32_t off[W_DR];   // per instruction: lane offset less 1024 (i % 4), or OOB less that
    __device__ __forceinline__ void init(int64_t ld_bytes, int cols_valid, int wave) {
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int i = 0; i < W_DR; i++) {
            const int row = 2 * (W_DR * wave + i) + (lane >> 5);
            const int c = (lane & 31) ^ (4 * (row & 3));
            off[i] = (c * 8 < cols_valid ? (uint32_t)(row * ld_bytes + c * 16) : OOB) - 1024u * (uint32_t)(i & 3);
        }
    }
    // load I of this wave; rs: resource from token row 0 of the chunk whose
    // record count ends at the item's last row (0: nothing in range)
    template <int I>
    __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, char *lds_region, int wave) const {
        dma16_imm<(I & 3) * 1024>(rs, lds_region + (W_DR * wave + (I & ~3)) * 1024, off[I], 0);
    }
};

// Token-major tiles: two transposing reads per fragment.  In a group of 16
// lanes, lane s = 4e + q reads 8 bytes at token row k0 + e, feature col0 + 4q;
// output lane i then holds features col0 + i at tokens k0 .. k0 + 3.
__device__ __forceinline__ u32x4 p_frag_tr(const char *tile, int krow0, int col) {
    // krow0: this lane's token row for read 0 (multiple of 4 plus e); col: its
    // 4-feature column start
    u32x4 r;
#pragma unroll
    for (int rd = 0; rd < 2; rd++) {
        const int k = krow0 + 4 * rd;
        const int chunk = (col >> 3) ^ (4 * (k & 3));
        const char *p = tile + k * 512 + chunk * 16 + (col & 7) * 2;
        v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4i16 *)p);
        const u32x2 u = __builtin_bit_cast(u32x2, v);
        if (rd == 0) { r.x = u.x; r.y = u.y; } else { r.z = u.x; r.w = u.y; }
    }
    return r;
}

// Fragments of K quarter kk (16 tokens) of a stage: X^T rows wm * 128 .. and
// dY^T columns wn * 128 ..
__device__ __forceinline__ void w_read_q(const char *st, u32x4 (&a)[4], u32x4 (&b)[4], int wm, int wn,
                                         int lane, int kk) {
    const int g = (lane & 63) >> 4, s = lane & 15, e = s >> 2, q = s & 3;
    const int krow0 = 16 * kk + 8 * (g >> 1) + e;
    const int cofs = 16 * (g & 1) + 4 * q;
#pragma unroll
    for (int f = 0; f < 4; f++) a[f] = p_frag_tr(st, krow0, wm * 128 + 32 * f + cofs);
#pragma unroll
    for (int f = 0; f < 4; f++) b[f] = p_frag_tr(st + W_OP, krow0, wn * 128 + 32 * f + cofs);
}

__device__ __forceinline__ void p_mma(f32x16 (&acc)[4][4], const u32x4 (&a)[4], const u32x4 (&b)[4]) {
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, a[i]), __builtin_bit_cast(bf16x8, b[j]), acc[i][j], 0, 0, 0);
}

// Workgroup barrier after an explicit wait: vmcnt(N) (this wave's loads up to
// all but its N latest are complete) and lgkmcnt(0).  Unlike __syncthreads it
// does not wait for every outstanding load.
template <int N>
__device__ __forceinline__ void w_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt is six bits");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0070);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
}

__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_dw_kernel(GroupArgs ga) {
    constexpr int ES = 2;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, h = lane >> 5;

    // chunks of item (tile, split) sp of problem pi: its tokens, rounded up
    // to an even count
    auto item_chunks = [&](int pi, int sp, int64_t &kbeg, int64_t &klen) __attribute__((always_inline)) {
        const int64_t kps = ga.p[pi].kps;
        kbeg = (int64_t)sp * kps;
        klen = min((int64_t)ga.p[pi].K, kbeg + kps) - kbeg;
        const int n = (int)((klen + W_KC - 1) / W_KC);
        return (n + 1) & ~1;
    };

    // ---- issue side: chunk ic of item ij (problem ipi); iv false once the
    // items run out (every record count is then 0: zeros into LDS, no memory
    // access)
    int ij = 0, ic = 0, itm = 0, itn = 0, isp = 0, ipi = 0, inch = 0;
    const char *ia = nullptr, *ib = nullptr;   // token row of chunk ic in each operand
    int64_t irem = 0;                          // token rows of the item from chunk ic on
    int64_t lda = 0, ldb = 0;                  // bytes per token row of the item's operands
    DmaTok da, db;
    int tcx = 0, tcy = 0;                      // features of the item's X / dY panel inside M / N
    bool iv = g_item(ga, 0, ipi, itm, itn, isp);
    auto set_itile = [&]() __attribute__((always_inline)) {
        const GemmArgs &ig = ga.p[ipi];
        lda = (int64_t)ig.in * ES;
        ldb = (int64_t)ig.out * ES;
        int64_t ikbeg = 0, iklen = 0;
        inch = item_chunks(ipi, isp, ikbeg, iklen);
        irem = iv ? iklen : 0;
        ia = (const char *)ig.act0 + ikbeg * lda + (int64_t)itm * 256 * ES;
        ib = (const char *)ig.act1 + ikbeg * ldb + (int64_t)itn * 256 * ES;
        da.init(lda, ig.M - itm * 256, wave);
        db.init(ldb, ig.N - itn * 256, wave);
        tcx = ig.M - itm * 256;
        tcy = ig.N - itn * 256;
    };
    set_itile();
    // record count of rows bytes (rows of ld bytes), saturated to the 31-bit range
    auto nrec = [&](int64_t rows, int64_t ld) __attribute__((always_inline)) {
        const int64_t b = rows * ld;
        return __builtin_amdgcn_readfirstlane((uint32_t)(b <= 0 ? 0 : (b > 0x7FFFFFF0 ? 0x7FFFFFF0 : b)));
    };
    // ---- compute side: item cj (problem cpi)
    int cj = 0, ctm = 0, ctn = 0, csp = 0, cpi = 0;
    int64_t ckbeg = 0, cklen = 0;
    bool cv = g_item(ga, 0, cpi, ctm, ctn, csp);
    int cnch = cv ? item_chunks(cpi, csp, ckbeg, cklen) : 0;

    f32x16 acc[4][4];
    u32x4 f0a[2][4], f0b[2][4];   // K quarter 0 fragments of the current / next chunk
    uint32_t tq[2][2] = {{0u, 0u}, {0u, 0u}}, tsink = 0u;   // warm-up loads per chunk slot
    int sc = 0;                   // LDS stage of the current chunk

    auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int fm = 0; fm < 4; fm++)
#pragma unroll
            for (int fn = 0; fn < 4; fn++)
#pragma unroll
                for (int i = 0; i < 16; i++) acc[fm][fn][i] = 0.0f;
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    // the issue side's step to the next chunk (and item)
    auto next_chunk = [&]() __attribute__((always_inline)) {
        ia += W_KC * lda;
        ib += W_KC * ldb;
        irem -= W_KC;
        if (++ic == inch) {
            ic = 0;
            if (iv) {
                ++ij;
                iv = g_item(ga, ij, ipi, itm, itn, isp);
                set_itile();
            }
        }
    };
    // The 16 MFMAs of the last K quarter with the X half of the refill of
    // stage s with the chunk after the next (one load per two MFMAs) and, after
    // each MFMA, one of the next chunk's quarter-0 reads.
    auto p_mma_dma16 = [&](const u32x4 (&a)[4], const u32x4 (&b)[4], int s) __attribute__((always_inline)) {
        char *st = w_lds + s * W_STAGE;
        const __amdgpu_buffer_rsrc_t ra = make_rsrc_n(ia, nrec(irem, lda));
        auto one = [&](auto k_c) __attribute__((always_inline)) {
            constexpr int K = decltype(k_c)::value;
            constexpr int i = K >> 2, j = K & 3;
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[i]),
                                                                __builtin_bit_cast(bf16x8, b[j]), acc[i][j], 0, 0, 0);
            if constexpr (K % 2 == 1) da.template issue<K / 2>(ra, st, wave);
        };
        one(std::integral_constant<int, 0>{}); one(std::integral_constant<int, 1>{});
        one(std::integral_constant<int, 2>{}); one(std::integral_constant<int, 3>{});
        one(std::integral_constant<int, 4>{}); one(std::integral_constant<int, 5>{});
        one(std::integral_constant<int, 6>{}); one(std::integral_constant<int, 7>{});
        one(std::integral_constant<int, 8>{}); one(std::integral_constant<int, 9>{});
        one(std::integral_constant<int, 10>{}); one(std::integral_constant<int, 11>{});
        one(std::integral_constant<int, 12>{}); one(std::integral_constant<int, 13>{});
        one(std::integral_constant<int, 14>{}); one(std::integral_constant<int, 15>{});
        // each MFMA followed by one of the next chunk's 16 quarter-0
        // transposing reads (issued just before this call), every second one
        // also by a refill load
#pragma unroll
        for (int k = 0; k < 16; k++) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (k % 2 == 1) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    // first K quarter of a chunk: its 16 MFMAs with the dY half of the refill
    // begun in the previous chunk's last quarter (stage sc ^ 1, one load per
    // two MFMAs), then the issue side's step to the next chunk
    auto p_mma_dmab = [&](const u32x4 (&a)[4], const u32x4 (&b)[4], uint32_t &t0, uint32_t &t1)
                          __attribute__((always_inline)) {
        char *st = w_lds + (sc ^ 1) * W_STAGE;
        const __amdgpu_buffer_rsrc_t rb = make_rsrc_n(ib, nrec(irem, ldb));
        auto one = [&](auto k_c) __attribute__((always_inline)) {
            constexpr int K = decltype(k_c)::value;
            constexpr int i = K >> 2, j = K & 3;
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[i]),
                                                                __builtin_bit_cast(bf16x8, b[j]), acc[i][j], 0, 0, 0);
            if constexpr (K % 2 == 1) db.template issue<K / 2>(rb, st + W_OP, wave);
        };
        one(std::integral_constant<int, 0>{});
        one(std::integral_constant<int, 1>{});
        one(std::integral_constant<int, 2>{});
        one(std::integral_constant<int, 3>{});
        one(std::integral_constant<int, 4>{});
        one(std::integral_constant<int, 5>{});
        one(std::integral_constant<int, 6>{});
        one(std::integral_constant<int, 7>{});
        one(std::integral_constant<int, 8>{});
        one(std::integral_constant<int, 9>{});
        one(std::integral_constant<int, 10>{});
        one(std::integral_constant<int, 11>{});
        one(std::integral_constant<int, 12>{});
        one(std::integral_constant<int, 13>{});
        one(std::integral_constant<int, 14>{});
        one(std::integral_constant<int, 15>{});
#pragma unroll
        for (int k = 0; k < 16; k++) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (k % 2 == 1) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        {
            // L2 warm-up of the chunk three beyond the one whose refill this
            // quarter finishes: one 4-byte load per 128-byte line of its X and
            // dY rows (lane: row 16 wave + lane / 4, line lane % 4).  Its L2
            // misses, a fifth of the lines, are what the barrier waited on:
            // their latency now runs under about two chunks of MFMAs, and its
            // refill finds the lines in L2.  Lanes past the panel's columns and
            // rows past the item read nothing (out-of-range offset, record
            // counts of the remaining rows); the values go to a sink.
            const int trow = wave * 16 + (lane >> 2), tcol = (lane & 3) * 128;
            constexpr int64_t AHEAD = 3 * W_KC;
            const __amdgpu_buffer_rsrc_t tx = make_rsrc_n(ia + AHEAD * lda, nrec(irem - AHEAD, lda));
            const __amdgpu_buffer_rsrc_t ty = make_rsrc_n(ib + AHEAD * ldb, nrec(irem - AHEAD, ldb));
            const uint32_t ox = tcol < 2 * tcx ? (uint32_t)(trow * lda + tcol) : OOB;
            const uint32_t oy = tcol < 2 * tcy ? (uint32_t)(trow * ldb + tcol) : OOB;
            t0 = __builtin_amdgcn_raw_buffer_load_b32(tx, ox, 0, 0);
            t1 = __builtin_amdgcn_raw_buffer_load_b32(ty, oy, 0, 0);
        }
        next_chunk();
    };

    // one chunk (fragment slot SL): run K quarters 0 .. W_Q - 2, reading each
    // next quarter's fragments during the current one's MFMAs (quarter 0 also
    // issues the dY half of the previous chunk's refill and the warm-up loads);
    // wait for the next chunk's loads in every wave (only the two warm-up
    // loads were issued after them), pass the
    // barrier, start the refill of this chunk's stage, read the next chunk's
    // quarter 0 fragments, and run the last quarter's MFMAs (its fragments are
    // already in registers).
    auto chunk = [&](auto sl_c) __attribute__((always_inline)) {
        constexpr int SL = decltype(sl_c)::value, SL1 = SL ^ 1;
        const char *st = w_lds + sc * W_STAGE;
        u32x4 qa[2][4], qb[2][4];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < W_Q - 1; q++) {
            w_read_q(st, qa[(q + 1) & 1], qb[(q + 1) & 1], wm, wn, lane, q + 1);
            if (q == 0) {
                p_mma_dmab(f0a[SL], f0b[SL], tq[SL][0], tq[SL][1]);
            } else {
                p_mma(acc, qa[q & 1], qb[q & 1]);
                // one MFMA, then one of the next quarter's 16 transposing reads:
                // the reads issue in the MFMAs' shadow instead of as a burst
#pragma unroll
                for (int i = 0; i < 16; i++) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // all but the two warm-up loads issued last
        w_barrier<2>();
        // the previous chunk's warm-up loads are older than this barrier's
        // wait: folding them costs no wait
        tsink ^= tq[SL1][0] ^ tq[SL1][1];
        // every wave has read all of this chunk's stage: its refill with the
        // chunk after the next one starts during the last quarter (the X half)
        const int sfree = sc;
        sc ^= 1;
        w_read_q(w_lds + sc * W_STAGE, f0a[SL1], f0b[SL1], wm, wn, lane, 0);
        p_mma_dma16(qa[(W_Q - 1) & 1], qb[(W_Q - 1) & 1], sfree);
        __builtin_amdgcn_sched_barrier(0);
    };

    // prologue: chunk 0 and the X half of chunk 1 in flight; the first one's
    // quarter 0 fragments
    auto issue_all = [&](int s) __attribute__((always_inline)) {
        char *st = w_lds + s * W_STAGE;
        const __amdgpu_buffer_rsrc_t ra = make_rsrc_n(ia, nrec(irem, lda)), rb = make_rsrc_n(ib, nrec(irem, ldb));
        da.template issue<0>(ra, st, wave);
        da.template issue<1>(ra, st, wave);
        da.template issue<2>(ra, st, wave);
        da.template issue<3>(ra, st, wave);
        da.template issue<4>(ra, st, wave);
        da.template issue<5>(ra, st, wave);
        da.template issue<6>(ra, st, wave);
        da.template issue<7>(ra, st, wave);
        db.template issue<0>(rb, st + W_OP, wave);
        db.template issue<1>(rb, st + W_OP, wave);
        db.template issue<2>(rb, st + W_OP, wave);
        db.template issue<3>(rb, st + W_OP, wave);
        db.template issue<4>(rb, st + W_OP, wave);
        db.template issue<5>(rb, st + W_OP, wave);
        db.template issue<6>(rb, st + W_OP, wave);
        db.template issue<7>(rb, st + W_OP, wave);
        next_chunk();
    };
    issue_all(0);
    {   // A half of chunk 1; its B half goes out in chunk 0's first quarter
        char *st = w_lds + W_STAGE;
        const __amdgpu_buffer_rsrc_t ra = make_rsrc_n(ia, nrec(irem, lda));
        da.template issue<0>(ra, st, wave);
        da.template issue<1>(ra, st, wave);
        da.template issue<2>(ra, st, wave);
        da.template issue<3>(ra, st, wave);
        da.template issue<4>(ra, st, wave);
        da.template issue<5>(ra, st, wave);
        da.template issue<6>(ra, st, wave);
        da.template issue<7>(ra, st, wave);
    }
    w_barrier<W_DR>();
    w_read_q(w_lds, f0a[0], f0b[0], wm, wn, lane, 0);
    zero_acc();
    while (cv) {
        for (int c = 0; c < cnch; c += 2) {
            chunk(I0{});
            chunk(I1{});
        }
        // ---- epilogue of item (ctm, ctn, csp).  acc[fm][fn][i] is C[m][n] with
        //   m = m0 + wm*128 + fm*32 + 8*(i/4) + 4*h + i%4,  n = n0 + wn*128 + fn*32 + l32
        const GemmArgs &g = ga.p[cpi];
        const int mw = ctm * 256 + wm * 128, nw = ctn * 256 + wn * 128;
        // buffer stores over this wave's 128 x 128 block: the lane offset holds
        // its column and 4h rows, the scalar offset the row group.  M is a
        // multiple of 8, so the 8-row test is wave-uniform.
        float *dst = (float *)g.out_ptr + (g.splits > 1 ? (int64_t)csp * g.M * g.N : 0);
        const __amdgpu_buffer_rsrc_t ro = make_rsrc(dst + (int64_t)mw * g.N + nw);
        uint32_t vo[4];
#pragma unroll
        for (int fn = 0; fn < 4; fn++)
            vo[fn] = nw + fn * 32 + l32 < g.N ? (uint32_t)((4 * h * g.N + fn * 32 + l32) * 4) : OOB;
        // One split: gq = G * scale[c] and the sgrad partial.  Several splits,
        // or accumulation: the raw G partial (scale 1 makes the store exact),
        // no sgrad partial; dw_reduce_kernel finishes gq and the partials.
        const bool split = g.splits > 1 || g.acc;
        // tern values of this lane's 64 rows x 4 columns, from the forward
        // fragment-ordered copy (its rows are the columns c, its K the rows r):
        // per 32-row fragment fm, the 16 bytes of each 8-row half hf hold the
        // lane's four columns.  Pre-shifted by 16h, row 8 (i / 4) + 4h + i % 4
        // of the fragment sits in nibble i % 4, at bits 1 and 3 (rows 0-15)
        // or 0 and 2 (rows 16-31).
        const int nchf = (g.M + 31) >> 5;
        u32x4 tw[4][2];
#pragma unroll
        for (int fm = 0; fm < 4; fm++) {
            const int sch = ctm * 8 + wm * 4 + fm;
#pragma unroll
            for (int hf = 0; hf < 2; hf++) {
                const u32x4 z = {0u, 0u, 0u, 0u};
                tw[fm][hf] = (!split && sch < nchf)
                                 ? *(const u32x4 *)(g.frag + ((int64_t)(ctn * nchf + sch) * 512 +
                                                              (wn * 64 + hf * 32 + l32) * 4))
                                 : z;
                tw[fm][hf] >>= (uint32_t)(16 * h);
            }
        }
        float scv[4], ps[4];
#pragma unroll
        for (int fn = 0; fn < 4; fn++) {
            const int n = nw + fn * 32 + l32;
            scv[fn] = split ? 1.0f : (n < g.N ? g.scale[n] : 0.0f);
            ps[fn] = 0.0f;
        }
#pragma unroll
        for (int fm = 0; fm < 4; fm++)
#pragma unroll
            for (int i = 0; i < 16; i++) {
                const int rg = fm * 32 + 8 * (i >> 2);   // row group within the block
                if (mw + rg >= g.M) continue;
                const int so = (rg + (i & 3)) * g.N * 4;
                // k = 16 kk + 8 hf + e within the fragment, e = 4h + i % 4
                const int kk = i >> 3, hf = (i >> 2) & 1;
                const int pos = 4 * (i & 3) + 1 - kk;   // nonzero bit; the sign bit is 2 above
#pragma unroll
                for (int fn = 0; fn < 4; fn++) {
                    const float gv = acc[fm][fn][i];
                    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, gv * scv[fn]), ro, vo[fn], so,
                                                          0);
                    const uint32_t b = tw[fm][hf][fn] >> pos;
                    ps[fn] += gv * code_to_f32((b & 1u) | ((b >> 1) & 2u));
                }
            }
        if (!split) {
#pragma unroll
            for (int fn = 0; fn < 4; fn++) ps[fn] += __shfl_xor(ps[fn], 32);
            // cross-wave sum (the tile's two row halves) through a table of its own
            if (h == 0) {
#pragma unroll
                for (int fn = 0; fn < 4; fn++) w_red[wm * 256 + wn * 128 + fn * 32 + l32] = ps[fn];
            }
            __syncthreads();
            const int n0 = ctn * 256;
            if (tid < 256 && n0 + tid < g.N) g.part[(int64_t)ctm * g.N + n0 + tid] = w_red[tid] + w_red[256 + tid];
            __syncthreads();
        }
        zero_acc();
        ++cj;
        cv = g_item(ga, cj, cpi, ctm, ctn, csp);
        if (cv) cnch = item_chunks(cpi, csp, ckbeg, cklen);
    }
    // the last issues were out-of-range loads still writing zeros into the
    // stages: drain them before the workgroup ends
    wait_vm0();
    // the warm-up values are never used; a store under a condition the
    // compiler cannot decide (no group has a negative count) keeps the loads
    tsink ^= tq[0][0] ^ tq[0][1] ^ tq[1][0] ^ tq[1][1];
    if (ga.n < 0) ga.p[0].part[threadIdx.x] = __builtin_bit_cast(float, tsink);
}

// ---------------------------------------------------------------------------
// Fragment-ordered copies of the packed ternary matrix, read by the forward
// and dX GEMMs below.  View the operand as A[m][k] (forward: m = c, k = r;
// dX: m = r, k = c) in tiles of 256 rows and chunks of 32 K.  The 512 words of
// (tile, chunk) are ordered (wm, lane, fm): wm = 128-row half, lane = lane of
// the wave, fm = 32-row MFMA fragment, so one 16-byte load per lane brings a
// wave all four of its fragments.  Word (wm, lane, fm) holds the 16 ternary
// values of row m = 256 tile + 128 wm + 32 fm + lane % 32 at k = 32 chunk +
// 16 kk + 8 (lane / 32) + e (kk < 2, e < 8) in nibble e: bits 1 (nonzero) and
// 3 (negative) for kk = 0, bits 0 and 2 for kk = 1.  Masked with 0xAAAAAAAA
// (kk = 0) or shifted left by one and masked (kk = 1), a word is eight fp4
// (e2m1) values 0, +1.0 (0x2) or -1.0 (0xA), and byte j converts to the bf16
// pair of MFMA operand dword j in one instruction.  Values beyond the matrix
// are 0.
// ---------------------------------------------------------------------------
// 16 int8 of row r of q from column 16 wc (fewer at a ragged row end) ->
// one canonical word: code of column 16 wc + j at bits 2j, 01 = +1 (q >= theta),
// 11 = -1 (q <= -theta), 00 otherwise.  VEC: the 16 bytes are one aligned load.
template <bool VEC>
__device__ __forceinline__ uint32_t tern_word(const int8_t *__restrict__ q, int64_t out, int theta, int64_t r,
                                              int64_t wc) {
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
    return word;
}

// One workgroup writes D_G chunks of one tile of a copy.  It first builds, in
// LDS, the canonical words of the block of q it needs: for the dX operand, the
// tile's 256 rows m = r x the chunks' 2 D_G words of columns k = c; for the
// forward operand, the chunks' 32 D_G rows k = r x the tile's 16 words of
// columns m = c.
constexpr int D_G = 2;   // chunks per workgroup
constexpr int D_LDS = 256 * (2 * D_G + 1);   // words of the larger block (+1 word per row)
template <bool VEC, bool DXOP>
__device__ __forceinline__ void derive_block(const int8_t *__restrict__ q, int64_t in, int64_t out, int64_t wpr,
                                             int theta, int64_t nch, int64_t tile, int64_t sg,
                                             uint32_t *__restrict__ frag, uint32_t *blk) {
    // block rows x words (+1 word per row against bank conflicts)
    constexpr int BR = DXOP ? 256 : 32 * D_G, BW = DXOP ? 2 * D_G : 16, LD = BW + 1;
    static_assert(BR * LD <= D_LDS, "block does not fit");
    const int t = threadIdx.x;
    const int64_t r0 = DXOP ? tile * 256 : sg * (32 * D_G);   // first row of q
    const int64_t w0 = DXOP ? sg * (2 * D_G) : tile * 16;     // first word column
#pragma unroll
    for (int idx = t; idx < BR * BW; idx += 256) {
        const int row = idx / BW, w = idx % BW;
        const int64_t r = r0 + row, wc = w0 + w;
        blk[row * LD + w] = (r < in && wc < wpr) ? tern_word<VEC>(q, out, theta, r, wc) : 0u;
    }
    __syncthreads();
    const int64_t M = DXOP ? in : out;
#pragma unroll
    for (int o = t; o < 512 * D_G; o += 256) {
        const int sl = o >> 9, d = o & 511;            // chunk within the group, word within the chunk
        const int64_t chunk = sg * D_G + sl;
        if (chunk >= nch) continue;
        const int wm = d >> 8, lane = (d >> 2) & 63, fm = d & 3;
        const int ml = wm * 128 + fm * 32 + (lane & 31);  // row within the tile
        uint32_t word = 0;
        if (tile * 256 + ml < M) {
#pragma unroll
            for (int kk = 0; kk < 2; kk++) {
                const int k0 = sl * 32 + kk * 16 + (lane >> 5) * 8;   // first of the word's 8 k in the group
                uint32_t x;   // code of k0 + e at bits 4e and 4e + 1
                if constexpr (DXOP) {
                    // the 8 codes are adjacent in one canonical word of row ml
                    // (k0 % 16 is 0 or 8): spread 2-bit groups to nibbles
                    x = (blk[ml * LD + (k0 >> 4)] >> (2 * (k0 & 15))) & 0xFFFFu;
                    x = (x | (x << 8)) & 0x00FF00FFu;
                    x = (x | (x << 4)) & 0x0F0F0F0Fu;
                    x = (x | (x << 2)) & 0x33333333u;
                } else {
                    // column ml of 8 consecutive rows
                    const uint32_t *col = blk + k0 * LD + (ml >> 4);
                    const int sh = 2 * (ml & 15);
                    x = 0u;
#pragma unroll
                    for (int e = 0; e < 8; e++) x |= ((col[e * LD] >> sh) & 3u) << (4 * e);
                }
                // nonzero flag (bit 0 of a code) to bit 1 of the nibble, sign (bit 1,
                // when nonzero) to bit 3; one lower for the second K half.  Rows and
                // columns past the matrix are zero words in the block.
                const uint32_t nz = x & 0x11111111u, neg = (x >> 1) & nz;
                word |= ((nz << 1) | (neg << 3)) >> kk;
            }
        }
        frag[(tile * nch + chunk) * 512 + d] = word;
    }
}

// ---------------------------------------------------------------------------
// Forward and dX GEMM (bf16, persistent; 512 x 128 tiles, the accumulating
// dX 256 x 256).  Each wave computes its 128 x 128 block:
//   * its 128 activation rows (X or dY) stream into a ring of four LDS stages,
//     32 K per chunk, with direct-to-LDS buffer loads issued three chunks
//     ahead, together with the wave's fragment words of the chunk (and, for dX,
//     the chunk's 32 scales).  In a 512 x 128 tile all four waves read the
//     same rows: they share the stages and each loads a quarter of them;
//   * the ternary operand is decoded from the fragment words straight into
//     MFMA operand registers: never staged as bf16;
//   * each wave waits on its own loads (vmcnt); one workgroup barrier per
//     chunk, right after that wait, makes the partner's half visible and, as
//     every wave has finished reading the previous chunk's stage by then, frees
//     that stage for the refill issued in the next chunk.
// The two waves that share fragment words load them from L1.  The forward
// epilogue multiplies by scale[c] (staged in LDS when the tile starts); the dX
// operand carries +-bf16(scale[c]).  The accumulating dX keeps a private ring
// per wave and no barrier (its epilogue transposes through a free stage).
// ---------------------------------------------------------------------------
constexpr int R_KC = 32;                         // K per chunk
constexpr int R_NST = 4;                         // LDS stages per wave
constexpr int R_B = 128 * 64;                    // activation rows of a stage: 128 x 64 bytes
constexpr int R_A = 1024;                        // fragment words of a stage: 64 lanes x 16 bytes
constexpr int R_S = 256;                         // dX scales of a stage (one 4-byte DMA: 64 x 4 bytes)
constexpr int R_STAGE = R_B + R_A + R_S;         // 9472
constexpr int R_ESC = 4 * 512;                   // forward: scales of four tiles x 128 rows
constexpr int R_WAVE = R_NST * R_STAGE + R_ESC;  // 39936
// Shared layouts (the swapped kernels).  Wide: a 512 x 128 tile (columns x
// tokens), the four waves side by side along the columns, all reading the
// same 128 activation rows from one shared ring of stages, each wave loading
// 32 of the rows.  Pairs: a 256 x 256 tile, 2 x 2 waves; the two waves that
// read the same 128 rows share a ring, each loading 64 of them.  Fragment
// words, dX scales and the epilogue's scales stay per wave.
constexpr int R_PS = R_A + R_S;                      // per-wave part of a stage
constexpr int R_SH_WAVE = R_NST * R_PS + R_ESC;      // 7168
static_assert(2 * R_NST * R_B + 4 * R_SH_WAVE <= 4 * R_WAVE, "shared layouts fit the LDS array");
__shared__ __attribute__((aligned(16))) char r_lds[4 * R_WAVE];

__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t rs, void *lds_wave_base, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void *)lds_wave_base, 4, voff, 0, 0, 0);
}

// Wait until at most N vector memory operations of this wave are outstanding
// (and fence the compiler on both sides).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt is six bits");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
    __builtin_amdgcn_sched_barrier(0);
}

// Stage rows are 64 bytes (32 K); the 16-byte chunk c of row r sits in slot
// c ^ ((r / 4) % 4), which makes the 16 rows read by 16 lanes of a fragment
// load hit 16 different slots of a 256-byte bank window.
__device__ __forceinline__ void r_read_b(const char *st, u32x4 (&b)[4], int l32, int h, int kk) {
    const int ps = (2 * kk + h) ^ ((l32 >> 2) & 3);
#pragma unroll
    for (int f = 0; f < 4; f++) b[f] = *(const u32x4 *)(st + (f * 32 + l32) * 64 + ps * 16);
}

// Byte J of x (two fp4 e2m1 values, low nibble first) -> two bf16 values in
// one dword (the scale operand 1.0 leaves them unscaled).
template <int J>
__device__ __forceinline__ uint32_t fp4_pair_bf16(uint32_t x) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, 1.0f, J));
}
__device__ __forceinline__ uint32_t fp4_pair_bf16(uint32_t x, int j) {
    switch (j) {   // j is a constant wherever this is inlined
    case 0: return fp4_pair_bf16<0>(x);
    case 1: return fp4_pair_bf16<1>(x);
    case 2: return fp4_pair_bf16<2>(x);
    default: return fp4_pair_bf16<3>(x);
    }
}

// A bf16 pair v of ternary values (0x0000, 0x3F80 = +1 or 0xBF80 = -1 per
// half) times a pair of bf16 scales: q is the scale pair XOR 0x3F803F80.  v ^ q
// is the scale where v = +1 and its negation where v = -1; the mask comes from
// a byte permute with v as the selector (selector bytes 0x80, 0x3F and 0xBF
// give 0xFF, selector 0 picks the zero byte of the second source), so zero
// halves stay zero.
__device__ __forceinline__ uint32_t r_scaled_pair(uint32_t v, uint32_t q) {
    return (v ^ q) & __builtin_amdgcn_perm(0u, 0u, v);
}

// YBF: bf16 Y (forward only; every problem of a launch has the same Y type).
// WIDE: 512 x 128 tiles, else 256 x 256 (the accumulating dX: always).
template <int MODE, bool ACC = false, bool YBF = false, bool WIDE = true>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_rd_kernel(GroupArgs ga) {
    static_assert(MODE == MODE_FWD || MODE == MODE_DX, "forward and dX only");
    static_assert(!ACC || MODE == MODE_DX, "accumulation is a dX variant");
    static_assert(!YBF || MODE == MODE_FWD, "bf16 output is a forward variant");
    // operands swapped in the MFMAs (transposed accumulators, epilogue below)
    constexpr bool SWAP = !ACC;
    constexpr int ES = 2;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    // SHARE: the swapped kernels share their activation stages (one
    // workgroup barrier per chunk orders the loaders' parts): WIDE, 512 x 128
    // tiles whose four waves share one ring; else 256 x 256 tiles (2 x 2 waves
    // of 128 x 128) whose wave pairs with the same rows share a ring.  The
    // accumulating dX runs 256 x 256 tiles with private stages (its epilogue
    // transposes through a free stage).  wm: the wave's 128 columns, wn: its
    // 128 tokens.
    constexpr bool SHARE = SWAP;
    constexpr bool W4 = SHARE && WIDE;
    constexpr int TM = W4 ? 512 : 256, TN = W4 ? 128 : 256;   // tile: columns x tokens
    const int wm = W4 ? wave : wave >> 1, wn = W4 ? 0 : wave & 1, l32 = lane & 31, h = lane >> 5;
    char *wl = r_lds + wave * R_WAVE;
    constexpr int SH_ACT = (W4 ? 1 : 2) * R_NST * R_B;   // the shared rings
    char *const a_base = !SHARE ? wl : r_lds + wn * (R_NST * R_B);    // activation rows of stage 0
    constexpr int A_STRIDE = SHARE ? R_B : R_STAGE;
    char *const p_base = SHARE ? r_lds + SH_ACT + wave * R_SH_WAVE : wl + R_B;   // fragment words of stage 0
    constexpr int P_STRIDE = SHARE ? R_PS : R_STAGE;
    char *const e_base = SHARE ? r_lds + SH_ACT + wave * R_SH_WAVE + R_NST * R_PS : wl + R_NST * R_STAGE;
    // activation loads of this wave per chunk, and its first row in the stage
    constexpr int NACT = !SHARE ? 8 : W4 ? 2 : 4;
    const int arow0 = !SHARE ? 0 : W4 ? 32 * wave : 64 * wm;
    // vector memory operations per chunk issue: the activation loads + 1
    // fragment (+ 1 scale)
    constexpr int OPS = NACT + (MODE == MODE_DX ? 2 : 1);
    // slot of this lane's 16 bytes in every DMA row group, and its logical chunk
    const int cb = ((lane & 3) ^ ((lane >> 4) & 3)) * 16;

    // ---- issue side: chunk ic of tile ij (coordinates itm, itn).  Each tile
    // gets three buffer resources whose record counts end at the operand's
    // last byte: this wave's activation rows (to the end of the tensor), its
    // fragment words of the tile, and (dX) the scales.  A chunk only moves the
    // scalar offsets.  The range check covers vector + scalar + immediate
    // offsets per lane, so every byte past an edge reads as zero: the ragged
    // K end of the tensor's last row, the even-padding chunk of the fragment
    // words, and (record counts 0) every issue after the last tile.  Inside
    // the tensor, bytes past K belong to the next row: in a chunk that reaches
    // past K, the lanes whose 16 bytes lie there get an out-of-range offset
    // (a wave-uniform test, taken only in such chunks).  Four activation loads share
    // one M0: the immediate offset 1024 i moves the LDS destination and the
    // global address alike, and the lane offsets are stored less 1024 i
    // (which needs K >= 32: 16 rows of 2 K bytes span 1024 bytes).
    int ij = 0, ic = 0, itm = 0, itn = 0, isp = 0, ipi = 0;
    bool iv = g_item(ga, 0, ipi, itm, itn, isp);
    int i_nch2 = 0;             // chunks per tile of the issue side's problem, padded to even
    int ld32 = 0;               // bytes per activation row of that problem (K <= 2^20)
    const float *i_scale = nullptr;   // its scales
    const char *pa = nullptr;   // activation rows of tile ij (this wave's first row)
    const uint32_t *pf = nullptr;   // this wave's fragment words of tile ij
    uint32_t na = 0, nf = 0, ns = 0;   // record counts of the three resources
    uint32_t boff[8];   // activation load i: lane's row * ld + 16-byte column - 1024 (i % 4), or OOB
    const uint32_t soff_lane = lane < 32 ? (uint32_t)lane * 4u : OOB;   // dX scales: 32 per chunk
    auto set_itile = [&]() __attribute__((always_inline)) {
        const GemmArgs &g = ga.p[ipi];
        const int nch = g.nch;
        i_nch2 = (nch + 1) & ~1;
        const int64_t ld = (int64_t)g.K * ES;
        ld32 = g.K * ES;
        i_scale = g.scale;
        const int n0 = itn * TN + wn * 128;
        // bytes from this wave's first row to the end of the tensor (integer
        // arithmetic only: the int64 min / max overloads go through f64)
        int64_t rem = (int64_t)(g.N - n0) * ld;
        rem = (!iv || rem < 0) ? 0 : (rem > 0x7FFFFFF0 ? 0x7FFFFFF0 : rem);
        pa = (const char *)g.act0 + (int64_t)n0 * ld;
        na = __builtin_amdgcn_readfirstlane((uint32_t)rem);
        // the fragment copy is cut in 256-column tiles: this wave's 128
        // columns are half hf of tile ft, which exists if it starts below M
        const int ft = (itm * TM + wm * 128) >> 8, hf = wm & 1;
        pf = g.frag + ((int64_t)ft * nch * 512 + hf * 256);
        nf = __builtin_amdgcn_readfirstlane(iv && ft * 256 < g.M ? (uint32_t)(nch * 2048 - 1024) : 0u);
#pragma unroll
        for (int i = 0; i < NACT; i++) {
            const int row = arow0 + 16 * i + (lane >> 2);
            boff[i] = (n0 + row < g.N ? (uint32_t)(row * ld) + (uint32_t)cb : OOB) - 1024u * (uint32_t)(i & 3);
        }
        if constexpr (MODE == MODE_DX) {
            ns = __builtin_amdgcn_readfirstlane(iv ? (uint32_t)g.K * 4u : 0u);
        } else if (iv) {
            // this wave's 128 scales of the tile, for its epilogue
            const int mb = itm * TM + wm * 128;
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(g.scale + mb);
            char *esc = e_base + (ij & 3) * 512;
#pragma unroll
            for (int q = 0; q < 2; q++)
                dma4(rs, esc + q * 256, mb + 64 * q + lane < g.M ? (uint32_t)(64 * q + lane) * 4u : OOB);
        }
    };
    set_itile();

    // Part p of the issue of chunk ic into stage s: parts 0-3 are the
    // activation loads (wide tiles: one each in parts 0 and 1, 32 rows per
    // wave; private stages: two each, 8 in all), part 4 the fragment words
    // (and, dX, the scales) and the step to the next chunk.  The chunk loop
    // spreads the parts over its first five fragments, so the texture unit
    // sees the loads between the MFMAs instead of in one burst.
    auto issue_part = [&](int s, auto p_c) __attribute__((always_inline)) {
        constexpr int P = decltype(p_c)::value;
        char *ast = a_base + s * A_STRIDE;
        char *pst = p_base + s * P_STRIDE;
        if constexpr (P < 4 && SHARE) {
            if constexpr (P >= NACT) return;   // wide tiles: parts 2 and 3 issue nothing
            // one load of 16 rows: rows arow0 + 16 P .. + 15 of the shared stage
            const __amdgpu_buffer_rsrc_t ra = make_rsrc_n(pa, na);
            const int so = ic * R_KC * ES;
            uint32_t o0 = boff[P];
            if (so + R_KC * ES > ld32) {
                // a chunk reaching past K: lanes whose 16 bytes lie past K load nothing
                if (so + cb >= ld32) o0 = OOB - 1024u * (uint32_t)P;
            }
            dma16_imm<P * 1024>(ra, ast + arow0 * 64, o0, so);
        } else if constexpr (P < 4) {
            const __amdgpu_buffer_rsrc_t ra = make_rsrc_n(pa, na);
            const int so = ic * R_KC * ES;
            char *d = ast + (P >> 1) * 4096;
            uint32_t o0 = boff[2 * P], o1 = boff[2 * P + 1];
            if (so + R_KC * ES > ld32) {
                // a chunk reaching past K (the ragged last one or the padding
                // one): a lane whose 16 bytes lie past K loads nothing, so no
                // byte of the next token row meets the zero ternary codes (a
                // non-finite value there would turn the sum into NaN)
                if (so + cb >= ld32) {
                    o0 = OOB - 1024u * (uint32_t)((2 * P) & 3);
                    o1 = OOB - 1024u * (uint32_t)((2 * P + 1) & 3);
                }
            }
            dma16_imm<(P & 1) * 2048>(ra, d, o0, so);
            dma16_imm<(P & 1) * 2048 + 1024>(ra, d, o1, so);
        } else {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc_n(pf, nf), (LDS_AS void *)pst, 16,
                                                     (uint32_t)lane * 16u, ic * 2048, 0, 0);
            if constexpr (MODE == MODE_DX)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc_n(i_scale, ns), (LDS_AS void *)(pst + R_A), 4,
                                                         soff_lane, ic * R_KC * 4, 0, 0);
            if (++ic == i_nch2) {
                ic = 0;
                if (iv) {
                    ++ij;
                    iv = g_item(ga, ij, ipi, itm, itn, isp);
                    set_itile();
                }
            }
        }
    };
    auto issue = [&](int s) __attribute__((always_inline)) {
        issue_part(s, std::integral_constant<int, 0>{});
        issue_part(s, std::integral_constant<int, 1>{});
        issue_part(s, std::integral_constant<int, 2>{});
        issue_part(s, std::integral_constant<int, 3>{});
        issue_part(s, std::integral_constant<int, 4>{});
    };

    // ---- compute side: tile cj (problem cpi)
    int cj = 0, ctm = 0, ctn = 0, csp = 0, cpi = 0;
    bool cv = g_item(ga, 0, cpi, ctm, ctn, csp);
    int c_nch2 = cv ? (ga.p[cpi].nch + 1) & ~1 : 0;
    int hist = 0;   // bit 0: this chunk is one of a tile's first two after an epilogue

    f32x16 acc[4][4];
    u32x4 fa[2];        // fragment words (one dword per fm) of the current / next chunk
    u32x4 fb0[2][4];    // activation fragments, K quarter 0, of the current / next chunk
    u32x4 fb1[4];       // K quarter 1 of the current chunk
    uint32_t p4[2][8];  // dX: bf16 scale pairs ^ 0x3F803F80 of the current / next chunk

    auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int fm = 0; fm < 4; fm++)
#pragma unroll
            for (int fn = 0; fn < 4; fn++)
#pragma unroll
                for (int i = 0; i < 16; i++) acc[fm][fn][i] = 0.0f;
    };

    // fragment words, quarter-0 activation fragments and scales of stage S
    auto read_ahead = [&](int s, auto sl_c) __attribute__((always_inline)) {
        constexpr int SL = decltype(sl_c)::value;
        const char *pst = p_base + s * P_STRIDE;
        fa[SL] = *(const u32x4 *)(pst + lane * 16);
        r_read_b(a_base + s * A_STRIDE, fb0[SL], l32, h, 0);
        if constexpr (MODE == MODE_DX) {
            const float *sc = (const float *)(pst + R_A);
#pragma unroll
            for (int kk = 0; kk < 2; kk++) {
                const f32x4 lo = *(const f32x4 *)(sc + 16 * kk + 8 * h);
                const f32x4 hi = *(const f32x4 *)(sc + 16 * kk + 8 * h + 4);
                const f32x2 v0 = {lo.x, lo.y}, v1 = {lo.z, lo.w}, v2 = {hi.x, hi.y}, v3 = {hi.z, hi.w};
                p4[SL][4 * kk + 0] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v0, bf16x2)) ^ 0x3F803F80u;
                p4[SL][4 * kk + 1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v1, bf16x2)) ^ 0x3F803F80u;
                p4[SL][4 * kk + 2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v2, bf16x2)) ^ 0x3F803F80u;
                p4[SL][4 * kk + 3] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v3, bf16x2)) ^ 0x3F803F80u;
            }
        }
    };

    // dword j of decoded fragment f (K quarter f / 4, rows fm = f % 4) of
    // fragment words w4: the quarter's fp4 values (bits 1 and 3 of each
    // nibble) converted, times the dX scales
    auto dec = [&](const u32x4 &w4, const uint32_t (&pp)[8], int f, int j) __attribute__((always_inline)) {
        const int kk = f >> 2, fm = f & 3;
        const uint32_t x = (kk ? w4[fm] << 1 : w4[fm]) & 0xAAAAAAAAu;
        const uint32_t v = fp4_pair_bf16(x, j);
        if constexpr (MODE == MODE_FWD) return v;
        else return r_scaled_pair(v, pp[4 * kk + j]);
    };
    constexpr int DEC_OPS = MODE == MODE_FWD ? 2 : 5;   // VALU per decoded dword (with the masks)
    u32x4 acur;   // decoded fragment whose MFMAs come next (carried across chunks)

    int sc = 0;   // LDS stage of the current chunk

    // Epilogue of tile (ctm, ctn).  Every store is issued whatever the edges
    // (out-of-range stores get an out-of-range offset), so the vmcnt arithmetic
    // of the main loop holds; it counts at most 63, and any larger number of
    // stores issued after a chunk's loads only makes its wait stricter.
    //
    // The forward and the plain dX run the MFMAs with the operands swapped
    // (activations as A, ternary as B), which leaves the tile transposed in
    // the accumulators: acc[fm][fn][i] is the output at token n = nw + 32 fn +
    // 8 (i / 4) + 4 h + i % 4 and column m = mw + 32 fm + l32 (same products,
    // same sums).  Then the 32 lanes of each half-wave hold 32 consecutive
    // columns of one token row, and one 4-byte store per element writes whole
    // 128-byte lines (two per instruction) straight from the registers:
    // 256 stores per wave, no LDS round trip.  They carry the non-temporal
    // hint (whole lines, read by a later kernel, so they need not displace the
    // operand panels in L2).  bf16 Y: 2-byte stores, 64-byte halves of lines.
    auto epilogue = [&]() __attribute__((always_inline)) {
        const GemmArgs &g = ga.p[cpi];
        const int mw = ctm * TM + wm * 128, nw = ctn * TN + wn * 128;
        const int ldo = MODE == MODE_FWD ? g.out : g.in;
        constexpr bool obf = YBF;
        const int esz = obf ? 2 : 4;
        const __amdgpu_buffer_rsrc_t ro =
            make_rsrc((const char *)g.out_ptr + ((int64_t)nw * ldo + mw) * esz);
        const float *esc = (const float *)(e_base + (cj & 3) * 512);
        // Each lane's column test and scale once per 32-column group fm; the
        // row offsets (rows of ldo elements) in the scalar offset, computed
        // per 32-row group fn from a row pitch the compiler cannot see through
        // (an empty asm), so that it does not hoist all 64 of them at once.
        auto rows_s = [&]() __attribute__((always_inline)) {
            constexpr int EB = YBF ? 2 : 4;
            // every load issued so far (the next tile's first three chunks and
            // its scales) has landed before the first store: vmcnt counts in
            // issue order, and the next two chunks then need no wait behind
            // the 256 stores
            wait_vm<0>();
            // the explicit AGPR reads below are inline asm, which the
            // compiler's hazard tracking does not see: 24 wait states cover
            // an MFMA result read by a VALU instruction (the tile's last MFMAs
            // are far behind already)
            if constexpr (MODE == MODE_FWD) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
            float scl[4];
            uint32_t vcol[4];
            const uint32_t vb = (uint32_t)((4 * h * ldo + l32) * EB);
#pragma unroll
            for (int fm = 0; fm < 4; fm++) {
                scl[fm] = MODE == MODE_FWD ? esc[fm * 32 + l32] : 1.0f;
                vcol[fm] = mw + fm * 32 + l32 < g.M ? vb + (uint32_t)(fm * 32 * EB) : OOB;
            }
            const int rlim = g.N - nw - 4 * h;   // rows of this lane below N
#pragma unroll
            for (int fn = 0; fn < 4; fn++) {
                int pitch = ldo * EB;
                asm volatile("" : "+s"(pitch) : : "memory");
#pragma unroll
                for (int i = 0; i < 16; i++) {
                    const int row = fn * 32 + 8 * (i >> 2) + (i & 3);   // less the lane's 4 h
                    const int so = row * pitch;
                    const bool rok = row < rlim;
#pragma unroll
                    for (int fm = 0; fm < 4; fm++) {
                        const uint32_t off = rok ? vcol[fm] : OOB;
                        float v = acc[fm][fn][i];
                        if constexpr (MODE == MODE_FWD) {
                            // read the accumulator out of its AGPR here: with
                            // a VALU use in sight the allocator would move
                            // accumulators into VGPRs for the whole loop
                            float x;
                            asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(x) : "a"(v));
                            v = x * scl[fm];
                        }
                        if constexpr (YBF) {
                            const f32x2 v2 = {v, 0.0f};
                            const uint32_t w = __builtin_bit_cast(uint32_t, __builtin_convertvector(v2, bf16x2));
                            __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(w & 0xFFFFu), ro, off, so, 2);
                        } else {
                            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), ro, off, so, 2);
                        }
                    }
                }
            }
        };

        // The accumulating dX (operands in the usual order, the old values
        // added): each 32-row x 64-column piece of the
        // wave's block passes through the LDS stage the last chunk consumed
        // (free until the next chunk's first issue), transposed so that every
        // store writes 4 rows x 256 contiguous bytes (whole 128-byte lines)
        // instead of 32 rows x 32 bytes.  Lane (l32, h) holds row l32 of the
        // piece in 16-byte slots 8 (fm % 2) + 2 q + h; slot s of row t sits at
        // s ^ (t % 16), which makes both the writes and the reads free of bank
        // conflicts.  Still 64 stores per wave, in the same resource; they
        // carry the non-temporal hint (whole lines, read by a later kernel,
        // so they need not displace the operand panels in L2).
        auto rows_t = [&]() __attribute__((always_inline)) {
            char *eb = wl + ((sc + 3) & 3) * R_STAGE;
            // store offset of row t = 4 k + lane / 16 of piece (fn, fp), lane's 4 columns
            auto off_of = [&](int fn, int fp, int k) __attribute__((always_inline)) {
                const int row = fn * 32 + 4 * k + (lane >> 4), col = fp * 64 + (lane & 15) * 4;
                return nw + row < g.N && mw + col < g.M ? (uint32_t)((row * ldo + col) * 4) : OOB;
            };
            // ACC: the old values of a piece, loaded one piece ahead so that
            // their latency overlaps the previous piece's round trip
            f32x4 oldn[8];
            auto load_old = [&](int fn, int fp) __attribute__((always_inline)) {
#pragma unroll
                for (int k = 0; k < 8; k++)
                    oldn[k] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ro, off_of(fn, fp, k), 0, 0));
            };
            if constexpr (ACC) load_old(0, 0);
#pragma unroll
            for (int fn = 0; fn < 4; fn++) {
#pragma unroll
                for (int fp = 0; fp < 2; fp++) {
                    f32x4 oldc[8];
                    if constexpr (ACC) {
#pragma unroll
                        for (int k = 0; k < 8; k++) oldc[k] = oldn[k];
                        if (fn < 3 || fp == 0) load_old(fp ? fn + 1 : fn, fp ^ 1);
                    }
#pragma unroll
                    for (int f2 = 0; f2 < 2; f2++) {
                        const int fm = 2 * fp + f2;
#pragma unroll
                        for (int q = 0; q < 4; q++) {
                            f32x4 v = {acc[fm][fn][4 * q], acc[fm][fn][4 * q + 1], acc[fm][fn][4 * q + 2],
                                       acc[fm][fn][4 * q + 3]};
                            const int slot = (8 * f2 + 2 * q + h) ^ (l32 & 15);
                            *(f32x4 *)(eb + l32 * 256 + slot * 16) = v;
                        }
                    }
                    // the piece is in LDS before any lane reads another's row
                    __builtin_amdgcn_sched_barrier(0);
                    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int k = 0; k < 8; k++) {
                        const int t = 4 * k + (lane >> 4), pc = lane & 15;
                        f32x4 v = *(const f32x4 *)(eb + t * 256 + ((pc ^ (t & 15)) * 16));
                        if constexpr (ACC) v += oldc[k];   // out of range: zero
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), ro, off_of(fn, fp, k), 0,
                                                               2);
                    }
                    // every read has returned before the next piece (or the
                    // next chunk's loads) overwrites the stage
                    __builtin_amdgcn_sched_barrier(0);
                    __builtin_amdgcn_s_waitcnt(0xC07F);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        };

        if constexpr (SWAP) {
            rows_s();
        } else {
            rows_t();
        }
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;

    // one chunk (register slot SL): the eight fragments (K quarter, 32 rows) of
    // 4 MFMAs each, with the issue of the chunk three ahead spread over the
    // first five.  The next fragment is decoded one dword per MFMA while the
    // current one multiplies (the first fragment of the next chunk during the
    // last one of this chunk); halfway, wait for the next chunk's loads and
    // read its first fragments.
    auto chunk = [&](auto sl_c) __attribute__((always_inline)) {
        constexpr int SL = decltype(sl_c)::value, SL1 = SL ^ 1;
        const int sis = (sc + 3) & 3;
        r_read_b(a_base + sc * A_STRIDE, fb1, l32, h, 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int f = 0; f < 8; f++) {
            if (f < 4) {
                // f is a constant once the loop is unrolled
                if (f == 0) issue_part(sis, std::integral_constant<int, 0>{});
                if (f == 1) issue_part(sis, std::integral_constant<int, 1>{});
                if (f == 2) issue_part(sis, std::integral_constant<int, 2>{});
                if (f == 3) issue_part(sis, std::integral_constant<int, 3>{});
                __builtin_amdgcn_sched_barrier(0);
            }
            if (f == 4) {
                // loads issued after the next chunk's: the chunk two ahead
                // (OPS) and the 8 activation loads of the one three ahead.  In
                // a tile's first two chunks: SWAP, none (the epilogue waited
                // for every load before its stores, so those chunks' data is
                // in LDS and the stores can drain meanwhile); otherwise its 64
                // stores as well (where 63 waits for more than needed).
                if constexpr (SWAP) {
                    if (!hist) wait_vm<OPS + NACT>();
                } else {
                    wait_vm<63>();
                    if (!hist) wait_vm<OPS + NACT>();
                }
                if constexpr (SHARE) {
                    // the partner's half of the next chunk: it passed the same
                    // wait before this barrier.  lgkmcnt(0): this wave's reads
                    // of the stage the refill after the barrier overwrites
                    // (the previous chunk's, read at its start) are complete.
                    __builtin_amdgcn_sched_barrier(0);
                    __builtin_amdgcn_s_waitcnt(0xC07F);
                    __builtin_amdgcn_s_barrier();
                    __builtin_amdgcn_sched_barrier(0);
                }
                read_ahead((sc + 1) & 3, std::integral_constant<int, SL1>{});
                __builtin_amdgcn_sched_barrier(0);
                issue_part(sis, std::integral_constant<int, 4>{});
                __builtin_amdgcn_sched_barrier(0);
            }
            const int fm = f & 3;
            u32x4 anx;
#pragma unroll
            for (int fn = 0; fn < 4; fn++) {
                const bf16x8 xa = __builtin_bit_cast(bf16x8, f < 4 ? fb0[SL][fn] : fb1[fn]);
                const bf16x8 xt = __builtin_bit_cast(bf16x8, acur);
                if constexpr (SWAP)
                    acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa, xt, acc[fm][fn], 0, 0, 0);
                else
                    acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xt, xa, acc[fm][fn], 0, 0, 0);
                anx[fn] = f < 7 ? dec(fa[SL], p4[SL], f + 1, fn) : dec(fa[SL1], p4[SL1], 0, fn);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);        // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, DEC_OPS, 0);  // then the decode
            }
            acur = anx;
        }
        __builtin_amdgcn_sched_barrier(0);
        sc = (sc + 1) & 3;
        hist >>= 1;
    };

    // prologue: three chunks in flight, then the first one's fragments
    issue(0);
    issue(1);
    issue(2);
    wait_vm<2 * OPS>();
    if constexpr (SHARE) {
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_s_barrier();
    }
    read_ahead(0, I0{});
#pragma unroll
    for (int j = 0; j < 4; j++) acur[j] = dec(fa[0], p4[0], 0, j);
    zero_acc();
    // tiles, then their chunks (the issue side runs three chunks ahead, across
    // tile boundaries)
    while (cv) {
        for (int c = 0; c < c_nch2; c += 2) {
            chunk(I0{});
            chunk(I1{});
        }
        epilogue();
        zero_acc();
        ++cj;
        cv = g_item(ga, cj, cpi, ctm, ctn, csp);
        if (cv) c_nch2 = (ga.p[cpi].nch + 1) & ~1;
        hist = 3;
    }
    // the last issues were out-of-range loads still writing zeros into this
    // wave's stages: drain them (and the stores) before the workgroup ends
    wait_vm<0>();
}

// ---------------------------------------------------------------------------
// Small kernels
// ---------------------------------------------------------------------------

// Ternarise and pack, one launch for the whole handle.  Blocks [0, nb_canon):
// one thread per canonical word (16 codes of one row), and past the canonical
// words the zero padding up to the first copy.  The next nb_fwd blocks write
// the forward operand's copy, the rest the dX operand's copy; each of those
// ternarises the block of q it needs itself, so no block waits for another.
struct MatGrid {
    int64_t nwords, nfill;      // canonical words; words up to the forward copy
    int64_t nchf, nchd;         // 32-K chunks of the forward / dX copy
    int64_t fwd_off, dx_off;    // word offsets of the copies
    int nb_canon, ngf, nb_fwd, ngd;   // blocks: canonical part; chunk groups and blocks of the copies
};
template <bool VEC>
__device__ __forceinline__ void materialize_block(const int8_t *__restrict__ q, int64_t in, int64_t out, int64_t wpr,
                                                  int theta, uint32_t *__restrict__ packed, const MatGrid &mg, int b,
                                                  uint32_t *blk) {
    if (b < mg.nb_canon) {
        const int64_t i = (int64_t)b * 256 + threadIdx.x;
        if (i < mg.nwords) {
            const int64_t r = i / wpr;
            packed[i] = tern_word<VEC>(q, out, theta, r, i - r * wpr);
        } else if (i < mg.nfill) {
            packed[i] = 0u;   // alignment padding before the fragment-ordered copies
        }
        return;
    }
    b -= mg.nb_canon;
    if (b < mg.nb_fwd) {
        derive_block<VEC, false>(q, in, out, wpr, theta, mg.nchf, b / mg.ngf, b % mg.ngf, packed + mg.fwd_off, blk);
        return;
    }
    b -= mg.nb_fwd;
    derive_block<VEC, true>(q, in, out, wpr, theta, mg.nchd, b / mg.ngd, b % mg.ngd, packed + mg.dx_off, blk);
}

template <bool VEC>
__global__ __launch_bounds__(256) void materialize_kernel(const int8_t *__restrict__ q, int64_t in, int64_t out,
                                                          int64_t wpr, int theta, uint32_t *__restrict__ packed,
                                                          MatGrid mg) {
    __shared__ uint32_t blk[D_LDS];
    materialize_block<VEC>(q, in, out, wpr, theta, packed, mg, (int)blockIdx.x, blk);
}

// Several matrices in one launch: block b belongs to the matrix whose blocks
// start at or before it, and runs that matrix's block b - start.
struct MatOne {
    const int8_t *q;
    uint32_t *packed;
    int64_t in, out, wpr;
    int vec;
    MatGrid mg;
};
struct MatGroup {
    int n, theta;
    int start[kMaxGroup + 1];
    MatOne m[kMaxGroup];
};
__global__ __launch_bounds__(256) void materialize_group_kernel(MatGroup g) {
    __shared__ uint32_t blk[D_LDS];
    const int b = blockIdx.x;
    int p = 0;
    while (p + 1 < g.n && b >= g.start[p + 1]) p++;
    const MatOne &m = g.m[p];
    if (m.vec)
        materialize_block<true>(m.q, m.in, m.out, m.wpr, g.theta, m.packed, m.mg, b - g.start[p], blk);
    else
        materialize_block<false>(m.q, m.in, m.out, m.wpr, g.theta, m.packed, m.mg, b - g.start[p], blk);
}

// Split-K finish of dW: G = sum over splits (ascending), gq = G * scale (acc:
// gq + alpha * G * scale), and the sgrad partial of a block of kReduceRows rows
// (ascending r).  Each thread owns 4 consecutive columns (16-byte loads and
// stores); a block covers 1024 columns of kReduceRows rows, few enough rows
// that a 2048 x 2048 reduce has 2048 blocks (several waves per SIMD to hide
// the loads' latency), with its split loop unrolled.
__device__ __forceinline__ void dw_reduce_block(const float *__restrict__ ws, int splits,
                                                const float *__restrict__ scale,
                                                const uint32_t *__restrict__ packed, int in, int out, int64_t wpr,
                                                float *__restrict__ gq, float *__restrict__ part, int acc,
                                                float alpha, int bx, int by) {
    const int c = (bx * 256 + threadIdx.x) * 4;
    if (c >= out) return;
    const int r0 = by * kReduceRows;
    const int r1 = min(in, r0 + kReduceRows);
    const f32x4 s = *(const f32x4 *)(scale + c);
    const int64_t plane = (int64_t)in * out;
    f32x4 p = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 4
    for (int r = r0; r < r1; r++) {
        const int64_t o = (int64_t)r * out + c;
        f32x4 gv = *(const f32x4 *)(ws + o);
#pragma unroll 4
        for (int k = 1; k < splits; k++) gv += *(const f32x4 *)(ws + k * plane + o);
        f32x4 t = gv * s;
        if (acc) t = *(const f32x4 *)(gq + o) + alpha * t;
        *(f32x4 *)(gq + o) = t;
        // the 4 codes of columns c .. c + 3 (c % 4 == 0, so one word holds them)
        const uint32_t word = packed[(int64_t)r * wpr + (c >> 4)] >> (2 * (c & 15));
        p.x += gv.x * code_to_f32(word & 3u);
        p.y += gv.y * code_to_f32((word >> 2) & 3u);
        p.z += gv.z * code_to_f32((word >> 4) & 3u);
        p.w += gv.w * code_to_f32((word >> 6) & 3u);
    }
    *(f32x4 *)(part + (int64_t)by * out + c) = p;
}

__global__ __launch_bounds__(256) void dw_reduce_kernel(const float *__restrict__ ws, int splits,
                                                        const float *__restrict__ scale,
                                                        const uint32_t *__restrict__ packed, int in,
                                                        int out, int64_t wpr, float *__restrict__ gq,
                                                        float *__restrict__ part, int acc, float alpha) {
    dw_reduce_block(ws, splits, scale, packed, in, out, wpr, gq, part, acc, alpha, (int)blockIdx.x, (int)blockIdx.y);
}

// sgrad[c] = sum of the row-block partials in ascending order, in f64, as a
// fixed two-level sum: 8 consecutive groups of blocks are each summed in
// ascending order, then the 8 group sums in ascending order (acc: added, times
// alpha, to the existing sgrad in f64).  A block of 256 threads serves 32
// columns.
__device__ __forceinline__ void sgrad_reduce_block(const float *__restrict__ part, int nparts, int out,
                                                   float *__restrict__ sgrad, int acc, float alpha, int bx) {
    __shared__ double red[8][32];
    const int cl = threadIdx.x & 31, grp = threadIdx.x >> 5;
    const int c = bx * 32 + cl;
    const int chunk = (nparts + 7) / 8;
    const int p0 = grp * chunk, p1 = min(nparts, p0 + chunk);
    double a = 0.0;
    if (c < out) {
#pragma unroll 8
        for (int p = p0; p < p1; p++) a += (double)part[(int64_t)p * out + c];
    }
    red[grp][cl] = a;
    __syncthreads();
    if (grp == 0 && c < out) {
        double s = red[0][cl];
#pragma unroll
        for (int g2 = 1; g2 < 8; g2++) s += red[g2][cl];
        if (acc) s = (double)sgrad[c] + (double)alpha * s;
        sgrad[c] = (float)s;
    }
}

__global__ __launch_bounds__(256) void sgrad_reduce_kernel(const float *__restrict__ part, int nparts,
                                                           int out, float *__restrict__ sgrad, int acc,
                                                           float alpha) {
    sgrad_reduce_block(part, nparts, out, sgrad, acc, alpha, (int)blockIdx.x);
}

// The dW finishing kernels of the projections of a layer, one launch each:
// blockIdx.z is the projection; blocks past a projection's grid return.
struct ReduceOne {
    const float *ws;             // split partials (splits > 1)
    const float *scale;
    const uint32_t *packed;
    float *gq, *part, *sgrad;
    int in, out, splits, nparts;
    int64_t wpr;
};
struct ReduceGroup {
    int n;
    ReduceOne r[kMaxGroup];
};
__global__ __launch_bounds__(256) void dw_reduce_group_kernel(ReduceGroup g) {
    const ReduceOne &r = g.r[blockIdx.z];
    if (r.splits < 2 || (int)blockIdx.y * kReduceRows >= r.in) return;
    dw_reduce_block(r.ws, r.splits, r.scale, r.packed, r.in, r.out, r.wpr, r.gq, r.part, 0, 1.0f, (int)blockIdx.x,
                    (int)blockIdx.y);
}
__global__ __launch_bounds__(256) void sgrad_reduce_group_kernel(ReduceGroup g) {
    const ReduceOne &r = g.r[blockIdx.y];
    if ((int)blockIdx.x * 32 >= r.out) return;
    sgrad_reduce_block(r.part, r.nparts, r.out, r.sgrad, 0, 1.0f, (int)blockIdx.x);
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

// Compute units of the current device (cached per device).
int device_cus() {
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

// grid: from plan_group_walk (the walk's workgroups)
template <int MODE>
hipError_t launch_persistent(const GroupArgs &ga, int64_t grid, hipStream_t st) {
    if (grid <= 0) return hipSuccess;
    const dim3 pgrid((unsigned)grid), block(dev::NT);
    if constexpr (MODE == MODE_DW)
        hipLaunchKernelGGL(dev::gemm_dw_kernel, pgrid, block, 0, st, ga);
    else if (MODE == MODE_DX && ga.p[0].acc)
        hipLaunchKernelGGL((dev::gemm_rd_kernel<MODE_DX, true>), pgrid, block, 0, st, ga);
    else if (MODE == MODE_FWD && ga.p[0].y_bf16 && ga.rd_wide)
        hipLaunchKernelGGL((dev::gemm_rd_kernel<MODE_FWD, false, true, true>), pgrid, block, 0, st, ga);
    else if (MODE == MODE_FWD && ga.p[0].y_bf16)
        hipLaunchKernelGGL((dev::gemm_rd_kernel<MODE_FWD, false, true, false>), pgrid, block, 0, st, ga);
    else if (ga.rd_wide)
        hipLaunchKernelGGL((dev::gemm_rd_kernel<MODE, false, false, true>), pgrid, block, 0, st, ga);
    else
        hipLaunchKernelGGL((dev::gemm_rd_kernel<MODE, false, false, false>), pgrid, block, 0, st, ga);
    return hipGetLastError();
}

template <bool BF, int MODE>
hipError_t launch_mode(const GemmPlan &p, const GemmArgs &a, hipStream_t st) {
    const dim3 grid((unsigned)p.grid), block(dev::NT);
    if constexpr (BF) {
        // the shared-M0 loads need K >= 32 (forward / dX) and M, N >= 256 (dW)
        // (the exact two-term dX scale runs on the LDS-staged kernel)
        if (p.tile == TILE_256 && (MODE == MODE_DW ? a.M >= 256 && a.N >= 256 : a.K >= 32) &&
            !(MODE == MODE_DX && a.exact_scale)) {
            // persistent: at most one workgroup per compute unit, walking the
            // items of a group of one problem
            GroupArgs ga{};
            ga.n = 1;
            ga.start[0] = 0;
            ga.start[1] = (int)(p.tiles_m * p.tiles_n * p.splits);
            ga.p[0] = a;
            if (MODE != MODE_DW && !rd_items(ga)) return hipErrorInvalidValue;
            const int64_t items = ga.start[1], cus = device_cus();
            return launch_persistent<MODE>(ga, items < cus ? items : cus, st);
        }
    }
    switch (p.tile) {
        case TILE_256: hipLaunchKernelGGL((dev::gemm_kernel<BF, MODE, 256>), grid, block, 0, st, a); break;
        case TILE_128: hipLaunchKernelGGL((dev::gemm_kernel<BF, MODE, 128>), grid, block, 0, st, a); break;
        default: hipLaunchKernelGGL((dev::gemm_kernel<BF, MODE, 64>), grid, block, 0, st, a); break;
    }
    return hipGetLastError();
}
}  // namespace

hipError_t launch_gemm_group(int mode, const GroupArgs &ga_in, hipStream_t st) {
    if (ga_in.n < 1 || ga_in.n > kMaxGroup) return hipErrorInvalidValue;
    GroupArgs ga = ga_in;
    // the forward / dX items follow the kernel's tile, whatever the caller cut
    if (mode != MODE_DW && !rd_items(ga)) return hipErrorInvalidValue;
    int64_t cost[kMaxGroup];
    for (int p = 0; p < ga.n; p++)
        cost[p] = mode == MODE_DW ? cdiv(ga.p[p].kps, dev::W_KC) : (int64_t)ga.p[p].nch;
    const int64_t grid = plan_group_walk(ga, cost, device_cus());
    if (mode == MODE_FWD) return launch_persistent<MODE_FWD>(ga, grid, st);
    if (mode == MODE_DX) return launch_persistent<MODE_DX>(ga, grid, st);
    return launch_persistent<MODE_DW>(ga, grid, st);
}

hipError_t launch_gemm(const GemmPlan &p, bool bf16, const GemmArgs &a, hipStream_t st) {
    if (p.grid <= 0) return hipSuccess;
    // no kernel is enqueued with a pointer it dereferences missing
    if (check_gemm_args(p, a) != 0) return hipErrorInvalidValue;
    if (bf16) {
        if (p.mode == MODE_FWD) return launch_mode<true, MODE_FWD>(p, a, st);
        if (p.mode == MODE_DX) return launch_mode<true, MODE_DX>(p, a, st);
        return launch_mode<true, MODE_DW>(p, a, st);
    }
    if (p.mode == MODE_FWD) return launch_mode<false, MODE_FWD>(p, a, st);
    if (p.mode == MODE_DX) return launch_mode<false, MODE_DX>(p, a, st);
    return launch_mode<false, MODE_DW>(p, a, st);
}

namespace {
// Blocks of the materialize launch of one [in, out] matrix (0 if empty).
int64_t mat_grid(int64_t in, int64_t out, dev::MatGrid &mg) {
    const PackedLayout L = packed_layout(in, out);
    if (L.total == 0) return 0;
    const int64_t wpr = cdiv(out, 16);
    mg.nwords = in * wpr;
    mg.nfill = L.fwd_off;
    // forward operand: tiles over out, chunks over in; dX operand: the reverse
    mg.nchf = cdiv(in, kFragChunk);
    mg.nchd = cdiv(out, kFragChunk);
    mg.fwd_off = L.fwd_off;
    mg.dx_off = L.dx_off;
    const int64_t nb_canon = cdiv(mg.nfill, 256), ngf = cdiv(mg.nchf, dev::D_G), ngd = cdiv(mg.nchd, dev::D_G);
    const int64_t nb_fwd = cdiv(out, 256) * ngf, nb_dx = cdiv(in, 256) * ngd;
    const int64_t blocks = nb_canon + nb_fwd + nb_dx;
    mg.nb_canon = (int)nb_canon;
    mg.ngf = (int)ngf;
    mg.nb_fwd = (int)nb_fwd;
    mg.ngd = (int)ngd;
    return blocks;
}
}  // namespace

hipError_t launch_materialize(const int8_t *q, int64_t in, int64_t out, int theta, bool vec,
                              uint32_t *packed, hipStream_t st) {
    dev::MatGrid mg;
    const int64_t blocks = mat_grid(in, out, mg);
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    const int64_t wpr = cdiv(out, 16);
    const dim3 grid((unsigned)blocks), block(256);
    if (vec)
        hipLaunchKernelGGL((dev::materialize_kernel<true>), grid, block, 0, st, q, in, out, wpr, theta, packed, mg);
    else
        hipLaunchKernelGGL((dev::materialize_kernel<false>), grid, block, 0, st, q, in, out, wpr, theta, packed, mg);
    return hipGetLastError();
}

hipError_t launch_materialize_group(const MatOneHost *m, int n, int theta, hipStream_t st) {
    if (n < 1 || n > kMaxGroup) return hipErrorInvalidValue;
    dev::MatGroup g{};
    g.n = n;
    g.theta = theta;
    int64_t total = 0;
    for (int i = 0; i < n; i++) {
        dev::MatOne &o = g.m[i];
        o.q = m[i].q;
        o.packed = m[i].packed;
        o.in = m[i].in;
        o.out = m[i].out;
        o.wpr = cdiv(m[i].out, 16);
        o.vec = m[i].vec ? 1 : 0;
        g.start[i] = (int)total;
        total += mat_grid(m[i].in, m[i].out, o.mg);
        if (total > 0x7FFFFFFF) return hipErrorInvalidValue;
    }
    g.start[n] = (int)total;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(dev::materialize_group_kernel, dim3((unsigned)total), dim3(256), 0, st, g);
    return hipGetLastError();
}

hipError_t launch_dw_finish_group(const DwFinishHost *f, int n, hipStream_t st) {
    if (n < 1 || n > kMaxGroup) return hipErrorInvalidValue;
    dev::ReduceGroup g{};
    g.n = n;
    int64_t gx = 0, gy = 0, sx = 0;
    bool any_split = false;
    for (int i = 0; i < n; i++) {
        dev::ReduceOne &r = g.r[i];
        r.ws = f[i].ws;
        r.scale = f[i].scale;
        r.packed = f[i].packed;
        r.gq = f[i].gq;
        r.part = f[i].part;
        r.sgrad = f[i].sgrad;
        r.in = (int)f[i].in;
        r.out = (int)f[i].out;
        r.splits = (int)f[i].splits;
        r.nparts = (int)f[i].nparts;
        r.wpr = cdiv(f[i].out, 16);
        if (f[i].splits > 1) {
            any_split = true;
            gx = std::max<int64_t>(gx, cdiv(f[i].out, 1024));
            gy = std::max<int64_t>(gy, cdiv(f[i].in, kReduceRows));
        }
        sx = std::max<int64_t>(sx, cdiv(f[i].out, 32));
    }
    if (any_split) {
        hipLaunchKernelGGL(dev::dw_reduce_group_kernel, dim3((unsigned)gx, (unsigned)gy, (unsigned)n), dim3(256), 0,
                           st, g);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (sx == 0) return hipSuccess;
    hipLaunchKernelGGL(dev::sgrad_reduce_group_kernel, dim3((unsigned)sx, (unsigned)n), dim3(256), 0, st, g);
    return hipGetLastError();
}

hipError_t launch_dw_reduce(const float *ws, int splits, const float *scale, const uint32_t *packed,
                            int64_t in, int64_t out, float *gq, float *part, bool acc, float alpha,
                            hipStream_t st) {
    const dim3 grid((unsigned)cdiv(out, 1024), (unsigned)cdiv(in, kReduceRows)), block(256);
    hipLaunchKernelGGL(dev::dw_reduce_kernel, grid, block, 0, st, ws, splits, scale, packed, (int)in,
                       (int)out, cdiv(out, 16), gq, part, (int)acc, alpha);
    return hipGetLastError();
}

hipError_t launch_sgrad_reduce(const float *part, int64_t nparts, int64_t out, float *sgrad, bool acc, float alpha,
                               hipStream_t st) {
    if (out <= 0) return hipSuccess;
    const dim3 grid((unsigned)cdiv(out, 32)), block(256);
    hipLaunchKernelGGL(dev::sgrad_reduce_kernel, grid, block, 0, st, part, (int)nparts, (int)out, sgrad,
                       (int)acc, alpha);
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
