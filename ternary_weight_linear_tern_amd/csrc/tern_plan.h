// tern_plan.h -- HIP-free argument validation and launch planning for libtern.
//
// Everything here is plain C++ (no HIP headers) so the same decisions can be
// made and unit-tested on a machine without a GPU.  The kernels read their
// geometry from a GemmPlan; tern_linear_bwd_workspace_bytes and the launch
// wrappers derive the same plan from the same arguments.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace tern {

// Tile shapes of the MFMA GEMM kernels (all use 256 threads = 4 wave64s in a
// 2 x 2 arrangement).
enum TileId : int { TILE_256 = 0, TILE_128 = 1, TILE_64 = 2 };

inline int tile_bm(int t) { return t == TILE_256 ? 256 : t == TILE_128 ? 128 : 64; }

// The three products of the projection.  M x N is the output tile grid, K the
// reduction:
//   FWD: M = out (columns of W), N = T (tokens), K = in
//   DX : M = in,                 N = T,          K = out
//   DW : M = in,                 N = out,        K = T
enum GemmMode : int { MODE_FWD = 0, MODE_DX = 1, MODE_DW = 2 };

struct GemmPlan {
    int mode = 0;
    int tile = TILE_256;
    int64_t M = 0, N = 0, K = 0;
    int64_t tiles_m = 0, tiles_n = 0;
    int64_t splits = 1;        // K split count (DW only)
    int64_t k_per_split = 0;   // multiple of the K step
    int64_t grid = 0;          // workgroups
};

// K step of the main loop per element type: 64 bf16 or 32 fp32 (128 bytes).
inline int k_step(bool bf16) { return bf16 ? 64 : 32; }

// max_splits caps the dW split-K count (the planner picks the best count up to
// it; 0 means no cap).
GemmPlan plan_gemm(int mode, int64_t T, int64_t in, int64_t out, bool bf16, int64_t max_splits = 0);

// Kernel arguments of the three MFMA GEMMs (M, N, K as above).
struct GemmArgs {
    const void *act0;        // FWD: X, DX: dY, DW: X
    const void *act1;        // DW: dY
    const uint32_t *packed;  // tern, 2-bit packed [in][wpr]
    const uint32_t *frag;    // FWD / DX: this product's fragment-ordered copy of tern;
                             // DW: the forward copy (tern codes of the sgrad partials)
    const float *scale;      // [out]
    void *out_ptr;           // FWD: Y, DX: dX, DW: gq (1 split) or split partials
    float *part;             // DW with 1 split: sgrad partials [tiles_m][out]
    int M, N, K;
    int tiles_m, tiles_n, splits, kps;
    int in, out, wpr, T;
    int y_bf16;
    int nch;                 // FWD / DX: chunks of 32 K per tile in the fragment copy
    int acc;                 // DX: add to the existing dX; DW: raw G into out_ptr even with one split
    int exact_scale;         // DX, bf16: the scale as the sum of two bf16 terms (two passes over K)
};

// Host and device: the item walk below is shared by the kernels and by the
// planner's checks.
#if defined(__HIPCC__)
#define TERN_HD __host__ __device__
#else
#define TERN_HD
#endif

// Several independent problems of one mode in one persistent launch (the
// projections of a layer): their work items (tiles, times splits for dW) form
// one item space, problem by problem, and the grid walks it in one of three
// ways:
//   WALK_STATIC   persistent grid, workgroup b takes items b, b + G, b + 2G, ...
//   WALK_DYNAMIC  one workgroup per item, in item order (the dispatcher starts
//                 each as a unit frees up: longest first)
//   WALK_CLASSES  persistent grid in classes of workgroups: every workgroup of
//                 class k takes cls_cnt[k][p] items of problem p (problems in
//                 order), the class's items of p being cls_base[k][p] +
//                 e * (class size) + slot (e-th item of the workgroup in slot
//                 slot of its class).  The planner fills the classes longest
//                 items first onto the least loaded workgroups, so a layer of
//                 mixed reduction lengths keeps every unit busy to the end
//                 without giving up the walk's prefetch across items.
constexpr int kMaxGroup = 8;
constexpr int kMaxClass = 8;
enum GroupWalk : int { WALK_STATIC = 0, WALK_DYNAMIC = 1, WALK_CLASSES = 2 };
struct GroupArgs {
    int n;                          // problems
    int start[kMaxGroup + 1];       // first item of each problem; start[n] = all items
    int walk;                       // GroupWalk
    int ncls;                       // WALK_CLASSES: classes of workgroups
    int cls_wg[kMaxClass + 1];      // first workgroup of each class; cls_wg[ncls] = grid
    int cls_cnt[kMaxClass][kMaxGroup];    // items of problem p per workgroup of class k
    int cls_base[kMaxClass][kMaxGroup];   // first item of problem p (within it) taken by class k
    int rd_wide;                    // forward / dX: 512 x 128 tiles (else 256 x 256), set by rd_items
    GemmArgs p[kMaxGroup];
};

// Item j of workgroup b of a grid of G workgroups: its problem pi, tile
// (tm, tn) and split sp; false once the workgroup's items run out.  Consecutive
// items of a round go to one XCD (workgroups are dispatched round-robin over
// the 8 XCDs), and within a problem the tiles are grouped 8 along M, so the
// tiles resident on one XCD share operand panels in its L2.
TERN_HD inline bool group_item(const GroupArgs &ga, int G, int b, int j, int &pi, int &tm, int &tn, int &sp) {
    int L;
    if (ga.walk == WALK_CLASSES) {
        int k = 0;
        while (k + 1 < ga.ncls && b >= ga.cls_wg[k + 1]) k++;
        const int w0 = ga.cls_wg[k], m = ga.cls_wg[k + 1] - w0, r = b - w0;
        int p = 0, e = j;
        while (p < ga.n && e >= ga.cls_cnt[k][p]) {
            e -= ga.cls_cnt[k][p];
            p++;
        }
        if (p >= ga.n || r >= m) return false;
        const int slot = ((m | w0) & 7) == 0 ? (r & 7) * (m >> 3) + (r >> 3) : r;
        L = ga.start[p] + ga.cls_base[k][p] + e * m + slot;
    } else if (ga.walk == WALK_DYNAMIC) {
        // one item per workgroup; within each full run of 256 consecutive
        // workgroups (dispatched together, round-robin over the XCDs) the
        // items of one XCD are consecutive
        const int base = b & ~255, c = b & 255;
        L = j * G + base + (base + 256 <= G ? (c & 7) * 32 + (c >> 3) : c);
    } else {
        L = (G & 7) == 0 ? j * G + (b & 7) * (G >> 3) + (b >> 3) : j * G + b;
    }
    if (L >= ga.start[ga.n]) return false;
    int p = 0;
    while (p + 1 < ga.n && L >= ga.start[p + 1]) p++;
    pi = p;
    const int tiles_m = ga.p[p].tiles_m, tiles_n = ga.p[p].tiles_n;
    const int tiles = tiles_m * tiles_n;
    const int local = L - ga.start[p];
    sp = local / tiles;
    const int t = local - sp * tiles;
    constexpr int GM = 8;
    const int group = t / (GM * tiles_n);
    const int first = group * GM;
    const int gs = tiles_m - first < GM ? tiles_m - first : GM;
    const int within = t - group * GM * tiles_n;
    tm = first + within % gs;
    tn = within / gs;
    return true;
}

// Items of the persistent forward / dX kernels, one tile shape per launch:
// 512 x 128 tiles (output columns x tokens) for the plain products unless
// their padding makes the launch's multiply-adds more than 3 % above those of
// 256 x 256 tiles (columns off the 512 grid: 768 columns pad to 1024, against
// 768), 256 x 256 then and for the accumulating dX (every problem of a launch
// is plain or accumulating, as p[0].acc says).  Sets rd_wide, each problem's
// tiles_m / tiles_n and the item starts.  False when the items do not fit the
// walk's int range.
inline bool rd_items(GroupArgs &ga) {
    bool wide = !ga.p[0].acc;
    if (wide) {
        double w = 0.0, q = 0.0;
        for (int i = 0; i < ga.n; i++) {
            const GemmArgs &a = ga.p[i];
            const int64_t m = a.M, n = a.N;
            w += double((m + 511) / 512 * 512) * double((n + 127) / 128 * 128) * double(a.K);
            q += double((m + 255) / 256 * 256) * double((n + 255) / 256 * 256) * double(a.K);
        }
        wide = w <= 1.03 * q;
    }
    ga.rd_wide = wide ? 1 : 0;
    int64_t total = 0;
    for (int i = 0; i < ga.n; i++) {
        GemmArgs &a = ga.p[i];
        const int64_t bm = wide ? 512 : 256, bn = wide ? 128 : 256;
        const int64_t tm = (a.M + bm - 1) / bm, tn = (a.N + bn - 1) / bn;
        ga.start[i] = (int)total;
        total += tm * tn * a.splits;
        if (total > (int64_t(1) << 30)) return false;
        a.tiles_m = (int)tm;
        a.tiles_n = (int)tn;
    }
    ga.start[ga.n] = (int)total;
    return true;
}

// Chooses the walk of a group launch on `cus` compute units and fills its
// fields; returns the grid (0 for no items).  cost[p]: length of problem p's
// items (K steps).  Each item also pays about 2 steps of prologue and
// epilogue, which the persistent walks overlap with the neighbours' work.
// Static when its makespan is the best; classes when they shorten it (and fit
// in kMaxClass); one workgroup per item when neither is balanced.
int64_t plan_group_walk(GroupArgs &ga, const int64_t *cost, int64_t cus);

// The static walk's makespan and the classes' (WALK_CLASSES fields filled in
// ga; false when more than kMaxClass classes would be needed), in cost units
// with the 2-step overhead per item.  Exposed for the planner's checks.
int64_t static_makespan(const GroupArgs &ga, const int64_t *cost, int64_t cus, int64_t *total = nullptr);
bool plan_classes(GroupArgs &ga, const int64_t *cost, int64_t cus, int64_t &makespan);

// Tokens per split of the weight-gradient product shared by the problems of
// a layer (all have K = T; the split count is cdiv(T, result)): the count
// (a power of two within plan_gemm's limits: at least 8 K steps per split, at
// most 32) that minimises rounds of items over the chip times their length
// plus the traffic of the split partials.  tiles: the 256 x 256 tiles of all
// problems together.
int64_t plan_layer_dw_splits(int64_t T, int64_t tiles, int64_t sum_in_out, bool bf16);

// dX with bf16 activations: does the scale go into the operand as the sum of
// two bf16 terms (hi = bf16(scale), lo = bf16(scale - hi), two passes over K)
// instead of one rounded term?  One rounded term has a relative error of up to
// 2^-8 per column (rms 1.6e-3), and the rel-L2 of dX is a weighted mean of
// those errors, which concentrates near 1.66e-3 only with many reduction
// columns and many outputs; with few of either it exceeds 2e-3 for a sizeable
// fraction of inputs.  Two terms bring it to about 1e-5 at twice the dX
// product's matrix work, so they are used where that work is small: fewer
// than 512 columns (out) or fewer than 65536 outputs (T * in).
bool dx_exact_scale(int64_t T, int64_t in, int64_t out);
constexpr int64_t kFoldMinCols = 512;
constexpr int64_t kFoldMinOutputs = 65536;

// Host check of the pointers a launch of plan p dereferences: every operand,
// the output, the fragment copy, and the sgrad partial table wherever the dW
// epilogue writes partials (one split, not accumulating).  TERN_OK, or
// TERN_ERR_NULL for a missing operand or output, TERN_ERR_WORKSPACE for a
// missing partial table.  Every launcher calls it before enqueueing a kernel.
int check_gemm_args(const GemmPlan &p, const GemmArgs &a);

// Backward workspace layout (byte offsets, 256-byte aligned).
struct BwdLayout {
    GemmPlan dx, dw;
    int64_t part_rows = 0;     // rows of the sgrad partial table
    size_t part_off = 0, part_bytes = 0;
    size_t ws_off = 0, ws_bytes = 0;   // split-K partial products of G
    size_t total = 0;
};

// acc: the accumulating dW variant, whose G always goes through the split
// workspace (raw G, then the reduce kernel adds to gq).  ws_limit: the largest
// workspace the caller has; the dW split count is lowered until the layout
// fits (total > ws_limit only if even one split does not fit).
BwdLayout plan_bwd(int64_t T, int64_t in, int64_t out, bool bf16, bool acc = false,
                   size_t ws_limit = ~size_t(0));

// Workspace bytes that serve either activation type: the larger of the two
// plans (0 for invalid sizes).
size_t bwd_workspace_bytes(int64_t T, int64_t in, int64_t out, bool acc);

// Row-block height of the split-K reduction (and thus of its sgrad partials).
constexpr int kReduceRows = 4;

// Largest accepted dimensions: tile offsets stay well inside 32 bits.
constexpr int64_t kMaxInOut = int64_t(1) << 20;
constexpr int64_t kMaxT = (int64_t(1) << 31) - 1;

int validate_shape(int64_t T, int64_t in, int64_t out);

// Layout of a packed ternary handle (in uint32 words).  The canonical 2-bit
// matrix comes first; two fragment-ordered copies of it follow, one for the
// forward operand (rows m = output columns, K = input rows) and one for the dX
// operand (rows m = input rows, K = output columns).  Each copy holds, per
// tile of 256 rows and chunk of 32 K, 512 words in the order the persistent
// GEMMs load them (one 16-byte load per lane and chunk; a 512-column tile of
// the forward / dX kernel reads two such tiles).
constexpr int64_t kFragTileRows = 256;
constexpr int64_t kFragChunk = 32;
constexpr int64_t kFragWords = 512;   // words per (tile, chunk)

struct PackedLayout {
    int64_t canon_words = 0;           // in * ceil(out / 16)
    int64_t fwd_off = 0, fwd_words = 0;
    int64_t dx_off = 0, dx_words = 0;
    int64_t total = 0;
};

PackedLayout packed_layout(int64_t in, int64_t out);

// True if [a, a + na) and [b, b + nb) overlap (empty ranges never overlap).
bool ranges_overlap(const void *a, size_t na, const void *b, size_t nb);

}  // namespace tern
