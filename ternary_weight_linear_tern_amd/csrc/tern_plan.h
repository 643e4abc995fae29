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

GemmPlan plan_gemm(int mode, int64_t T, int64_t in, int64_t out, bool bf16);

// Backward workspace layout (byte offsets, 256-byte aligned).
struct BwdLayout {
    GemmPlan dx, dw;
    int64_t part_rows = 0;     // rows of the sgrad partial table
    size_t part_off = 0, part_bytes = 0;
    size_t ws_off = 0, ws_bytes = 0;   // split-K partial products of G
    size_t total = 0;
};

// acc: the accumulating dW variant, whose G always goes through the split
// workspace (raw G, then the reduce kernel adds to gq).
BwdLayout plan_bwd(int64_t T, int64_t in, int64_t out, bool bf16, bool acc = false);

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
// tile of 256 rows and chunk of 32 K, 512 words in the order the 256 x 256
// GEMMs load them (one 16-byte load per lane and chunk).
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
