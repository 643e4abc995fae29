// tern_plan.cpp -- HIP-free validation and planning (see tern_plan.h).
#include "tern_plan.h"

#include "../../include/tern.h"

namespace tern {

namespace {

constexpr int64_t kCUs = 256;  // MI355X compute units; one 256-thread workgroup each

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Relative efficiency of a tile shape once the chip is full: the larger wave
// tiles reuse each LDS fragment more and hide the operand staging better, and
// the 256 x 256 tiles run the persistent kernels.  Measured on MI355X: the
// forward of 1024 x 1024 at 8192 tokens takes 1.56 times as long with 128 x 128
// tiles filling the chip as with 256 x 256 tiles on half of it, so 128 x 128
// rates about 0.3; 64 x 64 tiles stay best for the smallest products, which
// keeps them at about 0.12.
double tile_eff(int t) { return t == TILE_256 ? 1.0 : t == TILE_128 ? 0.30 : 0.12; }

// Fraction of the chip's workgroup slots a grid keeps busy, counting the idle
// slots of a partial last wave.
double fill(int64_t grid) {
    if (grid <= 0) return 1.0;
    int64_t waves = cdiv(grid, kCUs);
    return double(grid) / double(waves * kCUs);
}

}  // namespace

int validate_shape(int64_t T, int64_t in, int64_t out) {
    if (T < 0 || in < 0 || out < 0) return TERN_ERR_SHAPE;
    if (in % 8 != 0 || out % 8 != 0) return TERN_ERR_SHAPE;
    if (in > kMaxInOut || out > kMaxInOut || T > kMaxT) return TERN_ERR_SHAPE;
    return TERN_OK;
}

PackedLayout packed_layout(int64_t in, int64_t out) {
    PackedLayout L;
    if (in <= 0 || out <= 0) return L;
    L.canon_words = in * cdiv(out, 16);
    L.fwd_off = cdiv(L.canon_words, 64) * 64;   // 256-byte aligned copies
    L.fwd_words = cdiv(out, kFragTileRows) * cdiv(in, kFragChunk) * kFragWords;
    L.dx_off = L.fwd_off + L.fwd_words;
    L.dx_words = cdiv(in, kFragTileRows) * cdiv(out, kFragChunk) * kFragWords;
    L.total = L.dx_off + L.dx_words;
    return L;
}

bool ranges_overlap(const void *a, size_t na, const void *b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

GemmPlan plan_gemm(int mode, int64_t T, int64_t in, int64_t out, bool bf16, int64_t max_splits) {
    GemmPlan p;
    p.mode = mode;
    if (mode == MODE_FWD) { p.M = out; p.N = T; p.K = in; }
    else if (mode == MODE_DX) { p.M = in; p.N = T; p.K = out; }
    else { p.M = in; p.N = out; p.K = T; }
    const int64_t kstep = k_step(bf16);
    if (p.M <= 0 || p.N <= 0 || p.K <= 0) { p.grid = 0; return p; }

    double best = -1.0;
    for (int t = TILE_256; t <= TILE_64; t++) {
        const int64_t bm = tile_bm(t);
        const int64_t tm = cdiv(p.M, bm), tn = cdiv(p.N, bm);
        const int64_t tiles = tm * tn;
        const int64_t ksteps = cdiv(p.K, kstep);
        // split K only for the weight gradient, whose K (= tokens) is long and
        // whose output grid (in x out) can be smaller than the chip
        int64_t max_s = 1;
        if (mode == MODE_DW) {
            max_s = ksteps / 8;  // keep >= 8 K steps per split
            if (max_s < 1) max_s = 1;
            if (max_s > 32) max_s = 32;
            if (max_splits > 0 && max_s > max_splits) max_s = max_splits;
        }
        for (int64_t s = 1; s <= max_s; s *= 2) {
            const int64_t kps = cdiv(ksteps, s) * kstep;
            const int64_t real_s = cdiv(p.K, kps);
            const int64_t grid = tiles * real_s;
            // useful MFMA rate relative to a full chip of 256x256 tiles
            double rate = tile_eff(t) * fill(grid) * (grid < kCUs ? 1.0 : 1.0);
            double flops = 2.0 * double(p.M) * double(p.N) * double(p.K);
            double t_mma = flops / (rate * 2.3e15);
            // split-K partials: written once, read once, in fp32
            double t_ws = real_s > 1 ? 2.0 * double(real_s) * double(p.M * p.N) * 4.0 / 5.0e12 : 0.0;
            // per-workgroup prologue/epilogue, roughly 2 K steps of work
            double t_edge = double(cdiv(grid, kCUs)) * 2.0 * 2.0 * bm * bm * kstep / (tile_eff(t) * 9.0e12);
            double score = 1.0 / (t_mma + t_ws + t_edge);
            if (score > best) {
                best = score;
                p.tile = t;
                p.tiles_m = tm;
                p.tiles_n = tn;
                p.splits = real_s;
                p.k_per_split = kps;
                p.grid = grid;
            }
        }
    }
    return p;
}

int64_t plan_layer_dw_splits(int64_t T, int64_t tiles, int64_t sum_in_out, bool bf16) {
    const int64_t kstep = k_step(bf16);
    const int64_t ksteps = cdiv(T, kstep);
    int64_t max_s = ksteps / 8;
    if (max_s < 1) max_s = 1;
    if (max_s > 32) max_s = 32;
    double best = -1.0;
    int64_t best_kps = ksteps * kstep;
    for (int64_t s = 1; s <= max_s; s *= 2) {
        const int64_t kps = cdiv(ksteps, s) * kstep;
        const int64_t real_s = cdiv(T, kps);
        const int64_t items = tiles * real_s;
        // rounds of items over the chip, each as long as one split's K steps,
        // plus the prologue / epilogue of each item (about 2 K steps)
        const double t_mma = double(cdiv(items, kCUs)) * double(kps / kstep + 2);
        // split partials: written once and read once in fp32 (in K-step units
        // of a 256 x 256 tile: 1 K step of 64 bf16 moves 64 KB at ~30 B/clk/CU,
        // i.e. ~2000 clk; here the whole chip moves the partials at 5 TB/s)
        const double step_s = 2000.0 / 2.1e9;
        const double t_ws = real_s > 1 ? 2.0 * double(real_s) * double(sum_in_out) * 4.0 / 5.0e12 / step_s : 0.0;
        const double score = 1.0 / (t_mma + t_ws);
        if (score > best) {
            best = score;
            best_kps = kps;
        }
    }
    return best_kps;
}

namespace {
constexpr int64_t kItemOverhead = 2;   // prologue + epilogue of an item, in K steps
}

int64_t static_makespan(const GroupArgs &ga, const int64_t *cost, int64_t cus, int64_t *total_out) {
    // workgroup w takes items w, w + G, w + 2G, ... (G = cus)
    int64_t worst = 0, total = 0;
    for (int64_t w = 0; w < cus; w++) {
        int64_t load = 0;
        for (int p = 0; p < ga.n; p++) {
            const int64_t s0 = ga.start[p], s1 = ga.start[p + 1];
            // k with s0 <= w + k G < s1
            const int64_t k0 = s0 > w ? (s0 - w + cus - 1) / cus : 0;
            const int64_t k1 = s1 > w ? (s1 - w + cus - 1) / cus : 0;
            if (k1 > k0) load += (k1 - k0) * (cost[p] + kItemOverhead);
        }
        worst = load > worst ? load : worst;
        total += load;
    }
    if (total_out) *total_out = total;
    return worst;
}

bool plan_classes(GroupArgs &ga, const int64_t *cost, int64_t cus, int64_t &makespan) {
    struct Cls {
        int64_t nwg, load;
        int cnt[kMaxGroup];
    };
    Cls c[kMaxClass] = {};
    int nc = 1;
    c[0].nwg = cus;
    // problems longest items first (stable), each item onto a least loaded
    // workgroup; the workgroups of a class share their history, so a class
    // whose turn takes fewer items than it has workgroups splits in two (the
    // ones that took an item first)
    int order[kMaxGroup];
    for (int p = 0; p < ga.n; p++) order[p] = p;
    for (int i = 1; i < ga.n; i++)
        for (int j = i; j > 0 && cost[order[j]] > cost[order[j - 1]]; j--) {
            const int t = order[j];
            order[j] = order[j - 1];
            order[j - 1] = t;
        }
    for (int oi = 0; oi < ga.n; oi++) {
        const int p = order[oi];
        const int64_t len = cost[p] + kItemOverhead;
        int64_t left = (int64_t)ga.start[p + 1] - ga.start[p];
        while (left > 0) {
            int k = 0;
            for (int i = 1; i < nc; i++)
                if (c[i].load < c[k].load) k = i;
            if (left >= c[k].nwg) {
                // every workgroup of the class takes one more item (in bulk
                // while the class stays the least loaded)
                int64_t rounds = left / c[k].nwg;
                int64_t next = -1;   // the lowest load of the other classes
                for (int i = 0; i < nc; i++)
                    if (i != k && (next < 0 || c[i].load < next)) next = c[i].load;
                if (next >= 0) {
                    // rounds after which this class is no longer below `next`
                    const int64_t r_max = (next - c[k].load) / len + 1;
                    rounds = rounds < r_max ? rounds : r_max;
                }
                c[k].cnt[p] += (int)rounds;
                c[k].load += rounds * len;
                left -= rounds * c[k].nwg;
            } else {
                if (nc == kMaxClass) return false;
                for (int i = nc; i > k; i--) c[i] = c[i - 1];
                nc++;
                c[k].nwg = left;
                c[k].cnt[p] += 1;
                c[k].load += len;
                c[k + 1].nwg -= left;
                left = 0;
            }
        }
    }
    makespan = 0;
    int64_t wg = 0;
    int base[kMaxGroup] = {};
    ga.ncls = nc;
    for (int k = 0; k < nc; k++) {
        makespan = c[k].load > makespan ? c[k].load : makespan;
        ga.cls_wg[k] = (int)wg;
        for (int p = 0; p < ga.n; p++) {
            ga.cls_cnt[k][p] = c[k].cnt[p];
            ga.cls_base[k][p] = base[p];
            base[p] += (int)(c[k].nwg * c[k].cnt[p]);
        }
        wg += c[k].nwg;
    }
    ga.cls_wg[nc] = (int)wg;
    return true;
}

int64_t plan_group_walk(GroupArgs &ga, const int64_t *cost, int64_t cus) {
    const int64_t items = ga.start[ga.n];
    ga.walk = WALK_STATIC;
    ga.ncls = 0;
    if (items <= 0) return 0;
    if (cus <= 0) cus = 1;
    if (items <= cus) return items;   // one item per workgroup
    int64_t total = 0;
    const int64_t worst = static_makespan(ga, cost, cus, &total);
    GroupArgs trial = ga;
    int64_t cls = 0;
    if (plan_classes(trial, cost, cus, cls) && cls < worst) {
        ga = trial;
        ga.walk = WALK_CLASSES;
        return ga.cls_wg[ga.ncls];
    }
    // one workgroup per item, longest first, each started as a unit frees up
    // (list scheduling): about the average load, or the longest item; the
    // prologue and epilogue of every item are no longer hidden
    int64_t longest = 0;
    for (int p = 0; p < ga.n; p++) longest = cost[p] > longest ? cost[p] : longest;
    double dyn_est = double(total) / double(cus) + double(kItemOverhead) * double(items) / double(cus);
    if (dyn_est < double(longest + 2 * kItemOverhead)) dyn_est = double(longest + 2 * kItemOverhead);
    if (double(worst) > 1.08 * dyn_est) {
        ga.walk = WALK_DYNAMIC;
        return items;
    }
    return cus;
}

bool dx_exact_scale(int64_t T, int64_t in, int64_t out) {
    return out < kFoldMinCols || T * in < kFoldMinOutputs;
}

int check_gemm_args(const GemmPlan &p, const GemmArgs &a) {
    if (p.grid <= 0) return TERN_OK;   // nothing is launched
    if (!a.act0 || !a.scale || !a.out_ptr) return TERN_ERR_NULL;
    if (p.mode == MODE_DW && !a.act1) return TERN_ERR_NULL;
    if (!a.packed) return TERN_ERR_NULL;
    // the 256-tile kernels read the fragment-ordered copies (the dW epilogue
    // its tern codes)
    if (p.tile == TILE_256 && !a.frag) return TERN_ERR_NULL;
    if (p.mode == MODE_DW && p.splits == 1 && !a.acc && !a.part) return TERN_ERR_WORKSPACE;
    return TERN_OK;
}

BwdLayout plan_bwd(int64_t T, int64_t in, int64_t out, bool bf16, bool acc, size_t ws_limit) {
    BwdLayout L;
    L.dx = plan_gemm(MODE_DX, T, in, out, bf16);
    auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    for (int64_t cap = 0;;) {
        L.dw = plan_gemm(MODE_DW, T, in, out, bf16, cap);
        L.part_rows = 0;
        L.part_off = L.part_bytes = L.ws_off = L.ws_bytes = 0;
        if (T > 0 && in > 0 && out > 0) {
            const int64_t bm = tile_bm(L.dw.tile);
            const bool raw = L.dw.splits > 1 || acc;   // G through the workspace and the reduce kernel
            L.part_rows = raw ? cdiv(in, kReduceRows) : cdiv(in, bm);
            L.part_off = 0;
            L.part_bytes = al(size_t(L.part_rows) * size_t(out) * 4);
            L.ws_off = L.part_bytes;
            L.ws_bytes = raw ? al(size_t(L.dw.splits) * size_t(in) * size_t(out) * 4) : 0;
        }
        L.total = L.part_bytes + L.ws_bytes;
        if (L.total <= ws_limit || L.dw.splits <= 1) break;
        cap = L.dw.splits - 1;   // the next plan has fewer splits
    }
    return L;
}

size_t bwd_workspace_bytes(int64_t T, int64_t in, int64_t out, bool acc) {
    if (validate_shape(T, in, out) != TERN_OK) return 0;
    const size_t a = plan_bwd(T, in, out, true, acc).total, b = plan_bwd(T, in, out, false, acc).total;
    return a > b ? a : b;
}

}  // namespace tern
