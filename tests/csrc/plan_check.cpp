// Host-side checks of the launch planner (no HIP): every launch whose dW
// epilogue writes the sgrad partial table is refused without that table, and
// a missing operand or output is refused for every product.  Built with g++
// against tern_plan.cpp alone; test infrastructure only.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "../../include/tern.h"
#include "../../ternary_weight_linear_tern_amd/csrc/tern_plan.h"

using namespace tern;

static int fails = 0;
#define CHECK(c)                                                          \
    do {                                                                  \
        if (!(c)) {                                                       \
            std::fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
            fails++;                                                      \
        }                                                                 \
    } while (0)

static GemmArgs full_args() {
    static char x[16], y[16], pk[16], sc[16], out[16], part[16], frag[16];
    GemmArgs a{};
    a.act0 = x;
    a.act1 = y;
    a.packed = (const uint32_t *)pk;
    a.frag = (const uint32_t *)frag;
    a.scale = (const float *)sc;
    a.out_ptr = out;
    a.part = (float *)part;
    return a;
}


// Every walk of a group visits every item exactly once: simulate group_item
// for all workgroups of the planned grid.  Returns the walk's makespan in cost
// units (with the 2-step overhead per item).
struct Prob {
    int tiles_m, tiles_n, splits;
    long cost;
};
static long check_walk(const std::vector<Prob> &ps, long cus, int *walk_out = nullptr) {
    GroupArgs ga{};
    ga.n = (int)ps.size();
    long cost[kMaxGroup];
    int total = 0;
    for (int i = 0; i < ga.n; i++) {
        ga.start[i] = total;
        ga.p[i].tiles_m = ps[i].tiles_m;
        ga.p[i].tiles_n = ps[i].tiles_n;
        ga.p[i].splits = ps[i].splits;
        cost[i] = ps[i].cost;
        total += ps[i].tiles_m * ps[i].tiles_n * ps[i].splits;
    }
    ga.start[ga.n] = total;
    int64_t cost64[kMaxGroup];
    for (int i = 0; i < ga.n; i++) cost64[i] = cost[i];
    const int64_t stat = static_makespan(ga, cost64, cus);
    const int64_t grid = plan_group_walk(ga, cost64, cus);
    if (walk_out) *walk_out = ga.walk;
    CHECK(grid > 0 && grid <= (total > cus && ga.walk != WALK_DYNAMIC ? cus : total));
    std::vector<int> seen(total, 0);
    long worst = 0;
    for (int b = 0; b < grid; b++) {
        long load = 0;
        for (int j = 0;; j++) {
            int pi = -1, tm = -1, tn = -1, sp = -1;
            if (!group_item(ga, (int)grid, b, j, pi, tm, tn, sp)) break;
            CHECK(pi >= 0 && pi < ga.n);
            if (pi < 0 || pi >= ga.n) break;
            const Prob &q = ps[pi];
            CHECK(tm >= 0 && tm < q.tiles_m && tn >= 0 && tn < q.tiles_n && sp >= 0 && sp < q.splits);
            if (!(tm >= 0 && tm < q.tiles_m && tn >= 0 && tn < q.tiles_n && sp >= 0 && sp < q.splits)) break;
            seen[ga.start[pi] + (sp * q.tiles_n + tn) * q.tiles_m + tm]++;
            load += q.cost + 2;
            CHECK(j <= total);
            if (j > total) break;
        }
        worst = load > worst ? load : worst;
    }
    for (int i = 0; i < total; i++) CHECK(seen[i] == 1);
    if (ga.walk == WALK_CLASSES) CHECK(worst < stat);
    if (ga.walk == WALK_STATIC && total > cus) CHECK(worst == stat);
    return worst;
}

int main() {
    // shapes that plan one split and several splits of the dW product
    const long shapes[][3] = {{32768, 4096, 4096}, {16384, 2048, 2048}, {4000, 1032, 1032}, {64, 64, 64},
                              {2048, 512, 512}};
    for (auto &s : shapes) {
        for (int bf = 0; bf < 2; bf++) {
            for (int mode = MODE_FWD; mode <= MODE_DW; mode++) {
                const GemmPlan p = plan_gemm(mode, s[0], s[1], s[2], bf);
                CHECK(p.grid > 0);
                GemmArgs a = full_args();
                CHECK(check_gemm_args(p, a) == TERN_OK);
                GemmArgs b = a;
                b.act0 = nullptr;
                CHECK(check_gemm_args(p, b) == TERN_ERR_NULL);
                b = a;
                b.out_ptr = nullptr;
                CHECK(check_gemm_args(p, b) == TERN_ERR_NULL);
                b = a;
                b.scale = nullptr;
                CHECK(check_gemm_args(p, b) == TERN_ERR_NULL);
                b = a;
                b.packed = nullptr;
                CHECK(check_gemm_args(p, b) == TERN_ERR_NULL);
                if (mode == MODE_DW) {
                    b = a;
                    b.act1 = nullptr;
                    CHECK(check_gemm_args(p, b) == TERN_ERR_NULL);
                    // the partial table: required exactly where the epilogue writes it
                    b = a;
                    b.part = nullptr;
                    const bool writes_part = p.splits == 1;
                    CHECK(check_gemm_args(p, b) == (writes_part ? TERN_ERR_WORKSPACE : TERN_OK));
                    b.acc = 1;   // the accumulating variant always writes raw G
                    CHECK(check_gemm_args(p, b) == TERN_OK);
                }
                if (p.tile == TILE_256) {
                    b = a;
                    b.frag = nullptr;
                    CHECK(check_gemm_args(p, b) == TERN_ERR_NULL);
                }
            }
        }
    }
    // an empty grid launches nothing and needs no pointer
    GemmPlan empty = plan_gemm(MODE_DW, 0, 64, 64, true);
    CHECK(empty.grid == 0);
    CHECK(check_gemm_args(empty, GemmArgs{}) == TERN_OK);
    // a workspace limit lowers the split count until the layout fits
    const BwdLayout free_ = plan_bwd(16384, 2048, 2048, true);
    CHECK(free_.dw.splits > 1);
    const BwdLayout capped = plan_bwd(16384, 2048, 2048, true, false, free_.total / 2);
    CHECK(capped.total <= free_.total / 2 && capped.dw.splits < free_.dw.splits);
    const BwdLayout one = plan_bwd(16384, 2048, 2048, true, false, 1);
    CHECK(one.dw.splits == 1);
    // either type's plan fits the three-argument workspace size
    for (auto &s : shapes) {
        const size_t w = bwd_workspace_bytes(s[0], s[1], s[2], false);
        CHECK(plan_bwd(s[0], s[1], s[2], true).total <= w && plan_bwd(s[0], s[1], s[2], false).total <= w);
        const size_t wa = bwd_workspace_bytes(s[0], s[1], s[2], true);
        CHECK(plan_bwd(s[0], s[1], s[2], true, true).total <= wa);
    }
    // item walks: a layer of mixed reduction lengths (d = 1024, ffn 4096,
    // 8192 tokens: forward items of 128 and 32 chunks) takes the classes and
    // reaches the balanced makespan; uniform layers stay static; random
    // groups cover every walk
    {
        int walk = -1;
        const long mid = check_walk({{4, 32, 1, 128}, {16, 32, 1, 32}, {4, 32, 1, 32}, {4, 32, 1, 32},
                                     {4, 32, 1, 32}, {4, 32, 1, 32}}, 256, &walk);
        CHECK(walk == WALK_CLASSES);
        CHECK(mid == 204);
        check_walk({{8, 64, 1, 256}, {32, 64, 1, 64}, {8, 64, 1, 64}, {8, 64, 1, 64}, {8, 64, 1, 64},
                    {8, 64, 1, 64}}, 256, &walk);
        CHECK(walk == WALK_STATIC);
        check_walk({{4, 4, 1, 128}, {16, 4, 1, 128}}, 256, &walk);   // fewer items than units
        CHECK(walk == WALK_STATIC);
        std::srand(12345);
        int walks[3] = {0, 0, 0};
        for (int it = 0; it < 3000; it++) {
            std::vector<Prob> ps;
            const int n = 1 + std::rand() % kMaxGroup;
            for (int i = 0; i < n; i++)
                ps.push_back({1 + std::rand() % 40, 1 + std::rand() % 40, 1 + std::rand() % 3, 1 + std::rand() % 300});
            const long cus_opts[] = {1, 7, 8, 80, 256, 304};
            check_walk(ps, cus_opts[std::rand() % 6], &walk);
            if (walk >= 0 && walk < 3) walks[walk]++;
        }
        CHECK(walks[WALK_STATIC] > 0 && walks[WALK_DYNAMIC] + walks[WALK_CLASSES] > 0 && walks[WALK_CLASSES] > 0);
        std::printf("walks over random groups: static %d, dynamic %d, classes %d\n", walks[0], walks[1], walks[2]);
    }
    // forward / dX items: 512 x 128 tiles (columns x tokens) unless their
    // column padding costs more than 3 % over 256 x 256 tiles, 256 x 256 for
    // the accumulating dX; ragged edges round up; too many items are refused
    {
        GroupArgs ga{};
        ga.n = 2;
        ga.p[0].M = 2048; ga.p[0].N = 4000; ga.p[0].K = 2048; ga.p[0].splits = 1;
        ga.p[1].M = 512; ga.p[1].N = 128; ga.p[1].K = 512; ga.p[1].splits = 1;
        CHECK(rd_items(ga));
        CHECK(ga.rd_wide == 1);
        CHECK(ga.p[0].tiles_m == 4 && ga.p[0].tiles_n == 32 && ga.p[1].tiles_m == 1 && ga.p[1].tiles_n == 1);
        CHECK(ga.start[0] == 0 && ga.start[1] == 128 && ga.start[2] == 129);
        ga.p[0].M = 1032;   // 1536 padded columns against 1280: square tiles
        CHECK(rd_items(ga));
        CHECK(ga.rd_wide == 0);
        CHECK(ga.p[0].tiles_m == 5 && ga.p[0].tiles_n == 16 && ga.p[1].tiles_m == 2 && ga.p[1].tiles_n == 1);
        CHECK(ga.start[1] == 80 && ga.start[2] == 82);
        ga.p[0].M = 768; ga.p[0].K = 1;   // 768 columns pad to 1024 wide, but that problem is light
        ga.p[1].M = 4096; ga.p[1].N = 8192; ga.p[1].K = 4096;
        CHECK(rd_items(ga));
        CHECK(ga.rd_wide == 1);
        ga.p[0].M = 2048; ga.p[0].K = 2048;
        ga.p[0].acc = ga.p[1].acc = 1;
        CHECK(rd_items(ga));
        CHECK(ga.rd_wide == 0 && ga.p[0].tiles_m == 8 && ga.p[0].tiles_n == 16);
        ga.n = 1;
        ga.p[0].acc = 0; ga.p[0].M = 1 << 20; ga.p[0].N = 2147483647;
        CHECK(!rd_items(ga));
        // the mid layer's forward on these tiles (d = 1024: 2 x 64 items; ffn
        // 8 x 64 and 2 x 64 with 128 chunks) walks every item once
        int walk = -1;
        check_walk({{2, 64, 1, 128}, {8, 64, 1, 32}, {2, 64, 1, 32}, {2, 64, 1, 32}, {2, 64, 1, 32},
                    {2, 64, 1, 32}}, 256, &walk);
        CHECK(walk == WALK_CLASSES || walk == WALK_STATIC);
    }
    if (fails) {
        std::fprintf(stderr, "%d checks failed\n", fails);
        return 1;
    }
    std::printf("planner checks passed\n");
    return 0;
}
