// Host-side checks of the launch planner (no HIP): every launch whose dW
// epilogue writes the sgrad partial table is refused without that table, and
// a missing operand or output is refused for every product.  Built with g++
// against tern_plan.cpp alone; test infrastructure only.
#include <cstdio>

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
    if (fails) {
        std::fprintf(stderr, "%d checks failed\n", fails);
        return 1;
    }
    std::printf("planner checks passed\n");
    return 0;
}
