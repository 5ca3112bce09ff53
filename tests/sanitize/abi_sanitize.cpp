// Host-side checks of libfp8bs's planner and C ABI argument validation, built with
// AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_sanitize_host.py builds and
// runs it; no GPU is needed).  The kernel launcher is replaced by a stand-in that checks
// the launch it is asked for against the plan and launches nothing, so every entry point's
// argument checks, planning and parameter marshalling run under the sanitizers.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "fp8bs.h"
#include "fp8bs_internal.h"

static int g_checks = 0, g_fails = 0;
#define CHECK(cond)                                                                       \
    do {                                                                                  \
        ++g_checks;                                                                       \
        if (!(cond)) {                                                                    \
            ++g_fails;                                                                    \
            fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond);               \
        }                                                                                 \
    } while (0)

static int g_launches = 0;

namespace fp8bs {
// Stand-in for the device launcher: the plan and the kernel parameters must agree.
int launch_instance(const Plan& plan, int layout, int scale_mode, const GemmParams& p,
                    hipStream_t, int form) {
    ++g_launches;
    CHECK(plan.instance >= 0 && plan.instance < kNumInstances);
    CHECK(layout >= kDense && layout <= kKGrouped);
    CHECK(scale_mode == kScaleF32 || scale_mode == kScaleUE8M0);
    CHECK(form >= kFormNT && form <= kFormTT);
    CHECK(p.splits == plan.splits && p.tiles == plan.tiles);
    CHECK(p.units >= p.tiles * p.splits);
    CHECK(plan.grid >= 1 && plan.grid <= p.units);
    CHECK(p.m_blocks == (p.m + plan.shape.block_m - 1) / plan.shape.block_m);
    CHECK(p.n_blocks == (p.n + plan.shape.block_n - 1) / plan.shape.block_n);
    CHECK(p.splits == 1 || p.ws != nullptr);
    return 0;
}
}  // namespace fp8bs

static void plan_grid() {
    const int64_t ms[] = {0, 1, 17, 64, 128, 255, 256, 1000, 4096, 33152};
    const int ns[] = {1, 16, 100, 2112, 7168};
    const int ks[] = {0, 100, 128, 512, 7168};
    const int gs[] = {1, 8};
    const int cus[] = {1, 132, 256};
    const int64_t wss[] = {0, 1 << 20, INT64_MAX};
    for (int code = 0; code <= 6; ++code)
        for (int e8 = 0; e8 < 2; ++e8)
            for (int64_t m : ms)
                for (int n : ns)
                    for (int k : ks)
                        for (int g : gs)
                            for (int c : cus)
                                for (int64_t ws : wss) {
                                    fp8bs_plan pl;
                                    memset(&pl, 0xA5, sizeof pl);
                                    const int lc = code | (e8 ? FP8BS_LAYOUT_UE8M0 : 0);
                                    const int st = fp8bs_plan_query(lc, m, n, k, g, m / 2, c, ws, &pl);
                                    CHECK(st >= FP8BS_OK && st <= FP8BS_ERR_HIP);
                                    if (st != FP8BS_OK) continue;
                                    CHECK(pl.instance >= 0 && pl.instance < fp8bs_num_instances());
                                    CHECK(pl.block_m > 0 && pl.block_n > 0 && pl.threads > 0);
                                    CHECK(pl.splits >= 1 && pl.grid >= 1);
                                    CHECK(pl.workspace_bytes >= 0 && pl.workspace_bytes <= ws);
                                    CHECK((pl.splits == 1) == (pl.workspace_bytes == 0));
                                    CHECK(!e8 || pl.ue8m0 == 1);
                                    const int64_t t = fp8bs_count_tiles(lc, m, n, g, pl.block_m, pl.block_n);
                                    CHECK(t == pl.tiles);
                                }
}

static void helpers() {
    CHECK(fp8bs_get_mk_alignment() == 128);
    CHECK(fp8bs_get_sfa_ld(-1) == -1 && fp8bs_get_sfa_ld(0) == 0 && fp8bs_get_sfa_ld(5) == 8);
    for (int s = -2; s < 8; ++s) CHECK(fp8bs_status_string(s) != nullptr);
    CHECK(fp8bs_count_tiles(9, 10, 10, 1, 16, 16) == -1);
    CHECK(fp8bs_count_tiles(0, -1, 10, 1, 16, 16) == -1);
    fp8bs_plan pl;
    CHECK(fp8bs_instance_info(-1, &pl) == FP8BS_ERR_UNSUPPORTED);
    CHECK(fp8bs_instance_info(fp8bs_num_instances(), &pl) == FP8BS_ERR_UNSUPPORTED);
    CHECK(fp8bs_instance_info(0, nullptr) == FP8BS_ERR_POINTER);
    for (int i = 0; i < fp8bs_num_instances(); ++i) {
        CHECK(fp8bs_instance_info(i, &pl) == FP8BS_OK);
        CHECK(pl.lds_bytes > 0 && pl.lds_bytes <= 160 * 1024);
    }
    CHECK(fp8bs_plan_query(0, 64, 64, 128, 1, 0, 256, 0, nullptr) == FP8BS_ERR_POINTER);
    CHECK(fp8bs_plan_query(7, 64, 64, 128, 1, 0, 256, 0, &pl) == FP8BS_ERR_UNSUPPORTED);
    CHECK(fp8bs_plan_query(0, 64, 64, 128, 1, 0, 0, 0, &pl) == FP8BS_ERR_UNSUPPORTED);
    CHECK(fp8bs_set_num_cus(-1) == -1);
    CHECK(fp8bs_force_instance(-5) == -2 && fp8bs_force_splits(-1) == -1);
    char buf[8];
    CHECK(fp8bs_describe_config(0, 64, 64, 128, 1, 0, nullptr, 8) == FP8BS_ERR_POINTER);
    CHECK(fp8bs_describe_config(99, 64, 64, 128, 1, 0, buf, sizeof buf) == FP8BS_ERR_UNSUPPORTED);
}

// Entry points: invalid requests are refused before any device query; empty requests are
// accepted without touching a pointer; valid requests plan on the current device (without
// one: FP8BS_ERR_HIP) and then reach the launcher stand-in.
static void entry_points() {
    alignas(16) static unsigned char buf[4096];
    void* f = buf;
    void* odd = buf + 4;
    const int have_dev = fp8bs_workspace_size(0, 64, 64, 128, 1, 0) >= 0;
    const int ok_or_hip = have_dev ? FP8BS_OK : FP8BS_ERR_HIP;
    int before = g_launches;
    // dense
    CHECK(fp8bs_dense_nt(f, (float*)f, f, (float*)f, f, 64, 64, 100, nullptr) == FP8BS_ERR_SHAPE);
    CHECK(fp8bs_dense_nt(f, (float*)f, f, (float*)f, f, 64, 0, 128, nullptr) == FP8BS_ERR_SHAPE);
    CHECK(fp8bs_dense_nt(f, (float*)f, f, (float*)f, odd, 64, 64, 128, nullptr) == FP8BS_ERR_POINTER);
    CHECK(fp8bs_dense_nt(nullptr, nullptr, nullptr, nullptr, nullptr, 0, 64, 128, nullptr) == FP8BS_OK);
    CHECK(fp8bs_dense_nt(f, (float*)f, f, (float*)f, f, 64, 64, 128, nullptr) == ok_or_hip);
    CHECK(fp8bs_dense_nt_ws(f, (float*)f, f, (float*)f, f, 64, 64, 128, odd, 64, nullptr) ==
          FP8BS_ERR_POINTER);
    CHECK(fp8bs_dense_nt_noalloc(f, (float*)f, f, (float*)f, f, 64, 64, 100, nullptr) ==
          FP8BS_ERR_SHAPE);
    CHECK(fp8bs_dense_nt_noalloc(nullptr, nullptr, nullptr, nullptr, nullptr, 0, 64, 128, nullptr) ==
          FP8BS_OK);
    // contiguous: m_total a multiple of 128, grouped_layout present
    CHECK(fp8bs_grouped_contiguous_nt(f, (float*)f, f, (float*)f, f, (int32_t*)f, 100, 64, 128, 2,
                                      nullptr) == FP8BS_ERR_SHAPE);
    CHECK(fp8bs_grouped_contiguous_nt(f, (float*)f, f, (float*)f, f, nullptr, 128, 64, 128, 2,
                                      nullptr) == FP8BS_ERR_POINTER);
    CHECK(fp8bs_grouped_contiguous_nt(f, (float*)f, f, (float*)f, f, (int32_t*)f, 128, 64, 128, 2,
                                      nullptr) == ok_or_hip);
    // masked
    CHECK(fp8bs_grouped_masked_nt(f, (float*)f, f, (float*)f, f, (int32_t*)f, 0, 64, 0, 64, 128,
                                  nullptr) == FP8BS_ERR_SHAPE);
    CHECK(fp8bs_grouped_masked_nt(f, (float*)f, f, (float*)f, f, nullptr, 2, 64, 0, 64, 128,
                                  nullptr) == FP8BS_ERR_POINTER);
    CHECK(fp8bs_grouped_masked_nt(f, (float*)f, f, (float*)f, f, (int32_t*)f, 2, 64, 32, 64, 128,
                                  nullptr) == ok_or_hip);
    // addend, UE8M0 and stored forms
    CHECK(fp8bs_dense_nt_c(f, (float*)f, f, (float*)f, (float*)odd, f, 64, 64, 128, nullptr, 0,
                           nullptr) == FP8BS_ERR_POINTER);
    CHECK(fp8bs_dense_nt_ue8m0(f, (int32_t*)f, f, (int32_t*)f, f, 64, 64, 128, nullptr, 0,
                               nullptr) == ok_or_hip);
    CHECK(fp8bs_dense_nn(f, (float*)f, f, (float*)f, nullptr, f, 64, 24, 128, nullptr, 0, nullptr) ==
          FP8BS_ERR_SHAPE);                             // stored [k][n] needs n % 16 == 0
    CHECK(fp8bs_dense_tn(f, (float*)f, f, (float*)f, nullptr, f, 24, 64, 128, nullptr, 0, nullptr) ==
          FP8BS_ERR_SHAPE);                             // stored [k][m] needs m % 16 == 0
    CHECK(fp8bs_dense_tt(f, (float*)f, f, (float*)f, nullptr, f, 64, 64, 128, nullptr, 0, nullptr) ==
          ok_or_hip);
    // K-grouped: host group sizes, multiples of 128 adding up to k_total
    int32_t ks_bad[2] = {128, 100}, ks_sum[2] = {128, 128}, ks_ok[2] = {128, 0};
    CHECK(fp8bs_k_grouped_tn_contiguous(f, (float*)f, f, (float*)f, nullptr, (float*)f, ks_bad, 2,
                                        64, 64, 228, nullptr, 0, nullptr) == FP8BS_ERR_SHAPE);
    CHECK(fp8bs_k_grouped_tn_contiguous(f, (float*)f, f, (float*)f, nullptr, (float*)f, ks_sum, 2,
                                        64, 64, 128, nullptr, 0, nullptr) == FP8BS_ERR_SHAPE);
    CHECK(fp8bs_k_grouped_tn_contiguous(f, (float*)f, f, (float*)f, nullptr, (float*)f, nullptr, 2,
                                        64, 64, 128, nullptr, 0, nullptr) == FP8BS_ERR_POINTER);
    CHECK(fp8bs_k_grouped_tn_contiguous(f, (float*)f, f, (float*)f, nullptr, (float*)f, ks_ok, 2,
                                        64, 64, 128, nullptr, 0, nullptr) == ok_or_hip);
    std::vector<int32_t> many(300, 128);
    CHECK(fp8bs_k_grouped_tn_contiguous(f, (float*)f, f, (float*)f, nullptr, (float*)f, many.data(),
                                        300, 64, 64, 300 * 128, nullptr, 0, nullptr) ==
          FP8BS_ERR_SHAPE);                              // at most 256 groups
    // sizes whose byte offsets would leave 32 bits are refused
    CHECK(fp8bs_dense_nt(f, (float*)f, f, (float*)f, f, 1 << 20, 64, 1 << 13, nullptr) ==
          FP8BS_ERR_SHAPE);
    if (!have_dev) CHECK(g_launches == before);         // nothing got past planning
    else CHECK(g_launches > before);
    // workspace queries
    CHECK(fp8bs_workspace_size(0, 64, 64, 100, 1, 0) == -FP8BS_ERR_SHAPE);
    CHECK(fp8bs_workspace_size(0, 0, 64, 128, 1, 0) == 0);
    CHECK(fp8bs_noalloc_scratch_bytes() == FP8BS_NOALLOC_SCRATCH_BYTES);
}

int main() {
    plan_grid();
    helpers();
    entry_points();
    printf("abi_sanitize: %d checks, %d failed, %d launches\n", g_checks, g_fails, g_launches);
    return g_fails == 0 ? 0 : 1;
}
