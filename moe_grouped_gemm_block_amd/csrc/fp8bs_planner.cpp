// fp8bs_planner.cpp -- host planner of libfp8bs: validation and the
// deterministic choice of tile shape and persistent launch shape.  No device
// access, so it runs (and is tested) on any host.
//
// The choice is made without autotuning, from the sizes alone, as the
// DeepGEMM README repost (lqnn.cn/news/60274, "优化技术 / 完全JIT设计") describes
// for its block sizes; tile shapes include non-power-of-two BLOCK_N so that
// the tile count fills the machine ("非对齐块大小": M=256, N=7168 gives 112
// tiles of 128x128 on 132 SMs but 128 tiles with BLOCK_N = 112).  Here the
// machine has 256 CUs and the model below scores each compiled shape.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "fp8bs_internal.h"

namespace fp8bs {

#define FP8BS_INSTANCE(BM, BN, WM, WN, OCC, CNS, TNS) \
    {BM, BN, WM, WN, OCC, kStages * stage_bytes(BM, BN), CNS, TNS},
const InstanceShape kInstances[] = {
#include "fp8bs_instances.inc"
};
#undef FP8BS_INSTANCE
const int kNumInstances = (int)(sizeof(kInstances) / sizeof(kInstances[0]));

int validate_sizes(int layout, int64_t m, int n, int k, int num_groups) {
    if (k < 128 || k % 128 != 0) return FP8BS_ERR_SHAPE;
    if (n < 1 || m < 0) return FP8BS_ERR_SHAPE;
    if (layout == kContiguous && m % 128 != 0) return FP8BS_ERR_SHAPE;
    if (layout != kDense && num_groups < 1) return FP8BS_ERR_SHAPE;
    if (layout == kDense && num_groups != 1) return FP8BS_ERR_SHAPE;
    if (m > (int64_t)0x7fffffff) return FP8BS_ERR_SHAPE;
    // copies address one A slot (m x k bytes) and one B group (n x k bytes) with 32-bit offsets
    if ((double)m * k >= 4294967296.0 || (double)n * k >= 4294967296.0) return FP8BS_ERR_SHAPE;
    // element offsets are 64-bit in the kernels; keep every operand below 2^62 bytes
    const double rows = (double)m * (layout == kMasked ? num_groups : 1);
    if (rows * k > 4.0e18 || rows * n * 2.0 > 4.0e18 || (double)num_groups * n * k > 4.0e18)
        return FP8BS_ERR_SHAPE;
    return FP8BS_OK;
}

// Cost model (nanoseconds).  A CU works through ceil(tiles / CUs) tiles, each costing
// chunks * chunk_ns + tile_ns (measured per instance); the whole chip cannot beat
// reading every operand byte once from HBM; and a launch that leaves CUs idle keeps
// fewer loads in flight, so under-fill is penalised.
static const double kHbmBytesPerNs = 8.0e12 / 1.0e9;

static void fill_launch(int i, int layout, int64_t m, int n, int num_groups, int num_cus,
                        Plan* out) {
    const InstanceShape& s = kInstances[i];
    const int64_t m_blocks = (m + s.block_m - 1) / s.block_m;
    const int64_t n_blocks = ((int64_t)n + s.block_n - 1) / s.block_n;
    const int64_t tiles = (layout == kMasked ? num_groups : 1) * m_blocks * n_blocks;
    const int64_t slots = (int64_t)num_cus * s.wg_per_cu;
    int64_t grid = tiles < slots ? tiles : slots;
    if (grid < 1) grid = 1;
    out->instance = i;
    out->shape = s;
    out->tiles = tiles;
    out->grid = grid;
    const int64_t raster = m_blocks < 8 ? m_blocks : 8;
    out->raster = raster < 1 ? 1 : (int)raster;
}

int plan_instance(int instance, int layout, int64_t m, int n, int num_groups, int num_cus,
                  Plan* out) {
    if (instance < 0 || instance >= kNumInstances || num_cus < 1) return FP8BS_ERR_UNSUPPORTED;
    const InstanceShape& s = kInstances[instance];
    if (layout == kContiguous && 128 % s.block_m != 0) return FP8BS_ERR_UNSUPPORTED;
    const int64_t tiles = (layout == kMasked ? num_groups : 1) * ((m + s.block_m - 1) / s.block_m) *
                          (((int64_t)n + s.block_n - 1) / s.block_n);
    if (tiles > 0x7fffffff) return FP8BS_ERR_UNSUPPORTED;
    fill_launch(instance, layout, m, n, layout == kMasked ? num_groups : 1, num_cus, out);
    return FP8BS_OK;
}

int plan_request(int layout, int64_t m, int n, int k, int num_groups, int expected_m,
                 int num_cus, Plan* out) {
    int st = validate_sizes(layout, m, n, k, layout == kDense ? 1 : num_groups);
    if (st != FP8BS_OK) return st;
    if (num_cus < 1) return FP8BS_ERR_UNSUPPORTED;
    const int G = layout == kDense ? 1 : num_groups;
    int64_t eff_rows = m;                        // rows per group the estimate assumes
    if (layout == kMasked && expected_m > 0 && expected_m < m) eff_rows = expected_m;
    // masked: expected_m is read as the mean of masked_m, spread uniformly over
    // 1 .. min(2 * expected_m, max_m); a group costs E[ceil(masked_m / block_m)] m-blocks
    const int64_t spread = layout == kMasked && expected_m > 0
                               ? (2 * (int64_t)expected_m < m ? 2 * (int64_t)expected_m : m)
                               : 0;
    double best_t = 0;
    int best = -1;
    Plan best_plan = {};
    for (int i = 0; i < kNumInstances; ++i) {
        const InstanceShape& s = kInstances[i];
        if (layout == kContiguous && 128 % s.block_m != 0) continue;
        const int64_t m_blocks = (m + s.block_m - 1) / s.block_m;
        const int64_t n_blocks = ((int64_t)n + s.block_n - 1) / s.block_n;
        const int64_t tiles = (layout == kMasked ? G : 1) * m_blocks * n_blocks;
        if (tiles > 0x7fffffff) continue;
        double eff_m_blocks = (double)((eff_rows + s.block_m - 1) / s.block_m);
        if (spread > 0) {                          // mean of ceil(x / block_m), x = 1 .. spread
            const int64_t full = spread / s.block_m, rest = spread % s.block_m;
            double sum = (double)s.block_m * full * (full + 1) / 2.0;
            sum += (double)rest * (full + 1);
            eff_m_blocks = sum / spread;
        }
        const int64_t eff_tiles =
            (int64_t)ceil((layout == kMasked ? G : 1) * eff_m_blocks * n_blocks - 1e-9);
        // the schedule is static: tiles (skipped ones included) are dealt round-robin, so a
        // CU may be handed ceil(tiles / CUs) tiles that all hold valid rows
        const int64_t per_cu = (tiles + num_cus - 1) / num_cus;
        const double bytes = (double)G * eff_rows * k + (double)G * n * k + (double)G * eff_rows * n * 2;
        const double t_hbm = bytes / kHbmBytesPerNs;
        double t = per_cu * ((k / 128) * (double)s.chunk_ns + s.tile_ns);
        if (t < t_hbm) t = t_hbm;
        const double fill = (double)(eff_tiles < num_cus ? eff_tiles : num_cus) / num_cus;
        t *= 1.0 + 0.1 * (1.0 - fill);
        if (best < 0 || t < best_t * (1.0 - 1e-9)) {
            best = i;
            best_t = t;
            fill_launch(i, layout, m, n, G, num_cus, &best_plan);
        }
    }
    if (best < 0) return FP8BS_ERR_UNSUPPORTED;
    *out = best_plan;
    return FP8BS_OK;
}

}  // namespace fp8bs

extern "C" int fp8bs_plan_query(int layout, int64_t m, int n, int k, int num_groups,
                                int expected_m, int num_cus, fp8bs_plan* out) {
    if (!out) return FP8BS_ERR_POINTER;
    if (layout < 0 || layout > 2) return FP8BS_ERR_UNSUPPORTED;
    fp8bs::Plan p;
    int st = fp8bs::plan_request(layout, m, n, k, layout == 0 ? 1 : num_groups, expected_m,
                                 num_cus, &p);
    if (st != FP8BS_OK) return st;
    out->block_m = p.shape.block_m;
    out->block_n = p.shape.block_n;
    out->waves_m = p.shape.waves_m;
    out->waves_n = p.shape.waves_n;
    out->threads = 64 * p.shape.waves_m * p.shape.waves_n;
    out->lds_bytes = p.shape.lds_bytes;
    out->wg_per_cu = p.shape.wg_per_cu;
    out->tiles = p.tiles;
    out->grid = p.grid;
    out->raster = p.raster;
    out->instance = p.instance;
    return FP8BS_OK;
}

extern "C" int64_t fp8bs_count_tiles(int layout, int64_t m, int n, int num_groups, int block_m,
                                     int block_n) {
    if (layout < 0 || layout > 2 || m < 0 || n < 1 || block_m < 1 || block_n < 1) return -1;
    if (layout == fp8bs::kMasked && num_groups < 1) return -1;
    const int64_t mb = (m + block_m - 1) / block_m;
    const int64_t nb = ((int64_t)n + block_n - 1) / block_n;
    return (layout == fp8bs::kMasked ? num_groups : 1) * mb * nb;
}

extern "C" int fp8bs_num_instances(void) { return fp8bs::kNumInstances; }

extern "C" int fp8bs_instance_info(int i, fp8bs_plan* out) {
    if (!out) return FP8BS_ERR_POINTER;
    if (i < 0 || i >= fp8bs::kNumInstances) return FP8BS_ERR_UNSUPPORTED;
    const fp8bs::InstanceShape& s = fp8bs::kInstances[i];
    *out = fp8bs_plan{};
    out->block_m = s.block_m;
    out->block_n = s.block_n;
    out->waves_m = s.waves_m;
    out->waves_n = s.waves_n;
    out->threads = 64 * s.waves_m * s.waves_n;
    out->lds_bytes = s.lds_bytes;
    out->wg_per_cu = s.wg_per_cu;
    out->instance = i;
    return FP8BS_OK;
}

extern "C" const char* fp8bs_status_string(int status) {
    switch (status) {
        case FP8BS_OK: return "ok";
        case FP8BS_ERR_SHAPE: return "invalid shape (K must be a positive multiple of 128, "
                                     "m_total a multiple of 128, sizes positive)";
        case FP8BS_ERR_POINTER: return "NULL or misaligned (not 16-byte) pointer";
        case FP8BS_ERR_UNSUPPORTED: return "no compiled kernel instance covers the request";
        case FP8BS_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

extern "C" int fp8bs_get_mk_alignment(void) { return 128; }

extern "C" int64_t fp8bs_get_sfa_ld(int64_t rows) {
    if (rows < 0) return -1;
    return (rows + 3) / 4 * 4;
}
