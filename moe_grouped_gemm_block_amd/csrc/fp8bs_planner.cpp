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

#define FP8BS_INSTANCE(KIND, BM, BN, WM, WN, NS, OCC, CNS, TNS, SCNS, STNS, E8, MN, MNE8) \
    {KIND, BM, BN, WM, WN, NS, OCC, instance_lds_bytes(KIND, BM, BN, NS), CNS, TNS, SCNS, STNS, E8, MN, MNE8},
const InstanceShape kInstances[] = {
#include "fp8bs_instances.inc"
};
#undef FP8BS_INSTANCE
const int kNumInstances = (int)(sizeof(kInstances) / sizeof(kInstances[0]));

bool decode_layout(int code, int* layout, int* form, int* scale_mode) {
    static const int table[7][2] = {{kDense, kFormNT},     {kContiguous, kFormNT},
                                    {kMasked, kFormNT},    {kKGrouped, kFormTN},
                                    {kDense, kFormNN},     {kDense, kFormTN},
                                    {kDense, kFormTT}};
    const bool e8 = (code & FP8BS_LAYOUT_UE8M0) != 0;
    code &= ~FP8BS_LAYOUT_UE8M0;
    if (code < 0 || code > 6) return false;
    *layout = table[code][0];
    *form = table[code][1];
    if (scale_mode) *scale_mode = e8 ? kScaleUE8M0 : kScaleF32;
    return true;
}

int validate_sizes(int layout, int64_t m, int n, int k, int num_groups, int form) {
    if (layout == kKGrouped) {
        // A [K_total][M], B [K_total][N]: MN-major rows are copied in 16-byte units
        if (k < 0 || k % 128 != 0) return FP8BS_ERR_SHAPE;
        if (m < 16 || m % 16 != 0 || n < 16 || n % 16 != 0) return FP8BS_ERR_SHAPE;
        if (num_groups < 1 || num_groups > kMaxKGroups) return FP8BS_ERR_SHAPE;
        if (m > (int64_t)0x7fffffff || (double)m * 128 * 2 >= 4294967296.0 ||
            (double)n * 128 * 2 >= 4294967296.0)
            return FP8BS_ERR_SHAPE;
        if ((double)num_groups * m * n * 4.0 > 4.0e18 || (double)k * (m + n) > 4.0e18)
            return FP8BS_ERR_SHAPE;
        return FP8BS_OK;
    }
    if (form != kFormNT && layout != kDense) return FP8BS_ERR_UNSUPPORTED;
    if (form_a_mn(form) && m % 16 != 0) return FP8BS_ERR_SHAPE;
    if (form_b_mn(form) && n % 16 != 0) return FP8BS_ERR_SHAPE;
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

int64_t split_workspace_bytes(const InstanceShape& shape, int64_t tiles, int splits) {
    if (splits <= 1) return 0;
    return tiles * splits * (int64_t)shape.block_m * shape.block_n * 4;
}

// Cost model (nanoseconds).  The persistent grid deals work units (tile, K split)
// round-robin, so a CU works through ceil(units / CUs) units, each costing
// chunks_per_unit * chunk_ns + tile_ns (measured per instance); the whole chip cannot beat
// reading every operand byte once from HBM (plus the FP32 partials of a split launch,
// written once and read once); a split launch adds the reduction kernel; and a launch
// that leaves CUs idle keeps fewer loads in flight, so under-fill is penalised.
static const double kHbmBytesPerNs = 8.0e12 / 1.0e9;
// second launch: fitted to traced cold decode calls (3.2 us + bytes / 9 TB/s), with the
// fixed part raised to cover the gap between the two dispatches
static const double kReduceFixedNs = 5000.0;
static const double kReduceBytesPerNs = 9.0e12 / 1.0e9;
static const int kMaxSplits = 16;
static const double kRidgeFlopPerByte = 629.0;       // dense FP8 MFMA peak / HBM bandwidth
// dense: measured on the M=128 and decode shapes, where the B-streaming tiles won every
// comparison; grouped layouts: the masked MoE shapes, where the 256x256 staged tile (B read
// once per slot) beats every B-streaming tile by 1.6x
static const double kStagedStreamingBias = 2.0;
static const double kStagedStreamingBiasGrouped = 1.25;

namespace {

struct Request {
    int layout;
    int form;
    int scale_mode;
    int64_t m;
    int n, k, G;
    int64_t eff_rows;    // rows per group the estimate assumes
    int64_t spread;      // masked: masked_m assumed uniform over 1 .. spread (0: off)
    int num_cus;
    int64_t workspace_bytes;
};

Request make_request(int layout, int64_t m, int n, int k, int num_groups, int expected_m,
                     int num_cus, int64_t workspace_bytes, int form, int scale_mode) {
    Request r;
    r.layout = layout;
    r.scale_mode = scale_mode;
    r.form = layout == kKGrouped ? kFormTN : form;
    r.m = m;
    r.n = n;
    r.k = k;
    r.G = layout == kDense ? 1 : num_groups;
    r.eff_rows = m;
    if (layout == kMasked && expected_m > 0 && expected_m < m) r.eff_rows = expected_m;
    // masked: expected_m is read as the mean of masked_m, spread uniformly over
    // 1 .. min(2 * expected_m, max_m); a group costs E[ceil(masked_m / block_m)] m-blocks
    r.spread = layout == kMasked && expected_m > 0
                   ? (2 * (int64_t)expected_m < m ? 2 * (int64_t)expected_m : m)
                   : 0;
    r.num_cus = num_cus;
    r.workspace_bytes = workspace_bytes < 0 ? 0 : workspace_bytes;
    return r;
}

int64_t tile_count(const Request& r, const InstanceShape& s) {
    const int64_t m_blocks = (r.m + s.block_m - 1) / s.block_m;
    const int64_t n_blocks = ((int64_t)r.n + s.block_n - 1) / s.block_n;
    return (r.layout == kMasked || r.layout == kKGrouped ? r.G : 1) * m_blocks * n_blocks;
}

bool instance_fits(const Request& r, const InstanceShape& s) {
    // MN-major operands (nn / tn / tt, K-grouped) need an instance compiled for them
    if ((r.form != kFormNT || r.layout == kKGrouped) && !s.mn) return false;
    // a contiguous-layout tile lies inside one 128-row expert block, or covers exactly two
    // (then each tile runs in two passes, one per expert)
    return !(r.layout == kContiguous && 128 % s.block_m != 0 && s.block_m != 256);
}

// Estimated time of instance s with `splits` K splits; < 0 when infeasible.
double estimate(const Request& r, const InstanceShape& s, int splits) {
    // K-grouped: a tile's chunks are its group's, on average K_total / 128 / G
    const bool kg = r.layout == kKGrouped;
    int kchunks = r.k / 128;
    if (kg) {
        kchunks = (kchunks + r.G - 1) / r.G;
        if (kchunks < 1) kchunks = 1;
    }
    // (K-grouped: any split count up to the total chunk count runs -- splits beyond a
    // group's chunks are empty units -- but the estimate uses the mean group)
    const int max_splits = kg ? (r.k / 128 > 1 ? r.k / 128 : 1) : kchunks;
    if (splits < 1 || splits > max_splits) return -1.0;
    // the kernels compute split bounds as splits x chunks in 32 bits
    if ((int64_t)splits * (r.k / 128) >= ((int64_t)1 << 32)) return -1.0;
    // two-pass contiguous tiles are never split
    const int passes = passes_per_tile(r.layout, s.block_m);
    if (passes > 1 && splits > 1) return -1.0;
    const int64_t tiles = tile_count(r, s);
    // unit indices (and unit + grid) stay well inside int
    if (tiles * splits * passes_per_tile(r.layout, s.block_m) > 0x7f000000) return -1.0;
    if (split_workspace_bytes(s, tiles, splits) > r.workspace_bytes) return -1.0;
    const int64_t n_blocks = ((int64_t)r.n + s.block_n - 1) / s.block_n;
    double eff_m_blocks = (double)((r.eff_rows + s.block_m - 1) / s.block_m);
    if (r.spread > 0) {                          // mean of ceil(x / block_m), x = 1 .. spread
        const int64_t full = r.spread / s.block_m, rest = r.spread % s.block_m;
        double sum = (double)s.block_m * full * (full + 1) / 2.0;
        sum += (double)rest * (full + 1);
        eff_m_blocks = sum / r.spread;
    }
    const double eff_tiles = (r.layout == kMasked || kg ? r.G : 1) * eff_m_blocks * n_blocks;
    // a second pass runs only for a tile whose two blocks hold different experts: about
    // one tile in 32 for segments of thousands of rows
    const int64_t units = passes > 1 ? tiles + (tiles + 31) / 32 : tiles * splits;
    int64_t per_cu = (units + r.num_cus - 1) / r.num_cus;
    const int64_t chunks_per_unit = (kchunks + splits - 1) / splits;
    // Operands stream from HBM when a byte of A or B feeds fewer flops than the chip's
    // ridge point (MFMA peak / HBM bandwidth): 2 x rows x N / (rows + N) flops per byte.
    const bool streaming =
        2.0 * (double)r.eff_rows * r.n / ((double)r.eff_rows + r.n) < kRidgeFlopPerByte;
    // The compute-regime chunk cost is the CU's throughput with wg_per_cu workgroups
    // sharing it; a workgroup alone on its CU (fewer units than CUs) is not faster per
    // chunk than that (measured on MI355X: the 128x128 two-workgroup tile takes 1.37-1.41 us
    // per chunk alone, twice its shared-CU cost).
    if (!streaming && per_cu < s.wg_per_cu) per_cu = s.wg_per_cu;
    const double c_ns = streaming ? s.stream_chunk_ns : s.chunk_ns;
    const double t_ns = streaming ? s.stream_tile_ns : s.tile_ns;
    double t = per_cu * (chunks_per_unit * c_ns + t_ns);
    // The staged kernels' streaming-regime fit is loose (their direct-to-LDS copies slow
    // down unevenly as they miss in L2); measured, they lose to the B-streaming kernel
    // unless the model favours them by a wide margin.
    if (streaming && s.kind == kStaged)
        t *= r.layout == kDense ? kStagedStreamingBias : kStagedStreamingBiasGrouped;
    if (kg)                                      // measured K-grouped cost of the instance
        t *= (r.scale_mode == kScaleUE8M0 ? s.mn_e8 : s.mn) / 100.0;
    const double d_bytes = (double)r.G * r.eff_rows * r.n * (kg ? 4 : 2);
    double bytes = kg ? (double)r.k * (r.m + r.n) + d_bytes
                      : (double)r.G * r.eff_rows * r.k + (double)r.G * r.n * r.k + d_bytes;
    const double partial_bytes = splits > 1 ? eff_tiles * splits * s.block_m * s.block_n * 4.0 : 0.0;
    bytes += 2.0 * partial_bytes;
    const double t_hbm = bytes / kHbmBytesPerNs;
    if (t < t_hbm) t = t_hbm;
    const double eff_units = ceil(eff_tiles * splits - 1e-9);
    const double fill = (eff_units < r.num_cus ? eff_units : (double)r.num_cus) / r.num_cus;
    t *= 1.0 + 0.1 * (1.0 - fill);
    if (splits > 1)
        t += kReduceFixedNs + (partial_bytes + d_bytes) / kReduceBytesPerNs;
    return t;
}

void fill_launch(int i, const Request& r, int splits, Plan* out) {
    const InstanceShape& s = kInstances[i];
    const int64_t m_blocks = (r.m + s.block_m - 1) / s.block_m;
    const int64_t tiles = tile_count(r, s);
    const int64_t slots = (int64_t)r.num_cus * s.wg_per_cu;
    const int64_t units = tiles * splits * passes_per_tile(r.layout, s.block_m);
    // kStaged: persistent grid; kStreamB: one workgroup per unit
    int64_t grid = (s.kind == kStreamB || units < slots) ? units : slots;
    if (grid < 1) grid = 1;
    out->instance = i;
    out->shape = s;
    if (r.layout == kKGrouped) out->shape.lds_bytes = s.stages * kgrouped_stage_bytes(s.block_m, s.block_n);
    out->tiles = tiles;
    out->grid = grid;
    const int64_t raster = m_blocks < 8 ? m_blocks : 8;
    out->raster = raster < 1 ? 1 : (int)raster;
    out->splits = splits;
    out->workspace_bytes = split_workspace_bytes(s, tiles, splits);
}

}  // namespace

int plan_instance(int instance, int splits, int layout, int64_t m, int n, int k, int num_groups,
                  int expected_m, int num_cus, int64_t workspace_bytes, Plan* out,
                  int scale_mode, int form) {
    if (instance < 0 || instance >= kNumInstances || num_cus < 1) return FP8BS_ERR_UNSUPPORTED;
    const Request r = make_request(layout, m, n, k, num_groups, expected_m, num_cus,
                                   workspace_bytes, form, scale_mode);
    const InstanceShape& s = kInstances[instance];
    if (!instance_fits(r, s)) return FP8BS_ERR_UNSUPPORTED;
    if (scale_mode == kScaleUE8M0 && !s.ue8m0) return FP8BS_ERR_UNSUPPORTED;
    int best_s = -1;
    if (splits >= 1) {
        if (estimate(r, s, splits) < 0) return FP8BS_ERR_UNSUPPORTED;
        best_s = splits;
    } else {
        double best_t = 0;
        for (int sp = 1; sp <= kMaxSplits; ++sp) {
            const double t = estimate(r, s, sp);
            if (t >= 0 && (best_s < 0 || t < best_t * (1.0 - 1e-9))) {
                best_s = sp;
                best_t = t;
            }
        }
        if (best_s < 0) return FP8BS_ERR_UNSUPPORTED;
    }
    fill_launch(instance, r, best_s, out);
    return FP8BS_OK;
}

int plan_request(int layout, int64_t m, int n, int k, int num_groups, int expected_m,
                 int num_cus, int64_t workspace_bytes, Plan* out, int scale_mode, int form,
                 int splits) {
    int st = validate_sizes(layout, m, n, k, layout == kDense ? 1 : num_groups, form);
    if (st != FP8BS_OK) return st;
    if (num_cus < 1) return FP8BS_ERR_UNSUPPORTED;
    const Request r = make_request(layout, m, n, k, num_groups, expected_m, num_cus,
                                   workspace_bytes, form, scale_mode);
    double best_t = 0;
    int best = -1, best_s = 1;
    for (int i = 0; i < kNumInstances; ++i) {
        const InstanceShape& s = kInstances[i];
        if (!instance_fits(r, s)) continue;
        if (scale_mode == kScaleUE8M0 && !s.ue8m0) continue;
        for (int sp = splits > 0 ? splits : 1; sp <= (splits > 0 ? splits : kMaxSplits); ++sp) {
            const double t = estimate(r, s, sp);
            if (t < 0) continue;
            if (best < 0 || t < best_t * (1.0 - 1e-9)) {
                best = i;
                best_s = sp;
                best_t = t;
            }
        }
    }
    if (best < 0) return FP8BS_ERR_UNSUPPORTED;
    fill_launch(best, r, best_s, out);
    return FP8BS_OK;
}

void export_plan(const Plan& p, fp8bs_plan* out) {
    *out = fp8bs_plan{};
    out->block_m = p.shape.block_m;
    out->block_n = p.shape.block_n;
    out->waves_m = p.shape.waves_m;
    out->waves_n = p.shape.waves_n;
    out->threads = 64 * p.shape.waves_m * p.shape.waves_n;
    out->lds_bytes = p.shape.lds_bytes;
    out->wg_per_cu = p.shape.wg_per_cu;
    out->stages = p.shape.stages;
    out->tiles = p.tiles;
    out->grid = p.grid;
    out->raster = p.raster;
    out->instance = p.instance;
    out->splits = p.splits;
    out->workspace_bytes = p.workspace_bytes;
    out->kind = p.shape.kind;
    out->ue8m0 = p.shape.ue8m0;
    out->mn = p.shape.mn != 0;
}

}  // namespace fp8bs

extern "C" int fp8bs_plan_query(int layout_code, int64_t m, int n, int k, int num_groups,
                                int expected_m, int num_cus, int64_t workspace_bytes,
                                fp8bs_plan* out) {
    if (!out) return FP8BS_ERR_POINTER;
    int layout, form, scale_mode;
    if (!fp8bs::decode_layout(layout_code, &layout, &form, &scale_mode))
        return FP8BS_ERR_UNSUPPORTED;
    fp8bs::Plan p;
    int st = fp8bs::plan_request(layout, m, n, k, layout == fp8bs::kDense ? 1 : num_groups,
                                 expected_m, num_cus, workspace_bytes, &p, scale_mode, form);
    if (st != FP8BS_OK) return st;
    fp8bs::export_plan(p, out);
    return FP8BS_OK;
}

extern "C" int64_t fp8bs_count_tiles(int layout_code, int64_t m, int n, int num_groups,
                                     int block_m, int block_n) {
    int layout, form;
    if (!fp8bs::decode_layout(layout_code, &layout, &form, nullptr)) return -1;
    if (m < 0 || n < 1 || block_m < 1 || block_n < 1) return -1;
    const bool per_group = layout == fp8bs::kMasked || layout == fp8bs::kKGrouped;
    if (per_group && num_groups < 1) return -1;
    const int64_t mb = (m + block_m - 1) / block_m;
    const int64_t nb = ((int64_t)n + block_n - 1) / block_n;
    return (per_group ? num_groups : 1) * mb * nb;
}

extern "C" int fp8bs_num_instances(void) { return fp8bs::kNumInstances; }

extern "C" int fp8bs_instance_info(int i, fp8bs_plan* out) {
    if (!out) return FP8BS_ERR_POINTER;
    if (i < 0 || i >= fp8bs::kNumInstances) return FP8BS_ERR_UNSUPPORTED;
    fp8bs::Plan p = {};
    p.instance = i;
    p.shape = fp8bs::kInstances[i];
    p.splits = 1;
    fp8bs::export_plan(p, out);
    return FP8BS_OK;
}

extern "C" const char* fp8bs_status_string(int status) {
    switch (status) {
        case FP8BS_OK: return "ok";
        case FP8BS_ERR_SHAPE: return "invalid shape (K must be a positive multiple of 128, "
                                     "m_total a multiple of 128, sizes positive; MN-major "
                                     "operands: M / N multiples of 16; K-grouped: group sizes "
                                     "multiples of 128 adding up to K_total, at most 256 groups)";
        case FP8BS_ERR_POINTER: return "NULL or misaligned (not 16-byte) pointer";
        case FP8BS_ERR_UNSUPPORTED: return "no compiled kernel instance covers the request "
                                           "(or a pinned instance / split count does not fit it)";
        case FP8BS_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

extern "C" int fp8bs_get_mk_alignment(void) { return 128; }

extern "C" int64_t fp8bs_get_sfa_ld(int64_t rows) {
    if (rows < 0) return -1;
    return (rows + 3) / 4 * 4;
}
