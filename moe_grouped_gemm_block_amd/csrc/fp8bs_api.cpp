// fp8bs_api.cpp -- the C ABI of libfp8bs (declared in include/fp8bs.h):
// argument checks, the planner call and the kernel launch on the caller's
// stream.  No allocation, no synchronisation, no host reads of device data.
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <cstdint>
#include <mutex>

#include "fp8bs_internal.h"

// The no-allocation entry point's split-K workspace: a library-owned device array, one
// copy per GPU (each device that loads the library holds it until the process ends).  Host
// code never uses the array's name as an address: its device address is looked up once per
// device with hipGetSymbolAddress and kept in g_scratch_ptr.
static __device__ __attribute__((aligned(256))) uint8_t scratch[FP8BS_NOALLOC_SCRATCH_BYTES];

namespace {

std::atomic<int> g_cu_cap{0};
// Test pins: per thread, so that one thread's pin never changes another thread's calls.
thread_local int t_forced_instance = -1;
thread_local int t_forced_splits = 0;
constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_cus[kMaxDevices];   // 0 = not queried yet

bool print_configs() {
    static const int on = [] {
        const char* e = getenv("FP8BS_PRINT_CONFIGS");
        return (e && e[0] && e[0] != '0') ? 1 : 0;
    }();
    return on != 0;
}

std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of the current device's scratch array; nullptr on error.
void* scratch_ptr() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::call_once(g_scratch_once[dev], [dev] {
        void* p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
    });
    return g_scratch_ptr[dev];
}

// Compute units of the current device, capped by fp8bs_set_num_cus; 0 on error.
int current_num_cus() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    int cus = (dev >= 0 && dev < kMaxDevices) ? g_dev_cus[dev].load(std::memory_order_relaxed) : 0;
    if (cus == 0) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        if (dev >= 0 && dev < kMaxDevices) g_dev_cus[dev].store(cus, std::memory_order_relaxed);
    }
    const int cap = g_cu_cap.load(std::memory_order_relaxed);
    return (cap > 0 && cap < cus) ? cap : cus;
}

bool aligned16(const void* p) { return p && ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return p && ((uintptr_t)p & 3u) == 0; }

// Names of the public layout codes (FP8BS_LAYOUT_*).
int layout_code(int layout, int form) {
    if (layout == fp8bs::kKGrouped) return 3;
    if (layout == fp8bs::kDense && form != fp8bs::kFormNT) return 3 + form;
    return layout;
}

void format_plan(const fp8bs::Plan& pl, int layout, int form, int64_t m, int n, int k, int g,
                 int expected_m, int cus, char* buf, size_t len,
                 int scale_mode = fp8bs::kScaleF32) {
    static const char* names[7] = {"dense", "contiguous", "masked", "k-grouped tn",
                                   "dense nn", "dense tn", "dense tt"};
    snprintf(buf, len,
             "fp8bs %s%s m=%lld n=%d k=%d groups=%d expected_m=%d cus=%d -> %s block %dx%d "
             "waves %dx%d threads %d stages %d lds %dB wg/cu %d tiles %lld splits %d "
             "workspace %lldB grid %lld raster %d instance %d",
             names[layout_code(layout, form)], scale_mode == fp8bs::kScaleUE8M0 ? " ue8m0" : "",
             (long long)m, n, k, g, expected_m, cus,
             pl.shape.kind == fp8bs::kStreamB ? "stream-B" : "staged", pl.shape.block_m,
             pl.shape.block_n, pl.shape.waves_m, pl.shape.waves_n,
             64 * pl.shape.waves_m * pl.shape.waves_n, pl.shape.stages, pl.shape.lds_bytes,
             pl.shape.wg_per_cu, (long long)pl.tiles, pl.splits, (long long)pl.workspace_bytes,
             (long long)pl.grid, pl.raster, pl.instance);
}

// The last few plans of this thread, keyed by every input of the planner (the plan is a
// pure function of them), so that a repeated call skips the cost model.
struct PlanKey {
    int64_t m, ws_bytes;
    int layout, n, k, num_groups, expected_m, scale_mode, form, cus, forced, splits;
    bool operator==(const PlanKey& o) const {
        return m == o.m && ws_bytes == o.ws_bytes && layout == o.layout && n == o.n &&
               k == o.k && num_groups == o.num_groups && expected_m == o.expected_m &&
               scale_mode == o.scale_mode && form == o.form && cus == o.cus &&
               forced == o.forced && splits == o.splits;
    }
};
struct PlanCacheEntry {
    bool valid;
    PlanKey key;
    fp8bs::Plan plan;
};
constexpr int kPlanCacheEntries = 8;
thread_local PlanCacheEntry t_plans[kPlanCacheEntries];
thread_local int t_plan_next = 0;

// Plan for a request on the current device, honouring the test pins.
int make_plan(int layout, int64_t m, int n, int k, int num_groups, int expected_m,
              int64_t ws_bytes, int* cus_out, fp8bs::Plan* pl, int scale_mode = fp8bs::kScaleF32,
              int form = fp8bs::kFormNT) {
    const int cus = current_num_cus();
    if (cus <= 0) return FP8BS_ERR_HIP;
    *cus_out = cus;
    const int forced = t_forced_instance;
    const int splits = ws_bytes > 0 ? t_forced_splits : 1;
    const PlanKey key{m, ws_bytes, layout, n, k, num_groups, expected_m, scale_mode, form, cus,
                      forced, splits};
    for (const PlanCacheEntry& e : t_plans) {
        if (e.valid && e.key == key) {
            *pl = e.plan;
            return FP8BS_OK;
        }
    }
    // a pinned split count alone: the best instance that runs with it (so that the plan a
    // workspace was sized for is found again when that workspace is lent)
    int st = fp8bs::plan_request(layout, m, n, k, num_groups, expected_m, cus, ws_bytes, pl,
                                 scale_mode, form, forced >= 0 ? 0 : splits);
    if (st != FP8BS_OK) return st;
    if (forced >= 0 || splits > 0)
        st = fp8bs::plan_instance(forced >= 0 ? forced : pl->instance, splits, layout, m, n, k,
                                  num_groups, expected_m, cus, ws_bytes, pl, scale_mode, form);
    if (st == FP8BS_OK) {
        PlanCacheEntry& e = t_plans[t_plan_next];
        t_plan_next = (t_plan_next + 1) % kPlanCacheEntries;
        e.valid = true;
        e.key = key;
        e.plan = *pl;
    }
    return st;
}

// group_data: contiguous grouped_layout / masked masked_m (device); K-grouped: the host
// array of group sizes along K.
int run(int layout, const void* a, const float* sfa, const void* b, const float* sfb, void* d,
        const int32_t* group_data, int64_t m, int n, int k, int num_groups, int expected_m,
        void* ws, size_t ws_bytes, hipStream_t stream, int scale_mode = fp8bs::kScaleF32,
        const float* c = nullptr, bool want_c = false, int form = fp8bs::kFormNT) {
    int st = fp8bs::validate_sizes(layout, m, n, k, num_groups, form);
    if (st != FP8BS_OK) return st;
    const bool kg = layout == fp8bs::kKGrouped;
    if (kg) {                                    // host-side group sizes
        if (!group_data) return FP8BS_ERR_POINTER;
        int64_t total = 0;
        for (int g = 0; g < num_groups; ++g) {
            if (group_data[g] < 0 || group_data[g] % 128 != 0) return FP8BS_ERR_SHAPE;
            total += group_data[g];
        }
        if (total != k) return FP8BS_ERR_SHAPE;
    }
    // No output rows: nothing is launched and no pointer is dereferenced, so none is
    // checked (an empty torch tensor, say a batch routed to no expert, has a NULL pointer).
    if (m == 0) return FP8BS_OK;
    // (a K-grouped call with k_total == 0 reads no operand: those pointers may be NULL)
    const bool operands_read = !(kg && k == 0);
    if (operands_read &&
        (!aligned16(a) || !aligned16(sfa) || !aligned16(b) || !aligned16(sfb)))
        return FP8BS_ERR_POINTER;
    if (!aligned16(d)) return FP8BS_ERR_POINTER;
    if (layout != fp8bs::kDense && !kg && !aligned4(group_data)) return FP8BS_ERR_POINTER;
    if (ws_bytes > 0 && !aligned16(ws)) return FP8BS_ERR_POINTER;
    if (want_c && !aligned16(c)) return FP8BS_ERR_POINTER;
    const int64_t ws_cap = ws_bytes > (size_t)INT64_MAX ? INT64_MAX : (int64_t)ws_bytes;
    int cus = 0;
    fp8bs::Plan pl;
    st = make_plan(layout, m, n, k, num_groups, expected_m, ws_cap, &cus, &pl, scale_mode, form);
    if (st != FP8BS_OK) return st;
    if (print_configs()) {
        char line[512];
        format_plan(pl, layout, form, m, n, k, num_groups, expected_m, cus, line, sizeof line,
                    scale_mode);
        fprintf(stderr, "%s\n", line);
    }
    fp8bs::GemmParams p;
    p.a = (const uint8_t*)a;
    p.sfa = sfa;
    p.b = (const uint8_t*)b;
    p.sfb = sfb;
    p.d = (uint16_t*)d;
    p.grouped_layout = layout == fp8bs::kContiguous ? group_data : nullptr;
    p.masked_m = layout == fp8bs::kMasked ? group_data : nullptr;
    p.m = (int)m;
    p.n = n;
    p.k = k;
    p.num_groups = num_groups;
    p.sfa_ld = (int)fp8bs_get_sfa_ld(m);
    p.m_blocks = (int)((m + pl.shape.block_m - 1) / pl.shape.block_m);
    p.n_blocks = (n + pl.shape.block_n - 1) / pl.shape.block_n;
    p.tiles = (int)pl.tiles;
    p.raster = pl.raster;
    p.splits = pl.splits;
    p.units = (int)(pl.tiles * pl.splits * fp8bs::passes_per_tile(layout, pl.shape.block_m));
    p.ws = pl.splits > 1 ? (float*)ws : nullptr;
    p.c = want_c ? c : nullptr;
    p.sfb_ld = (int)fp8bs_get_sfa_ld(n);
    p.kg_chunk0[0] = 0;
    if (kg) {
        p.grouped_layout = nullptr;
        for (int g = 0; g < num_groups; ++g) p.kg_chunk0[g + 1] = p.kg_chunk0[g] + group_data[g] / 128;
    }
    const int err = fp8bs::launch_instance(pl, layout, scale_mode, p, stream, form);
    return err == (int)hipSuccess ? FP8BS_OK : FP8BS_ERR_HIP;
}

}  // namespace

extern "C" {

int fp8bs_dense_nt(const void* a, const float* sfa, const void* b, const float* sfb, void* d,
                   int m, int n, int k, hipStream_t stream) {
    return run(fp8bs::kDense, a, sfa, b, sfb, d, nullptr, m, n, k, 1, 0, nullptr, 0, stream);
}

int fp8bs_grouped_contiguous_nt(const void* a, const float* sfa, const void* b, const float* sfb,
                                void* d, const int32_t* grouped_layout, int m_total, int n, int k,
                                int num_groups, hipStream_t stream) {
    return run(fp8bs::kContiguous, a, sfa, b, sfb, d, grouped_layout, m_total, n, k, num_groups,
               0, nullptr, 0, stream);
}

int fp8bs_grouped_masked_nt(const void* a, const float* sfa, const void* b, const float* sfb,
                            void* d, const int32_t* masked_m, int num_groups, int max_m,
                            int expected_m, int n, int k, hipStream_t stream) {
    if (num_groups < 1) return FP8BS_ERR_SHAPE;
    return run(fp8bs::kMasked, a, sfa, b, sfb, d, masked_m, max_m, n, k, num_groups, expected_m,
               nullptr, 0, stream);
}

int fp8bs_dense_nt_ws(const void* a, const float* sfa, const void* b, const float* sfb, void* d,
                      int m, int n, int k, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
    return run(fp8bs::kDense, a, sfa, b, sfb, d, nullptr, m, n, k, 1, 0, workspace,
               workspace_bytes, stream);
}

int fp8bs_grouped_contiguous_nt_ws(const void* a, const float* sfa, const void* b,
                                   const float* sfb, void* d, const int32_t* grouped_layout,
                                   int m_total, int n, int k, int num_groups, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
    return run(fp8bs::kContiguous, a, sfa, b, sfb, d, grouped_layout, m_total, n, k, num_groups,
               0, workspace, workspace_bytes, stream);
}

int fp8bs_grouped_masked_nt_ws(const void* a, const float* sfa, const void* b, const float* sfb,
                               void* d, const int32_t* masked_m, int num_groups, int max_m,
                               int expected_m, int n, int k, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
    if (num_groups < 1) return FP8BS_ERR_SHAPE;
    return run(fp8bs::kMasked, a, sfa, b, sfb, d, masked_m, max_m, n, k, num_groups, expected_m,
               workspace, workspace_bytes, stream);
}

int fp8bs_dense_nt_c(const void* a, const float* sfa, const void* b, const float* sfb,
                     const float* c, void* d, int m, int n, int k, void* workspace,
                     size_t workspace_bytes, hipStream_t stream) {
    return run(fp8bs::kDense, a, sfa, b, sfb, d, nullptr, m, n, k, 1, 0, workspace,
               workspace_bytes, stream, fp8bs::kScaleF32, c, true);
}

int fp8bs_grouped_contiguous_nt_c(const void* a, const float* sfa, const void* b,
                                  const float* sfb, const float* c, void* d,
                                  const int32_t* grouped_layout, int m_total, int n, int k,
                                  int num_groups, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
    return run(fp8bs::kContiguous, a, sfa, b, sfb, d, grouped_layout, m_total, n, k, num_groups,
               0, workspace, workspace_bytes, stream, fp8bs::kScaleF32, c, true);
}

int fp8bs_grouped_masked_nt_c(const void* a, const float* sfa, const void* b, const float* sfb,
                              const float* c, void* d, const int32_t* masked_m, int num_groups,
                              int max_m, int expected_m, int n, int k, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
    if (num_groups < 1) return FP8BS_ERR_SHAPE;
    return run(fp8bs::kMasked, a, sfa, b, sfb, d, masked_m, max_m, n, k, num_groups, expected_m,
               workspace, workspace_bytes, stream, fp8bs::kScaleF32, c, true);
}

int fp8bs_dense_nt_ue8m0(const void* a, const int32_t* sfa, const void* b, const int32_t* sfb,
                         void* d, int m, int n, int k, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
    return run(fp8bs::kDense, a, (const float*)sfa, b, (const float*)sfb, d, nullptr, m, n, k, 1, 0,
               workspace, workspace_bytes, stream, fp8bs::kScaleUE8M0);
}

int fp8bs_grouped_contiguous_nt_ue8m0(const void* a, const int32_t* sfa, const void* b,
                                      const int32_t* sfb, void* d, const int32_t* grouped_layout,
                                      int m_total, int n, int k, int num_groups, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
    return run(fp8bs::kContiguous, a, (const float*)sfa, b, (const float*)sfb, d, grouped_layout,
               m_total, n, k, num_groups, 0, workspace, workspace_bytes, stream,
               fp8bs::kScaleUE8M0);
}

int fp8bs_grouped_masked_nt_ue8m0(const void* a, const int32_t* sfa, const void* b,
                                  const int32_t* sfb, void* d, const int32_t* masked_m,
                                  int num_groups, int max_m, int expected_m, int n, int k,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (num_groups < 1) return FP8BS_ERR_SHAPE;
    return run(fp8bs::kMasked, a, (const float*)sfa, b, (const float*)sfb, d, masked_m, max_m, n,
               k, num_groups, expected_m, workspace, workspace_bytes, stream, fp8bs::kScaleUE8M0);
}

int fp8bs_dense_nn(const void* a, const float* sfa, const void* b, const float* sfb,
                   const float* c, void* d, int m, int n, int k, void* workspace,
                   size_t workspace_bytes, hipStream_t stream) {
    return run(fp8bs::kDense, a, sfa, b, sfb, d, nullptr, m, n, k, 1, 0, workspace,
               workspace ? workspace_bytes : 0, stream, fp8bs::kScaleF32, c, c != nullptr,
               fp8bs::kFormNN);
}

int fp8bs_dense_tn(const void* a, const float* sfa, const void* b, const float* sfb,
                   const float* c, void* d, int m, int n, int k, void* workspace,
                   size_t workspace_bytes, hipStream_t stream) {
    return run(fp8bs::kDense, a, sfa, b, sfb, d, nullptr, m, n, k, 1, 0, workspace,
               workspace ? workspace_bytes : 0, stream, fp8bs::kScaleF32, c, c != nullptr,
               fp8bs::kFormTN);
}

int fp8bs_dense_tt(const void* a, const float* sfa, const void* b, const float* sfb,
                   const float* c, void* d, int m, int n, int k, void* workspace,
                   size_t workspace_bytes, hipStream_t stream) {
    return run(fp8bs::kDense, a, sfa, b, sfb, d, nullptr, m, n, k, 1, 0, workspace,
               workspace ? workspace_bytes : 0, stream, fp8bs::kScaleF32, c, c != nullptr,
               fp8bs::kFormTT);
}

int fp8bs_k_grouped_tn_contiguous(const void* a, const float* sfa, const void* b,
                                  const float* sfb, const float* c, float* d, const int32_t* ks,
                                  int num_groups, int m, int n, int k_total, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
    return run(fp8bs::kKGrouped, a, sfa, b, sfb, d, ks, m, n, k_total, num_groups, 0, workspace,
               workspace ? workspace_bytes : 0, stream, fp8bs::kScaleF32, c, c != nullptr);
}

int fp8bs_dense_nn_ue8m0(const void* a, const int32_t* sfa, const void* b, const int32_t* sfb,
                         const float* c, void* d, int m, int n, int k, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
    return run(fp8bs::kDense, a, (const float*)sfa, b, (const float*)sfb, d, nullptr, m, n, k, 1, 0,
               workspace, workspace ? workspace_bytes : 0, stream, fp8bs::kScaleUE8M0, c,
               c != nullptr, fp8bs::kFormNN);
}

int fp8bs_dense_tn_ue8m0(const void* a, const int32_t* sfa, const void* b, const int32_t* sfb,
                         const float* c, void* d, int m, int n, int k, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
    return run(fp8bs::kDense, a, (const float*)sfa, b, (const float*)sfb, d, nullptr, m, n, k, 1, 0,
               workspace, workspace ? workspace_bytes : 0, stream, fp8bs::kScaleUE8M0, c,
               c != nullptr, fp8bs::kFormTN);
}

int fp8bs_dense_tt_ue8m0(const void* a, const int32_t* sfa, const void* b, const int32_t* sfb,
                         const float* c, void* d, int m, int n, int k, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
    return run(fp8bs::kDense, a, (const float*)sfa, b, (const float*)sfb, d, nullptr, m, n, k, 1, 0,
               workspace, workspace ? workspace_bytes : 0, stream, fp8bs::kScaleUE8M0, c,
               c != nullptr, fp8bs::kFormTT);
}

int fp8bs_k_grouped_tn_contiguous_ue8m0(const void* a, const int32_t* sfa, const void* b,
                                        const int32_t* sfb, const float* c, float* d,
                                        const int32_t* ks, int num_groups, int m, int n,
                                        int k_total, void* workspace, size_t workspace_bytes,
                                        hipStream_t stream) {
    return run(fp8bs::kKGrouped, a, (const float*)sfa, b, (const float*)sfb, d, ks, m, n, k_total,
               num_groups, 0, workspace, workspace ? workspace_bytes : 0, stream,
               fp8bs::kScaleUE8M0, c, c != nullptr);
}

int fp8bs_dense_nt_noalloc(const void* a, const float* sfa, const void* b, const float* sfb,
                           void* d, int m, int n, int k, hipStream_t stream) {
    // sizes first: an invalid or empty request is answered without touching the device
    const int st = fp8bs::validate_sizes(fp8bs::kDense, m, n, k, 1);
    if (st != FP8BS_OK || m == 0) return st;
    void* ws = scratch_ptr();
    if (!ws) return FP8BS_ERR_HIP;
    // The planner only picks plans whose partial tiles fit the array; a pinned split count
    // that needs more is refused (FP8BS_ERR_UNSUPPORTED) before anything is launched.
    return run(fp8bs::kDense, a, sfa, b, sfb, d, nullptr, m, n, k, 1, 0, ws,
               FP8BS_NOALLOC_SCRATCH_BYTES, stream);
}

size_t fp8bs_noalloc_scratch_bytes(void) { return FP8BS_NOALLOC_SCRATCH_BYTES; }

int64_t fp8bs_workspace_size(int layout_code, int64_t m, int n, int k, int num_groups,
                             int expected_m) {
    int layout, form, scale_mode;
    if (!fp8bs::decode_layout(layout_code, &layout, &form, &scale_mode))
        return -FP8BS_ERR_UNSUPPORTED;
    const int g = layout == fp8bs::kDense ? 1 : num_groups;
    int st = fp8bs::validate_sizes(layout, m, n, k, g, form);
    if (st != FP8BS_OK) return -st;
    if (m == 0) return 0;
    int cus = 0;
    fp8bs::Plan pl;
    // the planner's choice with unlimited workspace, then any pins
    st = make_plan(layout, m, n, k, g, expected_m, INT64_MAX, &cus, &pl, scale_mode, form);
    if (st != FP8BS_OK) return -st;
    return pl.workspace_bytes;
}

int fp8bs_set_num_cus(int n) {
    if (n < 0) return -1;
    return g_cu_cap.exchange(n);
}

int fp8bs_get_num_cus(void) { return g_cu_cap.load(); }

int fp8bs_force_instance(int i) {
    if (i < -1 || i >= fp8bs::kNumInstances) return -2;
    const int prev = t_forced_instance;
    t_forced_instance = i;
    return prev;
}

int fp8bs_force_splits(int s) {
    if (s < 0) return -1;
    const int prev = t_forced_splits;
    t_forced_splits = s;
    return prev;
}

int fp8bs_describe_config(int layout_code, int64_t m, int n, int k, int num_groups,
                          int expected_m, char* buf, size_t len) {
    if (!buf || len == 0) return FP8BS_ERR_POINTER;
    int layout, form, scale_mode;
    if (!fp8bs::decode_layout(layout_code, &layout, &form, &scale_mode))
        return FP8BS_ERR_UNSUPPORTED;
    const int g = layout == fp8bs::kDense ? 1 : num_groups;
    int cus = 0;
    fp8bs::Plan pl;
    const int st = make_plan(layout, m, n, k, g, expected_m, INT64_MAX, &cus, &pl, scale_mode,
                             form);
    if (st != FP8BS_OK) {
        snprintf(buf, len, "%s", fp8bs_status_string(st));
        return st;
    }
    format_plan(pl, layout, form, m, n, k, g, expected_m, cus, buf, len, scale_mode);
    return FP8BS_OK;
}

}  // extern "C"
