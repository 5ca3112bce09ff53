// fp8bs_internal.h -- types shared by the host planner, the C ABI and the
// kernel instances of libfp8bs.  Not part of the public interface.
#pragma once
#include <stdint.h>

#include "fp8bs.h"

namespace fp8bs {

// kKGrouped: groups run along K (MoE weight gradients): A [K_total][M], B [K_total][N],
// per-group K ranges, FP32 output D [G][M][N].
enum Layout : int { kDense = 0, kContiguous = 1, kMasked = 2, kKGrouped = 3 };

// Stored forms of the dense operands: whether A is [M][K] ("n") or [K][M] ("t") and B is
// [N][K] ("t") or [K][N] ("n").  kFormNT is the K-major form every layout supports.
enum Form : int { kFormNT = 0, kFormNN = 1, kFormTN = 2, kFormTT = 3 };
constexpr bool form_a_mn(int form) { return form == kFormTN || form == kFormTT; }
constexpr bool form_b_mn(int form) { return form == kFormNN || form == kFormTN; }

// Most groups a K-grouped launch takes (their K offsets travel in the kernel arguments).
constexpr int kMaxKGroups = 256;

// Kernel families.
//   kStaged: A and B tiles both staged in LDS (direct-to-LDS copies), persistent grid;
//            for shapes with enough rows that B tiles are shared by several wavefronts.
//   kStreamB: B fragments loaded from global memory straight into registers (no LDS),
//            A and the scales staged in LDS; one work unit per workgroup; for few-row
//            (decode) shapes, where every B byte is used by one wavefront only and HBM
//            bandwidth bounds the GEMM.
enum Kind : int { kStaged = 0, kStreamB = 1 };

// Scale formats: FP32 factors (promotion on the VALU), or power-of-two factors given as
// E8M0 exponents packed four K groups per 32-bit word (applied by the matrix core).
enum ScaleMode : int { kScaleF32 = 0, kScaleUE8M0 = 1 };

// Shape of one compiled kernel instance: an output tile of block_m x block_n
// computed by waves_m x waves_n wavefronts (64 lanes each), each owning a
// (block_m / waves_m) x (block_n / waves_n) sub-tile made of 16x16 MFMA tiles,
// with a ring of `stages` LDS stages (one 128-K chunk each) in flight.
struct InstanceShape {
    int kind;
    int block_m, block_n, waves_m, waves_n;
    int stages;
    int wg_per_cu;       // workgroups per CU the launch assumes (LDS / register bound)
    int lds_bytes;
    int chunk_ns;        // cost model: CU time per 128-K chunk of one tile
    int tile_ns;         // cost model: CU time per tile (prologue / epilogue)
    int stream_chunk_ns; // the same two when the operands stream from HBM (few rows)
    int stream_tile_ns;
    int ue8m0;           // 1: also compiled for packed UE8M0 scales
    int mn;              // > 0: also compiled for MN-major operands (nn / tn / tt, K-grouped);
                         // the K-grouped layout's cost in percent of the model
    int mn_e8;           // the same cost for the K-grouped layout with UE8M0 scales
};

// LDS bytes of one pipeline stage: the A tile, the B tile (128 K bytes per
// row), the tile's block_m A scales and up to 64 B-scale values.
constexpr int stage_bytes(int block_m, int block_n) {
    return (block_m + block_n) * 128 + block_m * 4 + 256;
}
// The K-grouped layout scales B per column: block_n B-scale values per stage.
constexpr int kgrouped_stage_bytes(int block_m, int block_n) {
    return (block_m + block_n) * 128 + block_m * 4 + (block_n * 4 > 256 ? block_n * 4 : 256);
}
// kStreamB: one stage holds the A tile, its A scales (at least 256 bytes: one per lane of
// a copy instruction) and 256 bytes of B scales.
constexpr int stream_sa_bytes(int block_m) { return block_m * 4 > 256 ? block_m * 4 : 256; }
constexpr int stream_stage_bytes(int block_m) { return block_m * 128 + stream_sa_bytes(block_m) + 256; }
constexpr int instance_lds_bytes(int kind, int block_m, int block_n, int stages) {
    return stages * (kind == kStreamB ? stream_stage_bytes(block_m) : stage_bytes(block_m, block_n));
}
constexpr int kLdsBytesPerCu = 160 * 1024;

// The instance table (defined next to the kernels, read by the planner).
extern const InstanceShape kInstances[];
extern const int kNumInstances;

// Everything a kernel needs; plain values and device pointers.
struct GemmParams {
    const uint8_t* a;
    const float* sfa;
    const uint8_t* b;
    const float* sfb;
    uint16_t* d;
    const int32_t* grouped_layout;   // contiguous only
    const int32_t* masked_m;         // masked only
    int m;              // dense: M; contiguous: m_total; masked: max_m (rows per slot)
    int n, k;
    int num_groups;
    int sfa_ld;         // leading dimension of the MN-major SFA (per slot for masked)
    int m_blocks;       // ceil(m / block_m)
    int n_blocks;       // ceil(n / block_n)
    int tiles;          // (num_groups for masked) x m_blocks x n_blocks
    int raster;         // m-blocks per raster group
    int splits;         // K splits per tile (1: no workspace use)
    int units;          // tiles x splits
    float* ws;          // splits > 1: FP32 partial tiles, [tile][split][block_m*block_n]
    const float* c;     // optional FP32 addend with D's shape (nullptr: none)
    // K-grouped only: leading dimension of the MN-major SFB, and the first 128-K chunk of
    // each group (kg_chunk0[g] .. kg_chunk0[g+1]-1 are group g's chunks)
    int sfb_ld;
    int kg_chunk0[kMaxKGroups + 1];
};

struct Plan {
    int instance;
    InstanceShape shape;
    int64_t tiles;
    int64_t grid;
    int raster;
    int splits;
    int64_t workspace_bytes;    // bytes of workspace the launch uses (0 when splits == 1)
};

// Work units per tile and split: the contiguous layout with tiles taller than one
// 128-row expert block runs each tile in two passes (one per expert it may hold).
constexpr int passes_per_tile(int layout, int block_m) {
    return layout == kContiguous && block_m > 128 ? 2 : 1;
}

// Workspace bytes a launch of `shape` with `splits` K splits needs.
int64_t split_workspace_bytes(const InstanceShape& shape, int64_t tiles, int splits);

// Host planner: deterministic choice of an instance, a K split count (only when the
// caller offers at least that much workspace) and launch shape; splits > 0 restricts the
// choice to instances that run with that split count.
// Returns FP8BS_OK or an error status.  No device access.
int plan_request(int layout, int64_t m, int n, int k, int num_groups, int expected_m,
                 int num_cus, int64_t workspace_bytes, Plan* out, int scale_mode = kScaleF32,
                 int form = kFormNT, int splits = 0);

// Launch shape for a given instance and split count (used when either is pinned;
// splits < 1 picks the best split count for the instance within the workspace).
int plan_instance(int instance, int splits, int layout, int64_t m, int n, int k, int num_groups,
                  int expected_m, int num_cus, int64_t workspace_bytes, Plan* out,
                  int scale_mode = kScaleF32, int form = kFormNT);

// Copies a plan into the public struct.
void export_plan(const Plan& p, fp8bs_plan* out);

// Validates sizes for an entry point (FP8BS_OK or FP8BS_ERR_SHAPE).  K-grouped: k is
// K_total (0 allowed); MN-major operands need their M / N to be a multiple of 16.
int validate_sizes(int layout, int64_t m, int n, int k, int num_groups, int form = kFormNT);

// Public layout code (FP8BS_LAYOUT_*, optionally OR-ed with FP8BS_LAYOUT_UE8M0) -> internal
// layout, stored form and scale format (scale_mode may be null); false if unknown.
bool decode_layout(int code, int* layout, int* form, int* scale_mode);

// Launches instance `plan.instance` for `layout`, scale format and stored form; returns a
// hipError_t value.
int launch_instance(const Plan& plan, int layout, int scale_mode, const GemmParams& p,
                    hipStream_t stream, int form = kFormNT);

}  // namespace fp8bs
