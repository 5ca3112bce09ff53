// fp8bs_gemm.hip -- the block-scaled FP8 GEMM kernel for gfx950 (CDNA4).
//
// One kernel template serves the dense, contiguous-grouped and masked-grouped
// layouts (the DeepGEMM README repost, lqnn.cn/news/60274, "DeepGEMM" and
// "优化技术": one core kernel and one block scheduler for grouped and
// non-grouped GEMMs).  Per output tile and per 128-wide K chunk:
//
//   1. the A tile (block_m x 128 e4m3) and the B tile (block_n x 128 e4m3) are
//      staged in LDS (double buffered, 16-byte XOR swizzle per 128-byte row);
//   2. each wavefront computes its 16x16 sub-tiles with one
//      v_mfma_f32_16x16x128_f8f6f4 each (OCP e4m3 x e4m3, FP32 result) into a
//      partial that starts from zero every chunk;
//   3. the partial is promoted into the FP32 accumulator with
//      acc += partial * (sfa[row] * sfb[col block]) on the vector ALU
//      (two-level accumulation, section "DeepGEMM" of the same page);
//   4. after the last chunk the accumulator is rounded to BF16 (nearest even)
//      and stored, only at valid rows and columns.
//
// The tile scheduler is persistent: workgroup w processes tiles w, w + grid,
// ... in a rasterised order (groups of `raster` m-blocks sweep the n-blocks,
// so concurrently running tiles share B column stripes and A row stripes in
// L2), and workgroup ids are remapped so that each XCD (workgroups are handed
// to the 8 XCDs round-robin) runs a contiguous range of that order.
#include <hip/hip_runtime.h>

#include "fp8bs_internal.h"

namespace fp8bs {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// FP8 (OCP e4m3) x FP8 -> FP32 16x16x128 matrix product with a zero addend.
// Lane l supplies row (l % 16) of A and column (l % 16) of B, each as 32 bytes
// of K; the K position of each byte is the same function of (l / 16, byte) for
// both operands, so any fixed assignment of the chunk's 128 K values to those
// slots (the same for A and B) yields the full chunk dot product.  Result:
// lane l holds rows 4 * (l / 16) + v, v = 0..3, of column l % 16.
__device__ __forceinline__ f32x4 mfma_e4m3_16x16x128(const i32x8& a, const i32x8& b) {
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    // format codes 0/0 = e4m3 for both operands; no block scaling (scale 0, opsel 0)
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ uint16_t to_bf16_rne(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);   // v_cvt_pk_bf16_f32, nearest even
}

// Workgroup id -> position in the schedule: workgroup b runs on XCD b % 8, so
// XCD x is given the contiguous range [x * grid/8, (x+1) * grid/8).
__device__ __forceinline__ int logical_block_id() {
    const int n = gridDim.x, b = blockIdx.x;
    if ((n & 7) != 0) return b;
    return (b & 7) * (n >> 3) + (b >> 3);
}

// Schedule position -> (slot, m-block, n-block).  Masked: slot-major.  Within
// a slot, groups of `raster` m-blocks sweep all n-blocks column by column.
template <int LAYOUT>
__device__ __forceinline__ void map_tile(const GemmParams& p, int t, int& g, int& mb, int& nb) {
    int rest = t;
    g = 0;
    if (LAYOUT == kMasked) {
        const int per_slot = p.m_blocks * p.n_blocks;
        g = t / per_slot;
        rest = t - g * per_slot;
    }
    const int per_group = p.raster * p.n_blocks;
    const int grp = rest / per_group;
    const int r = rest - grp * per_group;
    const int first = grp * p.raster;
    const int rows_in = min(p.raster, p.m_blocks - first);
    mb = first + r % rows_in;
    nb = r / rows_in;
}

template <int BM, int BN, int WM, int WN, int LAYOUT>
__global__ void __launch_bounds__(64 * WM * WN) fp8bs_gemm_kernel(GemmParams p) {
    constexpr int NT = 64 * WM * WN;
    constexpr int WTM = BM / WM, WTN = BN / WN;      // wavefront sub-tile
    constexpr int TM = WTM / 16, TN = WTN / 16;      // 16x16 MFMA tiles per wavefront
    static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wavefront tile must be a multiple of 16");
    constexpr int A_BYTES = BM * 128, STAGE = (BM + BN) * 128;
    constexpr int A_UNITS = BM * 8, B_UNITS = BN * 8;                 // 16-byte units per chunk
    constexpr int A_PER = (A_UNITS + NT - 1) / NT, B_PER = (B_UNITS + NT - 1) / NT;

    __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int kchunks = p.k / 128;
    const int64_t K = p.k;
    const int nsb = (p.n + 127) / 128;               // B scale blocks along N

    for (int t = logical_block_id(); t < p.tiles; t += gridDim.x) {
        int g, mb, nb;
        map_tile<LAYOUT>(p, t, g, mb, nb);
        const int m0 = mb * BM, n0 = nb * BN;
        int row_limit = p.m;                         // rows of this slot that exist/are valid
        if (LAYOUT == kMasked) {
            const int v = min(max(p.masked_m[g], 0), p.m);
            if (m0 >= v) continue;                   // nothing valid in this tile
            row_limit = v;
        } else if (LAYOUT == kContiguous) {
            const int e = p.grouped_layout[m0];      // a block holds one expert, then padding
            if (e < 0 || e >= p.num_groups) continue;
            g = e;
        }

        const uint8_t* a_g = p.a + (LAYOUT == kMasked ? (int64_t)g * p.m * K : (int64_t)0);
        const uint8_t* b_g = p.b + (int64_t)g * p.n * K;
        const float* sfa_g = p.sfa + (LAYOUT == kMasked ? (int64_t)g * kchunks * p.sfa_ld : (int64_t)0);
        const float* sfb_g = p.sfb + (int64_t)g * nsb * kchunks;

        // ---- per-thread global->LDS copy assignment (16 bytes per unit) ----
        int64_t a_src[A_PER];
        int a_dst[A_PER];
        bool a_ok[A_PER];
#pragma unroll
        for (int i = 0; i < A_PER; ++i) {
            const int u = tid + i * NT;
            const int row = u >> 3, q = u & 7;
            a_ok[i] = (A_UNITS % NT == 0) || u < A_UNITS;
            const int grow = min(m0 + row, row_limit - 1);      // clamp: never read past the slot
            a_src[i] = (int64_t)grow * K + q * 16;
            a_dst[i] = row * 128 + ((q ^ (row & 7)) << 4);
        }
        int64_t b_src[B_PER];
        int b_dst[B_PER];
        bool b_ok[B_PER];
#pragma unroll
        for (int i = 0; i < B_PER; ++i) {
            const int u = tid + i * NT;
            const int row = u >> 3, q = u & 7;
            b_ok[i] = (B_UNITS % NT == 0) || u < B_UNITS;
            const int grow = min(n0 + row, p.n - 1);
            b_src[i] = (int64_t)grow * K + q * 16;
            b_dst[i] = A_BYTES + row * 128 + ((q ^ (row & 7)) << 4);
        }

        // ---- per-lane fragment addresses in a stage ----
        const int kg = lane >> 4;                     // which 32-byte quarter of the chunk
        int a_frag[TM][2], b_frag[TN][2];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int row = wm * WTM + i * 16 + (lane & 15);
#pragma unroll
            for (int h = 0; h < 2; ++h) a_frag[i][h] = row * 128 + (((2 * kg + h) ^ (row & 7)) << 4);
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int row = wn * WTN + j * 16 + (lane & 15);
#pragma unroll
            for (int h = 0; h < 2; ++h)
                b_frag[j][h] = A_BYTES + row * 128 + (((2 * kg + h) ^ (row & 7)) << 4);
        }
        // rows of the four accumulator values this lane holds in sub-tile i
        int sa_row[TM];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int r4 = m0 + wm * WTM + i * 16 + kg * 4;
            sa_row[i] = r4 < p.sfa_ld ? r4 : 0;       // groups of 4 rows lie wholly inside or outside
        }
        int sb_blk[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) sb_blk[j] = min(n0 + wn * WTN + j * 16, p.n - 1) / 128;

        f32x4 acc[TM][TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

        i32x4 ra[A_PER], rb[B_PER];
        // prologue: chunk 0 -> stage 0
#pragma unroll
        for (int i = 0; i < A_PER; ++i)
            if (a_ok[i]) ra[i] = *(const i32x4*)(a_g + a_src[i]);
#pragma unroll
        for (int i = 0; i < B_PER; ++i)
            if (b_ok[i]) rb[i] = *(const i32x4*)(b_g + b_src[i]);
#pragma unroll
        for (int i = 0; i < A_PER; ++i)
            if (a_ok[i]) *(i32x4*)(smem + a_dst[i]) = ra[i];
#pragma unroll
        for (int i = 0; i < B_PER; ++i)
            if (b_ok[i]) *(i32x4*)(smem + b_dst[i]) = rb[i];
        __syncthreads();

        for (int c = 0; c < kchunks; ++c) {
            const bool more = c + 1 < kchunks;
            if (more) {
                const int64_t off = (int64_t)(c + 1) * 128;
#pragma unroll
                for (int i = 0; i < A_PER; ++i)
                    if (a_ok[i]) ra[i] = *(const i32x4*)(a_g + a_src[i] + off);
#pragma unroll
                for (int i = 0; i < B_PER; ++i)
                    if (b_ok[i]) rb[i] = *(const i32x4*)(b_g + b_src[i] + off);
            }
            // scales of chunk c
            f32x4 sa[TM];
#pragma unroll
            for (int i = 0; i < TM; ++i) sa[i] = *(const f32x4*)(sfa_g + (int64_t)c * p.sfa_ld + sa_row[i]);
            float sb[TN];
#pragma unroll
            for (int j = 0; j < TN; ++j) sb[j] = sfb_g[sb_blk[j] * kchunks + c];

            const uint8_t* st = smem + (c & 1) * STAGE;
            i32x8 af[TM], bf[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const i32x4 lo = *(const i32x4*)(st + a_frag[i][0]);
                const i32x4 hi = *(const i32x4*)(st + a_frag[i][1]);
                af[i] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const i32x4 lo = *(const i32x4*)(st + b_frag[j][0]);
                const i32x4 hi = *(const i32x4*)(st + b_frag[j][1]);
                bf[j] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            }
#pragma unroll
            for (int i = 0; i < TM; ++i) {
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const f32x4 part = mfma_e4m3_16x16x128(af[i], bf[j]);
#pragma unroll
                    for (int v = 0; v < 4; ++v) acc[i][j][v] += part[v] * (sa[i][v] * sb[j]);
                }
            }
            if (more) {
                uint8_t* nx = smem + ((c + 1) & 1) * STAGE;
#pragma unroll
                for (int i = 0; i < A_PER; ++i)
                    if (a_ok[i]) *(i32x4*)(nx + a_dst[i]) = ra[i];
#pragma unroll
                for (int i = 0; i < B_PER; ++i)
                    if (b_ok[i]) *(i32x4*)(nx + b_dst[i]) = rb[i];
            }
            __syncthreads();
        }

        // ---- epilogue: BF16 stores at valid rows / columns only ----
        uint16_t* d_g = p.d + (LAYOUT == kMasked ? (int64_t)g * p.m * p.n : (int64_t)0);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = m0 + wm * WTM + i * 16 + kg * 4 + v;
                bool row_ok = row < row_limit;
                if (LAYOUT == kContiguous && row_ok) row_ok = p.grouped_layout[row] == g;
                if (!row_ok) continue;
                uint16_t* drow = d_g + (int64_t)row * p.n;
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int col = n0 + wn * WTN + j * 16 + (lane & 15);
                    if (col < p.n) drow[col] = to_bf16_rne(acc[i][j][v]);
                }
            }
        }
    }
}

typedef void (*KernelFn)(GemmParams);

struct InstanceEntry {
    KernelFn fn[3];
    int threads;
};

#define FP8BS_INSTANCE(BM, BN, WM, WN, OCC)                                   \
    {{fp8bs_gemm_kernel<BM, BN, WM, WN, kDense>,                              \
      fp8bs_gemm_kernel<BM, BN, WM, WN, kContiguous>,                         \
      fp8bs_gemm_kernel<BM, BN, WM, WN, kMasked>},                            \
     64 * (WM) * (WN)},
const InstanceEntry kEntries[] = {
#include "fp8bs_instances.inc"
};
#undef FP8BS_INSTANCE

}  // namespace

int launch_instance(const Plan& plan, int layout, const GemmParams& p, hipStream_t stream) {
    if (plan.instance < 0 || plan.instance >= (int)(sizeof(kEntries) / sizeof(kEntries[0])))
        return (int)hipErrorInvalidValue;
    const InstanceEntry& e = kEntries[plan.instance];
    GemmParams args = p;
    void* argv[] = {&args};
    return (int)hipLaunchKernel((const void*)e.fn[layout], dim3((unsigned)plan.grid),
                                dim3(e.threads), argv, 0, stream);
}

}  // namespace fp8bs
