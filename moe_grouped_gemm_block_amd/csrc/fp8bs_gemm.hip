// fp8bs_gemm.hip -- the block-scaled FP8 GEMM kernels for gfx950 (CDNA4).
//
// One kernel template serves the dense, contiguous-grouped and masked-grouped
// layouts (the DeepGEMM README repost, lqnn.cn/news/60274, sections
// "DeepGEMM" and "优化技术": one core kernel and one block scheduler for the
// grouped and non-grouped GEMMs).  Per output tile and per 128-wide K chunk:
//
//   1. The A tile (block_m x 128 e4m3), the B tile (block_n x 128 e4m3), the
//      tile's block_m A scales and its B-scale values are copied global -> LDS
//      by direct-to-LDS loads (global_load_lds_dwordx4 / _dword) into a ring of
//      NS stages: while one chunk is multiplied, the next NS-1 chunks -- of
//      this work unit or of the next ones the workgroup owns -- stream in.
//   2. Each wavefront multiplies its sub-tile with v_mfma_f32_16x16x128_f8f6f4
//      (OCP e4m3 x e4m3, FP32 result), one instruction per 16x16 output block
//      per chunk, into a partial that starts from zero every chunk.
//   3. The partial is promoted into the FP32 accumulator on the vector ALU:
//      acc += partial * (sfa[row] * sfb[column block]) -- the two-level
//      accumulation of the same page's "DeepGEMM" section.
//   4. After the unit's last chunk the accumulator is rounded to BF16 (nearest
//      even) and stored at valid rows and columns, or -- when the planner splits
//      K -- stored as an FP32 partial that fp8bs_splitk_reduce adds up in a
//      fixed order.
//
// MFMA operand roles are transposed: B rows feed the instruction's first
// operand and A rows its second, so each lane's four results share one A row
// (one row scale: one multiply per 16x16 block, not four) and cover four
// consecutive columns (one 8-byte BF16 store).  Lane j of a wavefront supplies
// TM consecutive A rows across its TM row blocks, so its row scales are one
// contiguous LDS read.
//
// The schedule is persistent: workgroup w processes work units w, w + grid, ...
// A unit is (K split s, tile t), split-major so that concurrent units share the
// K range; tiles are rasterised (groups of `raster` m-blocks sweep the n-blocks
// so that concurrent tiles share A and B stripes in L2), and workgroup ids are
// remapped so that each XCD (workgroups are dealt to the 8 XCDs round-robin)
// runs a contiguous range of that order.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "fp8bs_internal.h"

namespace fp8bs {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

#define GLOBAL_AS __attribute__((address_space(1)))
#define LDS_AS __attribute__((address_space(3)))

// 16x16x128 FP8 (OCP e4m3 x e4m3) matrix product with a zero addend.  Lane l
// supplies row l%16 of the first operand and column l%16 of the second, 32 K
// bytes each; the K position of each byte is the same function of (l/16, byte)
// for both operands, so any fixed assignment of the chunk's 128 K values to
// those slots (identical for both) gives the full chunk dot product.  Lane l
// receives rows 4*(l/16)+v, v = 0..3, of column l%16.
__device__ __forceinline__ f32x4 mfma_e4m3(const i32x8& first, const i32x8& second) {
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    // format codes 0/0 = e4m3 for both operands; block scales off (scale 0, opsel 0)
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(first, second, zero, 0, 0, 0, 0, 0, 0);
}

// Wait until this wavefront has at most N vector-memory operations (direct-to-LDS
// copies included) and no LDS / scalar-memory operation outstanding.
template <int N>
__device__ __forceinline__ void wait_loads() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    // gfx9 s_waitcnt layout: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[15:14]
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier without a memory fence: the explicit waits before it make this
// wavefront's copies and reads complete; the clobber keeps the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Cache policy of a copy: kCacheNormal, or kCacheStream (non-temporal, the "nt" bit) for
// operand bytes that one tile reads once and no other tile of the launch reads again.
constexpr int kCacheNormal = 0, kCacheStream = 2;
template <int CPOL = kCacheNormal>
__device__ __forceinline__ void dma16(const void* src, LDS_AS void* dst_wave_base) {
    __builtin_amdgcn_global_load_lds((const GLOBAL_AS void*)src, dst_wave_base, 16, 0, CPOL);
}

// B's cache policy per layout in the staged kernel (the B-streaming kernel always loads B
// non-temporally).  Masked: a slot's B block is read by the slot's m-blocks only -- one
// tile when block_m covers max_m -- so it is streamed non-temporally (measured on MI355X,
// the masked MoE shapes with 256-row tiles: 182 -> 155 us and 113 -> 96 us; plain
// streaming reads of a cold 1 GiB buffer: 4.6-4.9 TB/s normal, 6.1-7.1 TB/s with
// non-temporal loads).  Dense and contiguous B tiles are shared by the tiles of a raster
// group through L2, where non-temporal copies measured slower (up to 13%).
template <int LAYOUT>
constexpr int b_cache_policy() { return LAYOUT == kMasked ? kCacheStream : kCacheNormal; }

// Compile-time loop: f(std::integral_constant<int, I>) for I = B .. E-1.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));   // v_cvt_pk_bf16_f32
}

__device__ __forceinline__ uint16_t to_bf16(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// Workgroup id -> position in the schedule.  Workgroup b runs on XCD b % 8, so
// XCD x is handed the contiguous range [x * grid/8, (x+1) * grid/8).
__device__ __forceinline__ int logical_block_id() {
    const int n = gridDim.x, b = blockIdx.x;
    if ((n & 7) != 0) return b;
    return (b & 7) * (n >> 3) + (b >> 3);
}

// LDS transpose read (ds_read_b64_tr_b8, gfx950).  Within each group of 16 lanes, lane s
// supplies the address of an 8-byte row R_s; lane t receives byte (t % 8) of the rows
// R_{t/8}, R_{t/8 + 2}, ..., R_{t/8 + 14}, in that order (behaviour measured on MI355X).
// With lane s pointing at k-row kb + s/2, bytes 8*(s%2) .. +7 of a 16-column run of an
// MN-major tile, lane t therefore gets column t of the run at k = kb .. kb+7: eight
// consecutive K values of one operand row, as an MFMA fragment needs them.
typedef int i32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ i32x2_t lds_read_tr8(const uint8_t* p) {
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS i32x2_t*)(LDS_AS void*)p);
}

// Swizzle key of k-row `kr` of an MN-major tile with U 16-byte units per row (U = 2 .. 16):
// physical unit = logical unit ^ key.  A transpose read has each 16-lane group read one
// logical unit of 8 consecutive k-rows, and the two groups of a half-wavefront rows 32
// apart; the key spreads those 16 (row, unit) pairs over all 64 banks.  The key of rows
// 32q + 8r + j (j < 8) depends only on j and q % 2.
template <int U>
__device__ __forceinline__ int mn_key(int kr) {
    static_assert(U == 2 || U == 4 || U == 8 || U == 16, "MN-major tile width");
    constexpr int ROWS_PER_256B = 16 / U;
    return ((kr / ROWS_PER_256B) & (U / 2 - 1)) | (((kr >> 5) & 1) * (U / 2));
}

// LDS swizzle keys (see the fragment-address comment in the kernel).
__device__ __forceinline__ int b_key(int row) { return (row & 7) ^ ((row >> 3) & 1); }
template <int TM>
__device__ __forceinline__ int a_key(int row) {
    return TM > 1 ? (row / TM) & 7 : b_key(row);
}

struct Tile {
    int g, m0, n0, row_limit;
};

// Tile (slot / group g, m-block mb, n-block nb) -> its rows, columns and expert.  Returns
// false when the tile holds no valid row (masked: beyond masked_m; contiguous: padding).
template <int BM, int BN, int LAYOUT>
__device__ __forceinline__ bool tile_at_block(const GemmParams& p, int g, int mb, int nb,
                                              Tile& tl, int pass = 0) {
    tl.m0 = mb * BM;
    tl.n0 = nb * BN;
    tl.row_limit = p.m;
    if (LAYOUT == kMasked) {
        const int v = min(max(p.masked_m[g], 0), p.m);
        if (tl.m0 >= v) return false;
        tl.row_limit = v;
    } else if (LAYOUT == kContiguous) {
        // A 128-row block holds one expert's rows, then padding; its first row names it.
        auto expert = [&](int row) {
            if (row >= p.m) return -1;
            const int e = p.grouped_layout[row];
            return (e >= 0 && e < p.num_groups) ? e : -1;
        };
        const int e0 = expert(tl.m0);
        if constexpr (BM <= 128) {
            if (e0 < 0) return false;
            g = e0;
        } else {
            // A 256-row tile covers two blocks.  Pass 0 multiplies the tile with the first
            // block's expert (the second's when the first is all padding); pass 1 with the
            // second block's expert when that is a different one.  store_tile writes only
            // the rows whose index is the pass's expert.
            const int e1 = expert(tl.m0 + 128);
            if (pass == 0) {
                g = e0 >= 0 ? e0 : e1;
                if (g < 0) return false;
            } else {
                if (e0 < 0 || e1 < 0 || e1 == e0) return false;
                g = e1;
            }
        }
    }
    tl.g = g;
    return true;
}

// Schedule position -> tile.  Masked and K-grouped: group-major.  Within a slot, groups of
// `raster` m-blocks sweep the n-blocks column by column.  Returns false when
// the tile holds no valid row (masked: beyond masked_m; contiguous: padding).
template <int BM, int BN, int LAYOUT>
__device__ __forceinline__ bool tile_at(const GemmParams& p, int t, Tile& tl, int pass = 0) {
    int rest = t, g = 0;
    if (LAYOUT == kMasked || LAYOUT == kKGrouped) {
        const int per_slot = p.m_blocks * p.n_blocks;
        g = t / per_slot;
        rest = t - g * per_slot;
    }
    const int per_group = p.raster * p.n_blocks;
    const int grp = rest / per_group;
    const int r = rest - grp * per_group;
    const int first = grp * p.raster;
    const int rows_in = min(p.raster, p.m_blocks - first);
    return tile_at_block<BM, BN, LAYOUT>(p, g, first + r % rows_in, r / rows_in, tl, pass);
}

// First chunk of K split s of n chunks in `splits` ranges: floor(s * n / splits), in 32-bit
// unsigned arithmetic (the planner keeps splits * n below 2^32; a 64-bit division would cost
// every workgroup a division loop in its prologue).
__device__ __forceinline__ int split_bound(int s, int n, int splits) {
    return (int)((uint32_t)s * (uint32_t)n / (uint32_t)splits);
}

// A work unit: K split s of tile t, chunks [c0, c1).
struct Unit {
    int u, t, s, c0, c1;
    Tile tl;
};

struct NoEmptyUnits {
    __device__ void operator()(const Unit&) const {}
};

// Contiguous layout with 256-row tiles: the work list of (m-block, pass) pairs, one pass per
// expert an m-block holds (two when its 128-row halves belong to different experts),
// numbered densely so that the persistent workgroups share the real work evenly (unit
// indices past the list are empty and end the workgroup's stream).  "Virtual m-block" v
// is m-block mb's pass q, v = mb + (two-expert m-blocks before mb) + q; the i-th
// two-expert m-block B_i (in order) therefore has its second pass at v = B_i + i + 1.
// Experts are contiguous segments, so at most G - 1 m-blocks hold two; the list keeps up to
// 64 of them, lane i of one register holding B_i + i + 1 (lanes past the count: INT_MAX),
// and is decoded with two ballots -- no memory access inside the chunk loop.
constexpr int kPassListMax = 64;
struct PassList {
    int count;             // two-expert m-blocks; < 0: list not built, sparse pass-major units
    int vblocks;           // m-blocks plus two-expert m-blocks
    int second;            // this lane's B_i + i + 1
};

// Virtual m-block v -> (m-block, pass).
__device__ __forceinline__ void pass_decode(const PassList& pl, int v, int& mb, int& pass) {
    const int before = __popcll(__ballot(pl.second < v));   // second passes before v
    pass = __ballot(pl.second == v) != 0ull ? 1 : 0;
    mb = v - before - pass;
}

// Builds the list for this workgroup's wavefront (every wavefront builds its own copy from
// grouped_layout; no LDS).  Returns count = -1 when more than kPassListMax m-blocks hold two
// experts.
template <int BM>
__device__ __forceinline__ PassList pass_list_build(const GemmParams& p, int lane) {
    PassList pl{0, p.m_blocks, 0x7fffffff};
    int count = 0;
    for (int w0 = 0; w0 < p.m_blocks; w0 += 64) {
        const int mb = w0 + lane;
        bool two = false;
        if (mb < p.m_blocks) {
            const int r0 = mb * BM, r1 = r0 + 128;
            const int e0 = p.grouped_layout[r0];
            const int e1 = r1 < p.m ? p.grouped_layout[r1] : -1;
            two = e0 >= 0 && e0 < p.num_groups && e1 >= 0 && e1 < p.num_groups && e0 != e1;
        }
        const uint64_t bits = __ballot(two);
        const int n = __popcll(bits);
        if (count + n > kPassListMax) return PassList{-1, p.m_blocks, 0x7fffffff};
        // lane count + k takes the k-th set bit of this word
        const int k = lane - count;
        if (k >= 0 && k < n) {
            int pos = 0;
            for (int step = 32; step > 0; step >>= 1)
                if (__popcll(bits & ((1ull << (pos + step)) - 1ull)) <= k) pos += step;
            pl.second = (w0 + pos) + lane + 1;
        }
        count += n;
    }
    pl.count = count;
    pl.vblocks = p.m_blocks + count;
    return pl;
}

// The next unit at or after schedule position u (stepping by the grid) that has chunks to
// multiply.  K-grouped: a unit's chunks are split s of its group's chunks, and a unit
// with none (an empty group, or more splits than the group has chunks) is handed to
// on_empty -- which stores its all-zero result -- and skipped.
template <int BM, int BN, int LAYOUT, typename OnEmpty = NoEmptyUnits>
__device__ __forceinline__ bool next_unit(const GemmParams& p, int u, Unit& w,
                                          OnEmpty&& on_empty = OnEmpty{},
                                          const PassList* pl = nullptr) {
    const int kchunks = p.k / 128;
    // contiguous layout, 256-row tiles: units are (pass, tile), never split
    constexpr bool PASSES = LAYOUT == kContiguous && BM > 128;
    if constexpr (PASSES) {
        if (pl && pl->count >= 0) {
            // dense (m-block, pass) list, rastered like tile_at's m-blocks
            for (; u < pl->vblocks * p.n_blocks; u += gridDim.x) {
                const int per_group = p.raster * p.n_blocks;
                const int grp = u / per_group;
                const int r = u - grp * per_group;
                const int first = grp * p.raster;
                const int rows_in = min(p.raster, pl->vblocks - first);
                int mb, pass;
                pass_decode(*pl, first + r % rows_in, mb, pass);
                const int nb = r / rows_in;
                if (!tile_at_block<BM, BN, LAYOUT>(p, 0, mb, nb, w.tl, pass)) continue;
                w.u = u;
                w.t = mb * p.n_blocks + nb;
                w.s = 0;
                w.c0 = 0;
                w.c1 = kchunks;
                return true;
            }
            return false;
        }
    }
    for (; u < p.units; u += gridDim.x) {
        const int q = u / p.tiles, t = u - q * p.tiles;
        const int s = PASSES ? 0 : q;
        if (!tile_at<BM, BN, LAYOUT>(p, t, w.tl, PASSES ? q : 0)) continue;
        w.u = u;
        w.t = t;
        w.s = s;
        if constexpr (LAYOUT == kKGrouped) {
            const int cb = p.kg_chunk0[w.tl.g];
            const int nch = p.kg_chunk0[w.tl.g + 1] - cb;
            w.c0 = cb + split_bound(s, nch, p.splits);
            w.c1 = cb + split_bound(s + 1, nch, p.splits);
            if (w.c0 == w.c1) {
                on_empty(w);
                continue;
            }
        } else {
            w.c0 = split_bound(s, kchunks, p.splits);
            w.c1 = split_bound(s + 1, kchunks, p.splits);
        }
        return true;
    }
    return false;
}

// 4x4 transpose of one register across the four 16-lane rows of a wavefront: on entry
// x[r] of row q is element (q, r); on exit x[r] of row q is element (r, q).
// v_permlane32_swap exchanges rows 2-3 of its first operand with rows 0-1 of its second,
// v_permlane16_swap the odd rows of the first with the even rows of the second.
__device__ __forceinline__ void transpose_quarters(uint32_t (&x)[4]) {
    auto a = __builtin_amdgcn_permlane32_swap(x[0], x[2], false, false);
    auto b = __builtin_amdgcn_permlane32_swap(x[1], x[3], false, false);
    auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
    auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
    x[0] = c[0];
    x[1] = c[1];
    x[2] = d[0];
    x[3] = d[1];
}

// Rows / columns this lane holds in a tile and the store of an accumulator set:
// lane (j = l%16, quarter kq = l/16) of wavefront (wm, wn) owns rows
// m0 + wm*WTM + TM*j + (i ^ flip) (ROWS16: m0 + wm*WTM + 16*i + j, the row order of an
// MN-major A read by transpose loads) and columns n0 + wn*WTN + 16*jn + 4*kq .. +3.
// BF16 output; the K-grouped layout stores FP32 into D [G][M][N].
template <int TM, int TN, int WTM, int WTN, int LAYOUT, bool ROWS16 = false>
__device__ __forceinline__ void store_tile(const GemmParams& p, const Tile& tl, const f32x4 (&acc)[TM][TN],
                                           int wm, int wn, int lj, int kq, int flip) {
    if constexpr (LAYOUT == kKGrouped) {
        const int64_t slot = (int64_t)tl.g * p.m * p.n;
        float* d_g = (float*)(void*)p.d + slot;
        const bool vec_ok = (p.n & 3) == 0;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int row = tl.m0 + wm * WTM + (ROWS16 ? 16 * i + lj : TM * lj + (i ^ flip));
            if (row >= tl.row_limit) continue;
            float* drow = d_g + (int64_t)row * p.n;
            const float* crow = p.c ? p.c + slot + (int64_t)row * p.n : nullptr;
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int col = tl.n0 + wn * WTN + 16 * j + 4 * kq;
                f32x4 v = acc[i][j];
                if (vec_ok && col + 3 < p.n) {
                    if (crow) v += *(const f32x4*)(crow + col);
                    *(f32x4*)(drow + col) = v;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (col + e < p.n) drow[col + e] = crow ? v[e] + crow[col + e] : v[e];
                }
            }
        }
        return;
    }
    const int64_t slot = LAYOUT == kMasked ? (int64_t)tl.g * p.m * p.n : (int64_t)0;
    uint16_t* d_g = p.d + slot;
    const bool vec_ok = (p.n & 3) == 0;
    const bool wide_ok = (p.n & 7) == 0;              // rows start 16-byte aligned
    constexpr int NG = TN / 4;                        // groups of four column blocks
    // this lane's four results of block j, plus C, as two BF16 pairs
    auto packed = [&](int i, int j, const float* crow, uint32_t& lo, uint32_t& hi) {
        const int col = tl.n0 + wn * WTN + 16 * j + 4 * kq;
        f32x4 v = acc[i][j];
        if (crow) {                                  // D = C + A B^T
            if (vec_ok && col + 3 < p.n) {
                v += *(const f32x4*)(crow + col);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (col + e < p.n) v[e] += crow[col + e];
            }
        }
        lo = pack_bf16x2(v[0], v[1]);
        hi = pack_bf16x2(v[2], v[3]);
    };
    // Contiguous: which of this wavefront's rows hold the tile's expert, found before any
    // store (a load between the stores would wait for every earlier store of the
    // wavefront: the memory counter retires in issue order).  Each lane reads one row of
    // each 64-row half of the wavefront's rows and a ballot turns the answers into a
    // 64-bit mask per half; the lane's own rows lie in one half.
    uint64_t expert_rows = 0;
    int expert_bit0 = 0;
    if constexpr (LAYOUT == kContiguous) {
        static_assert(!ROWS16 && WTM <= 128, "row masks cover two 64-row halves");
        uint64_t half[2] = {0, 0};
#pragma unroll
        for (int h = 0; h < (WTM + 63) / 64; ++h) {
            const int r = tl.m0 + wm * WTM + 64 * h + lj + 16 * kq;
            const bool mine = r < tl.row_limit &&
                              p.grouped_layout[min(r, tl.row_limit - 1)] == tl.g;
            half[h] = __ballot(mine);
        }
        expert_rows = (TM * lj) < 64 ? half[0] : half[1];
        expert_bit0 = (TM * lj) & 63;
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int row = tl.m0 + wm * WTM + (ROWS16 ? 16 * i + lj : TM * lj + (i ^ flip));
        bool ok = row < tl.row_limit;
        if constexpr (LAYOUT == kContiguous)
            ok = ok && ((expert_rows >> (expert_bit0 + (i ^ flip))) & 1u);
        uint16_t* drow = d_g + (int64_t)row * p.n;
        const float* crow = (p.c && ok) ? p.c + slot + (int64_t)row * p.n : nullptr;
        // Four column blocks at a time: the four lanes of a row (quarters kq = 0..3) hold
        // columns 4kq..4kq+3 of every block; a 4x4 exchange across quarters (two rounds of
        // gfx950 row swaps) leaves quarter kq with all 16 columns of block 4g + kq, stored
        // as two 16-byte writes, so a row's 4 blocks go out as one 128-byte run.  Every
        // lane takes part in the exchange; rows that are not written skip the stores.
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            uint32_t lo[4], hi[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) packed(i, 4 * g + jj, crow, lo[jj], hi[jj]);
            transpose_quarters(lo);
            transpose_quarters(hi);
            if (!ok) continue;
            const int cb = tl.n0 + wn * WTN + 16 * (4 * g + kq);
            if (wide_ok && cb + 15 < p.n) {
                *(uint4*)(drow + cb) = uint4{lo[0], hi[0], lo[1], hi[1]};
                *(uint4*)(drow + cb + 8) = uint4{lo[2], hi[2], lo[3], hi[3]};
            } else {
#pragma unroll
                for (int c = 0; c < 16; ++c) {
                    const uint32_t w = (c & 2) ? hi[c >> 2] : lo[c >> 2];
                    if (cb + c < p.n) drow[cb + c] = (uint16_t)(w >> (16 * (c & 1)));
                }
            }
        }
        if (!ok) continue;
#pragma unroll
        for (int j = 4 * NG; j < TN; ++j) {
            const int col = tl.n0 + wn * WTN + 16 * j + 4 * kq;
            uint32_t lo, hi;
            packed(i, j, crow, lo, hi);
            if (vec_ok && col + 3 < p.n) {
                *(uint2*)(drow + col) = uint2{lo, hi};
            } else {
                if (col < p.n) drow[col] = (uint16_t)lo;
                if (col + 1 < p.n) drow[col + 1] = (uint16_t)(lo >> 16);
                if (col + 2 < p.n) drow[col + 2] = (uint16_t)hi;
                if (col + 3 < p.n) drow[col + 3] = (uint16_t)(hi >> 16);
            }
        }
    }
}

// Offset (in f32x4) of accumulator (i, j) of this thread inside one unit's FP32 partial
// tile in the workspace: [wavefront][i][j][lane], so a wavefront's store is contiguous.
template <int TM, int TN>
__device__ __forceinline__ int partial_index(int wave, int i, int j, int lane) {
    return ((wave * TM + i) * TN + j) * 64 + lane;
}

template <int BM, int BN, int WM, int WN, int NS, int LAYOUT, int SCALE, bool AMN = false,
          bool BMN = false>
__global__ void __launch_bounds__(64 * WM * WN) fp8bs_gemm_kernel(GemmParams p) {
    // SCALE == kScaleF32: FP32 scales, per-chunk promotion on the VALU.
    // SCALE == kScaleUE8M0: power-of-two scales, E8M0 exponents packed four K groups per
    // 32-bit word; the matrix core applies them (v_mfma_scale_*: each operand row's
    // 32-element K blocks multiplied by 2^(e-127)) and accumulates across chunks itself,
    // so there is no promotion step.
    // AMN / BMN: A stored [K][M] / B stored [K][N] (MN-major).  Such a tile sits in LDS as
    // 128 k-rows of block_m (block_n) bytes, 16-byte units swizzled by mn_key, and its
    // fragments are read with transpose loads; an MN-major A's 16-row blocks are 16
    // consecutive rows (ROWS16 in store_tile).
    // LAYOUT == kKGrouped: both operands MN-major, per-group K ranges, B scaled per column
    // (SFB [K_total/128][sfb_ld], or packed words [ceil(K_total/512)][sfb_ld]), FP32 output.
    constexpr bool E8 = SCALE == kScaleUE8M0;
    constexpr bool KG = LAYOUT == kKGrouped;
    static_assert(!KG || (AMN && BMN), "the K-grouped layout has MN-major operands");
    static_assert(!(AMN || BMN) || LAYOUT == kDense || KG,
                  "MN-major operands: dense or K-grouped");
    constexpr int NW = WM * WN;                      // wavefronts per workgroup
    constexpr int WTM = BM / WM, WTN = BN / WN;      // wavefront sub-tile
    constexpr int TM = WTM / 16, TN = WTN / 16;      // 16x16 blocks per wavefront
    static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wavefront tile must be a multiple of 16");
    static_assert(BM % 8 == 0 && BN % 8 == 0 && BM <= 256, "tile shape");
    static_assert(TM == 1 || TM == 2 || TM == 4 || TM == 8, "row blocks per wavefront");
    static_assert(NS >= 2, "at least two stages");
    constexpr int A_OFF = 0, B_OFF = BM * 128, SA_OFF = (BM + BN) * 128, SB_OFF = SA_OFF + BM * 4;
    constexpr int STAGE = KG ? kgrouped_stage_bytes(BM, BN) : stage_bytes(BM, BN);
    static_assert(!AMN || (BM >= 32 && BM <= 256 && (BM & (BM - 1)) == 0), "MN-major A tile");
    static_assert(!BMN || (BN >= 32 && BN <= 256 && (BN & (BN - 1)) == 0), "MN-major B tile");
    constexpr int A_INS = BM / 8, B_INS = BN / 8;    // 1 KB (8 rows) per wavefront copy
    constexpr int A_PER = (A_INS + NW - 1) / NW, B_PER = (B_INS + NW - 1) / NW;
    static_assert(A_INS >= NW && B_INS >= NW, "every wavefront must own at least one A and one B copy");
    static_assert(NS * STAGE <= kLdsBytesPerCu, "LDS ring too large");
    constexpr int SB_SPAN = BN / 128 + 2;            // B-scale blocks a tile can touch
    // Every wavefront issues the same number of copies per chunk (A_PER + B_PER + one
    // scale copy; a wavefront with no copy left repeats one, writing identical bytes),
    // so "chunk q+1 has landed" is a constant vmcnt after the copies of NS-2 later chunks.
    constexpr int OPC = A_PER + B_PER + 1;
    static_assert((NS - 2) * OPC <= 63, "vmcnt range");
    // the wave's columns lie in one 128-column scale block for every tile
    constexpr bool UNIFORM_SB = (BN % 128 == 0) && (128 % WTN == 0);

    __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * STAGE];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int kchunks = p.k / 128;
    const int K = p.k;
    const int nsb = (p.n + 127) / 128;

    // ---- fragment read addresses (byte offsets in a stage) ----
    // Rows are 128 bytes; 16-byte unit u of row r is stored at slot u ^ key(r).  A read of
    // 16 bytes per lane is free of bank conflicts when lanes 0-7 (and 8-15) hit eight
    // distinct slots and lanes 0-15 hit sixteen distinct (row parity, slot) pairs.
    // A rows (TM > 1): lane j = l%16 owns rows wm*WTM + TM*j + (i ^ flip), flip = j / 8
    // (rows of lanes j and j+8 differ in parity), key = (row / TM) & 7 = j & 7.
    // B rows (and A rows when TM == 1): lane i' reads row base + i', key = (i' & 7) ^ (i' / 8).
    // Neither key depends on the block index, so block i / j is an immediate offset.
    const int lj = lane & 15;
    const int kq = lane >> 4;                         // 32-byte quarter of the chunk
    const int flip = (TM > 1 && !AMN) ? (lj >> 3) : 0;
    // MN-major operands: lane (lj, kq) supplies, for its four transpose reads r = 0..3,
    // k-row 32*kq + 8*r + lj/2 and bytes 8*(lj%2) .. +7 of the block's 16-byte unit; the
    // unit's swizzle key does not depend on r.
    const int tr_row = 32 * kq + (lj >> 1);
    const int a_tr = A_OFF + tr_row * BM + 8 * (lj & 1);
    const int a_tr_key = [&] {
        if constexpr (AMN) return mn_key<BM / 16>(tr_row);
        else return 0;
    }();
    const int b_tr = B_OFF + tr_row * BN + 8 * (lj & 1);
    const int b_tr_key = [&] {
        if constexpr (BMN) return mn_key<BN / 16>(tr_row);
        else return 0;
    }();
    int a_even[2], a_odd[2];                          // row block i at +128*i (even / odd i)
    {
        const int row0 = wm * WTM + TM * lj;
        const int key = a_key<TM>(row0);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int base = A_OFF + row0 * 128 + (((2 * kq + h) ^ key) << 4);
            a_even[h] = base + flip * 128;            // (i ^ flip) = i + flip for even i
            a_odd[h] = base - flip * 128;             // (i ^ flip) = i - flip for odd i
        }
    }
    int b_base[2];                                    // column block j at +2048*j
    {
        const int row0 = wn * WTN + lj;
        const int key = b_key(row0);
#pragma unroll
        for (int h = 0; h < 2; ++h) b_base[h] = B_OFF + row0 * 128 + (((2 * kq + h) ^ key) << 4);
    }
    const int sa_rd = SA_OFF + (wm * WTM + (AMN ? lj : TM * lj)) * 4;

    // ---- copies: wavefront copy `ins` moves tile rows 8*ins .. 8*ins+7; lane L fills LDS
    // slot L%8 of row 8*ins + L/8 with the global 16-byte unit (slot ^ key(row)) ----
    // The swizzle key of a copied row is the same for rows r and r + 8*NW, so the lane
    // offset of every copy of a tile is one value plus a uniform multiple of 8*NW rows.
    static_assert(AMN || (TM == 1 || NW % TM == 0), "copy offsets must repeat");
    static_assert(NW % 2 == 0, "wavefront count");
    const int cp_row = lane >> 3, cp_slot = lane & 7;
    const uint32_t a_lane = (uint32_t)(8 * wave + cp_row) * (uint32_t)K +
                            (uint32_t)((cp_slot ^ a_key<TM>(8 * wave + cp_row)) << 4);
    const uint32_t b_lane = (uint32_t)(8 * wave + cp_row) * (uint32_t)K +
                            (uint32_t)((cp_slot ^ b_key(8 * wave + cp_row)) << 4);
    // copy chunk c of tile `tl` into stage s
    // MN-major copy: wavefront copy `ins` fills LDS bytes ins*1024 .. +1023 of the tile,
    // k-rows of W bytes; lane L's 16 bytes are physical unit (16L % W) / 16 of k-row
    // (1024 ins + 16L) / W, read from the global row (leading dimension ld) at the
    // logical unit, clamped to the last whole unit of the row (lim = ld - 16) so that no
    // read leaves the operand; columns past the edge only feed outputs never stored.
    auto mn_copy = [&](const uint8_t* chunk, int ld, int lim, int col0, auto w_const, int ins,
                       LDS_AS void* dst) {
        constexpr int W = decltype(w_const)::value;
        const int off = ins * 1024 + 16 * lane;
        const int kr = off / W;
        const int u = ((off % W) >> 4) ^ mn_key<W / 16>(kr);
        const int col = min(col0 + 16 * u, lim);
        dma16(chunk + (uint32_t)(kr * ld + col), dst);
    };
    // The copies of chunk c into stage s are OPC parts: A copies 0 .. A_PER-1, B copies
    // A_PER .. A_PER+B_PER-1, the scale copy last.  issue_parts issues parts P0 .. P1-1.
    auto issue_parts = [&](const Tile& tl, int c, int s, auto p0_const, auto p1_const) {
        constexpr int P0 = decltype(p0_const)::value, P1 = decltype(p1_const)::value;
        constexpr bool ANY_A = P0 < A_PER, ANY_B = P0 < A_PER + B_PER && P1 > A_PER;
        constexpr bool SCALES = P1 == OPC;
        constexpr int A1 = P1 < A_PER ? P1 : A_PER;                 // A copies P0 .. A1-1
        constexpr int B0 = P0 > A_PER ? P0 - A_PER : 0;             // B copies B0 .. B1-1
        constexpr int B1 = P1 - A_PER < B_PER ? P1 - A_PER : B_PER;
        uint8_t* st = smem + s * STAGE;
        const uint8_t* a_base = p.a + (LAYOUT == kMasked ? (int64_t)tl.g * p.m * K : (int64_t)0) +
                                (int64_t)c * 128;
        const uint8_t* b_base = p.b + (KG ? (int64_t)0 : (int64_t)tl.g * p.n * K) + (int64_t)c * 128;
        if constexpr (!ANY_A) {
        } else if constexpr (AMN) {
            const uint8_t* a_chunk = p.a + (int64_t)c * 128 * p.m;
#pragma unroll
            for (int k = P0; k < A1; ++k) {
                const int kk = (A_INS % NW == 0 || wave + k * NW < A_INS) ? k : k - 1;
                mn_copy(a_chunk, p.m, p.m - 16, tl.m0, std::integral_constant<int, BM>{},
                        wave + kk * NW, (LDS_AS void*)(st + A_OFF + (wave + kk * NW) * 1024));
            }
        } else if (tl.m0 + BM <= tl.row_limit) {      // whole tile inside: no clamping
            const uint8_t* a_t = a_base + (int64_t)tl.m0 * K;
#pragma unroll
            for (int k = P0; k < A1; ++k) {
                const int kk = (A_INS % NW == 0 || wave + k * NW < A_INS) ? k : k - 1;
                dma16(a_t + (int64_t)kk * 8 * NW * K + a_lane,
                      (LDS_AS void*)(st + A_OFF + (wave + kk * NW) * 1024));
            }
        } else {
#pragma unroll
            for (int k = P0; k < A1; ++k) {
                const int ins = (A_INS % NW == 0 || wave + k * NW < A_INS) ? wave + k * NW : A_INS - 1;
                const int row = 8 * ins + cp_row;
                const int grow = min(tl.m0 + row, tl.row_limit - 1);
                const uint32_t off = (uint32_t)grow * (uint32_t)K + (uint32_t)((cp_slot ^ a_key<TM>(row)) << 4);
                dma16(a_base + off, (LDS_AS void*)(st + A_OFF + ins * 1024));
            }
        }
        if constexpr (!ANY_B) {
        } else if constexpr (BMN) {
            const uint8_t* b_chunk = p.b + (int64_t)c * 128 * p.n;
#pragma unroll
            for (int k = B0; k < B1; ++k) {
                const int kk = (B_INS % NW == 0 || wave + k * NW < B_INS) ? k : k - 1;
                mn_copy(b_chunk, p.n, p.n - 16, tl.n0, std::integral_constant<int, BN>{},
                        wave + kk * NW, (LDS_AS void*)(st + B_OFF + (wave + kk * NW) * 1024));
            }
        } else if (tl.n0 + BN <= p.n) {
            const uint8_t* b_t = b_base + (int64_t)tl.n0 * K;
#pragma unroll
            for (int k = B0; k < B1; ++k) {
                const int kk = (B_INS % NW == 0 || wave + k * NW < B_INS) ? k : k - 1;
                dma16<b_cache_policy<LAYOUT>()>(b_t + (int64_t)kk * 8 * NW * K + b_lane,
                      (LDS_AS void*)(st + B_OFF + (wave + kk * NW) * 1024));
            }
        } else {
#pragma unroll
            for (int k = B0; k < B1; ++k) {
                const int ins = (B_INS % NW == 0 || wave + k * NW < B_INS) ? wave + k * NW : B_INS - 1;
                const int row = 8 * ins + cp_row;
                const int grow = min(tl.n0 + row, p.n - 1);
                const uint32_t off = (uint32_t)grow * (uint32_t)K + (uint32_t)((cp_slot ^ b_key(row)) << 4);
                dma16<b_cache_policy<LAYOUT>()>(b_base + off, (LDS_AS void*)(st + B_OFF + ins * 1024));
            }
        }
        // scale words: one per K group (FP32), or one per four K groups (packed E8M0)
        const int sgrps = E8 ? (kchunks + 3) / 4 : kchunks;
        const int sgrp = E8 ? c / 4 : c;
        if constexpr (!SCALES) {
        } else if (wave == NW - 1) {
            // the chunk's block_m A scales (MN-major: contiguous)
            const uint8_t* sa_base = (const uint8_t*)(p.sfa +
                (LAYOUT == kMasked ? (int64_t)tl.g * sgrps * p.sfa_ld : (int64_t)0) +
                (int64_t)sgrp * p.sfa_ld);
            int r4 = tl.m0 + 4 * lane;                // rows past the scale array are unused
            if (r4 >= p.sfa_ld) r4 = 0;
            if (4 * lane < BM) dma16(sa_base + (uint32_t)r4 * 4u, (LDS_AS void*)(st + SA_OFF));
        } else if constexpr (KG) {
            // the tile's block_n per-column B scales of chunk c (MN-major SFB, contiguous);
            // wavefront NW-2 copies them, the others repeat its first 16 bytes so that
            // every wavefront issues one copy per chunk
            const uint8_t* sb_row = (const uint8_t*)(p.sfb + (int64_t)(E8 ? c / 4 : c) * p.sfb_ld);
            int c4 = tl.n0 + 4 * lane;                // columns past the scale row are unused
            if (c4 >= p.sfb_ld) c4 = 0;
            const bool mine = wave == NW - 2 ? 4 * lane < BN : lane == 0;
            if (wave != NW - 2) c4 = tl.n0 < p.sfb_ld ? tl.n0 : 0;
            if (mine) dma16(sb_row + (uint32_t)c4 * 4u, (LDS_AS void*)(st + SB_OFF));
        } else {
            // the B-scale values of the column blocks the tile touches (every other
            // wavefront writes the same bytes)
            const uint8_t* sb_base = (const uint8_t*)(p.sfb + (int64_t)tl.g * nsb * sgrps + sgrp);
            const uint32_t sb_off = (uint32_t)min(tl.n0 / 128 + lane, nsb - 1) * (uint32_t)sgrps * 4u;
            if (lane < SB_SPAN)
                __builtin_amdgcn_global_load_lds((const GLOBAL_AS void*)(sb_base + sb_off),
                                                 (LDS_AS void*)(st + SB_OFF), 4, 0, 0);
        }
    };
    auto issue = [&](const Tile& tl, int c, int s) {
        issue_parts(tl, c, s, std::integral_constant<int, 0>{}, std::integral_constant<int, OPC>{});
    };

    // ---- LDS fragment and scale readers (stage base `st`) ----
    // MN-major fragment of the 16-row block whose logical unit is u: four transpose reads,
    // read r giving the lane's K bytes 32*kq + 8*r .. +7 (the K-major reads' assignment)
    auto load_tr = [&](const uint8_t* st, int base, int key, int u, auto w_const) {
        constexpr int W = decltype(w_const)::value;
        const uint8_t* q = st + base + ((u ^ key) << 4);
        const i32x2_t r0 = lds_read_tr8(q), r1 = lds_read_tr8(q + 8 * W);
        const i32x2_t r2 = lds_read_tr8(q + 16 * W), r3 = lds_read_tr8(q + 24 * W);
        return i32x8{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
    };
    auto load_a = [&](const uint8_t* st, int i) {
        if constexpr (AMN) {
            return load_tr(st, a_tr, a_tr_key, wm * TM + i, std::integral_constant<int, BM>{});
        } else {
            const int* base = (i & 1) ? a_odd : a_even;
            const i32x4 lo = *(const i32x4*)(st + base[0] + 128 * i);
            const i32x4 hi = *(const i32x4*)(st + base[1] + 128 * i);
            return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
    };
    auto load_b = [&](const uint8_t* st, int j) {
        if constexpr (BMN) {
            return load_tr(st, b_tr, b_tr_key, wn * TN + j, std::integral_constant<int, BN>{});
        } else {
            const i32x4 lo = *(const i32x4*)(st + b_base[0] + 2048 * j);
            const i32x4 hi = *(const i32x4*)(st + b_base[1] + 2048 * j);
            return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
    };
    // The operand with fewer 16-row blocks stays in registers for the whole chunk; the
    // other is streamed block by block (double buffered).
    constexpr bool STREAM_A = TM >= TN;
    constexpr int NO = STREAM_A ? TM : TN;             // streamed blocks
    // Copies of a chunk issued in SPREAD shares rather than all at the top of the chunk,
    // so that their LDS writes do not all compete with the fragment reads at once.  Two
    // shares measured 2-4% faster for the 256-row tiles and 2-4% slower for 128 x 448
    // (MI355X, dense M = 4096 prefill shapes).
    constexpr int SPREAD = (BM >= 256 && NO >= 2) ? 2 : 1;
    constexpr int NI = STREAM_A ? TN : TM;             // resident blocks
    struct ChunkRegs {
        i32x8 res[NI];
        i32x8 first;
    };
    struct ScaleRegs {
        float sa[TM];
        float sb[UNIFORM_SB ? 1 : TN];
        f32x4 sbv[KG ? TN : 1];                       // K-grouped: the lane's four columns
        int sbw[KG && E8 ? TN : 1];                   // K-grouped UE8M0: the lane's B row's word
    };
    auto load_scales = [&](const uint8_t* st, const Tile& tl, ScaleRegs& r) {
        const float* sap = (const float*)(st + sa_rd);
        if constexpr (AMN) {
#pragma unroll
            for (int i = 0; i < TM; ++i) r.sa[i] = sap[16 * i];
        } else {
#pragma unroll
            for (int i = 0; i < TM; ++i) r.sa[i] = sap[i];
        }
        if constexpr (KG && E8) {
            // the exponent word of the B row this lane feeds to the matrix core (column
            // wn*WTN + 16j + lj), not of its output columns
#pragma unroll
            for (int j = 0; j < TN; ++j)
                r.sbw[j] = *(const int*)(st + SB_OFF + (wn * WTN + 16 * j + lj) * 4);
            return;
        } else if constexpr (KG) {
#pragma unroll
            for (int j = 0; j < TN; ++j)
                r.sbv[j] = *(const f32x4*)(st + SB_OFF + (wn * WTN + 16 * j + 4 * kq) * 4);
            return;
        }
        if (TM > 1 && !AMN) {
#pragma unroll
            for (int i = 0; i < TM; i += 2) {             // this lane's rows are i ^ flip
                const float x = r.sa[i], y = r.sa[i + 1];
                r.sa[i] = flip ? y : x;
                r.sa[i + 1] = flip ? x : y;
            }
        }
        const float* sbl = (const float*)(st + SB_OFF);
        const int blk0 = tl.n0 / 128;
        if (UNIFORM_SB) {
            r.sb[0] = sbl[min(tl.n0 + wn * WTN, p.n - 1) / 128 - blk0];
        } else {
#pragma unroll
            for (int j = 0; j < TN; ++j)
                r.sb[j] = sbl[min(tl.n0 + wn * WTN + 16 * j, p.n - 1) / 128 - blk0];
        }
    };

    // K-grouped units with no chunk (an empty group, or an empty split of a short one)
    // store their all-zero result -- D = C, or zeros -- when the compute cursor meets them.
    auto on_empty = [&](const Unit& w) {
        if constexpr (KG) {
            f32x4 z[TM][TN];
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) z[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (p.splits == 1) {
                store_tile<TM, TN, WTM, WTN, LAYOUT, AMN>(p, w.tl, z, wm, wn, lj, kq, flip);
            } else {
                f32x4* ws = (f32x4*)(p.ws + ((int64_t)w.t * p.splits + w.s) * (BM * BN));
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j) ws[partial_index<TM, TN>(wave, i, j, lane)] = z[i][j];
            }
        }
    };

    // ---- contiguous layout, 256-row tiles: the dense (m-block, pass) work list ----
    constexpr bool PASSES = LAYOUT == kContiguous && BM > 128;
    PassList plist{-1, 0, 0};
    if constexpr (PASSES) plist = pass_list_build<BM>(p, lane);
    const PassList* pl = PASSES ? &plist : nullptr;

    // ---- the two cursors over this workgroup's (unit, chunk) stream ----
    Unit cur;                                          // the chunk being multiplied
    if (!next_unit<BM, BN, LAYOUT>(p, logical_block_id(), cur, on_empty, pl)) return;
    Unit isu = cur;                                    // the next chunk to copy
    int ic = cur.c0;
    bool live = true;                                  // false: stream exhausted, repeat last
    auto advance_issue = [&]() {
        if (!live) return;
        if (++ic < isu.c1) return;
        Unit nx;
        if (next_unit<BM, BN, LAYOUT>(p, isu.u + gridDim.x, nx, NoEmptyUnits{}, pl)) {
            isu = nx;
            ic = nx.c0;
        } else {
            live = false;                              // keep copying the last chunk (harmless)
            ic = isu.c1 - 1;
        }
    };

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // prologue: chunks 0 .. NS-2 of the stream into stages 0 .. NS-2
#pragma unroll
    for (int q = 0; q < NS - 1; ++q) {
        issue(isu.tl, ic, q);
        advance_issue();
    }
    wait_loads<(NS - 2) * OPC>();
    block_barrier();                                   // chunk 0 is in stage 0
    ChunkRegs cr;
#pragma unroll
    for (int q = 0; q < NI; ++q) cr.res[q] = STREAM_A ? load_b(smem, q) : load_a(smem, q);
    cr.first = STREAM_A ? load_a(smem, 0) : load_b(smem, 0);

    int c = cur.c0;
    int sq = 0;                                        // stage of the chunk being multiplied
    int si = NS - 1;                                   // stage the next copy goes to
    for (;;) {
        // Invariant: chunk c of unit `cur` is in stage sq with its resident fragments and
        // first streamed fragment loaded (or in flight) in `cr`; every wavefront has
        // finished reading stage si, the one chunk c+NS-1 of the stream goes to.
        // The copies of chunk c+NS-1 of the stream go out in SPREAD shares: the first now,
        // share b after the first product of streamed block b-1.
        const Tile itl = isu.tl;
        const int icc = ic;
        issue_parts(itl, icc, si, std::integral_constant<int, 0>{},
                    std::integral_constant<int, OPC / SPREAD>{});
        advance_issue();

        const uint8_t* st = smem + sq * STAGE;
        float sc[TM][UNIFORM_SB ? 1 : TN];
        // E8M0 exponents; a B exponent per column block unless one serves the whole
        // wavefront (K-grouped: one per lane and block)
        constexpr bool SB_PER_J = KG || !UNIFORM_SB;
        int sae[E8 ? TM : 1], sbe[E8 ? (SB_PER_J ? TN : 1) : 1];
        float kg_sa[KG ? TM : 1];
        f32x4 kg_sb[KG ? TN : 1];
        {
            ScaleRegs sr;
            load_scales(st, cur.tl, sr);
            if constexpr (KG && E8) {
                const int sh = 8 * (c & 3);
#pragma unroll
                for (int i = 0; i < TM; ++i) sae[i] = (__builtin_bit_cast(int, sr.sa[i]) >> sh) & 0xFF;
#pragma unroll
                for (int j = 0; j < TN; ++j) sbe[j] = (sr.sbw[j] >> sh) & 0xFF;
            } else if constexpr (KG) {
#pragma unroll
                for (int i = 0; i < TM; ++i) kg_sa[i] = sr.sa[i];
#pragma unroll
                for (int j = 0; j < TN; ++j) kg_sb[j] = sr.sbv[j];
            } else if constexpr (E8) {
                const int sh = 8 * (c & 3);             // this chunk's byte of the packed word
#pragma unroll
                for (int i = 0; i < TM; ++i) sae[i] = (__builtin_bit_cast(int, sr.sa[i]) >> sh) & 0xFF;
#pragma unroll
                for (int j = 0; j < (UNIFORM_SB ? 1 : TN); ++j)
                    sbe[j] = (__builtin_bit_cast(int, sr.sb[j]) >> sh) & 0xFF;
            } else {
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < (UNIFORM_SB ? 1 : TN); ++j) sc[i][j] = sr.sa[i] * sr.sb[j];
            }
        }
        auto promote = [&](int o, int q, const f32x4& part) {
            const int i = STREAM_A ? o : q, j = STREAM_A ? q : o;
            if constexpr (KG && !E8)
                acc[i][j] += (part * kg_sa[i]) * kg_sb[j];  // row scale, then per column
            else
                acc[i][j] += part * sc[i][UNIFORM_SB ? 0 : j];
        };
        // Products are issued in the order (o, q), o = streamed block, q = resident block;
        // the result of product k is promoted after product k+LAG has issued, so its
        // latency is covered and only LAG+1 partials are live.
        constexpr int LAG = 2;
        f32x4 ring[LAG + 1];
        auto step = [&](int o, int q, const i32x8& fr, const i32x8* res) {
            const int k = o * NI + q;
            if constexpr (E8) {
                const int i = STREAM_A ? o : q, j = STREAM_A ? q : o;
                __builtin_amdgcn_s_setprio(1);
                // first operand B rows (scale: their 128x128 block), second A rows (row scale)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    STREAM_A ? res[q] : fr, STREAM_A ? fr : res[q], acc[i][j], 0, 0,
                    0, sbe[SB_PER_J ? j : 0], 0, sae[i]);
                __builtin_amdgcn_s_setprio(0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            } else {
                __builtin_amdgcn_s_setprio(1);         // favour the wave that feeds the MFMA pipe
                ring[k % (LAG + 1)] = STREAM_A ? mfma_e4m3(res[q], fr) : mfma_e4m3(fr, res[q]);
                __builtin_amdgcn_s_setprio(0);
                if (k >= LAG) promote((k - LAG) / NI, (k - LAG) % NI, ring[(k - LAG) % (LAG + 1)]);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // the MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // the promotion it covers
            }
        };

        // ---- streamed blocks 0 .. NO-2 ----
        // The next block's fragment is read after this block's first product has issued:
        // while copies are in flight the compiler can only wait for LDS reads with a zero
        // count (a direct-to-LDS copy counts against the same counter on this hardware), so
        // reads issued ahead of that product's wait would be waited for there as well.
        i32x8 fr = cr.first;
        static_for<0, NO - 1>([&](auto o_const) {
            constexpr int o = decltype(o_const)::value;
            step(o, 0, fr, cr.res);
            const i32x8 next_fr = STREAM_A ? load_a(st, o + 1) : load_b(st, o + 1);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);       // next fragment reads
            if constexpr (o + 1 < SPREAD)
                issue_parts(itl, icc, si, std::integral_constant<int, (o + 1) * OPC / SPREAD>{},
                            std::integral_constant<int, (o + 2) * OPC / SPREAD>{});
#pragma unroll
            for (int q = 1; q < NI; ++q) step(o, q, fr, cr.res);
            fr = next_fr;
        });

        // ---- last block: every read of stage sq has been issued.  Wait for them and for
        // this wavefront's copies of the next chunk, meet the other wavefronts, then start
        // reading the next chunk while the last products of this chunk issue.  (Branch
        // free: after the last chunk the barrier and the reads are harmless, and one basic
        // block lets the scheduler interleave the whole chunk.) ----
        wait_loads<(NS - 2) * OPC>();
        block_barrier();
        const int sn = sq + 1 == NS ? 0 : sq + 1;
        ChunkRegs nr;
        {
            const uint8_t* nst = smem + sn * STAGE;
#pragma unroll
            for (int q = 0; q < NI; ++q) {
                step(NO - 1, q, fr, cr.res);   // frees resident fragment q ...
                nr.res[q] = STREAM_A ? load_b(nst, q) : load_a(nst, q);   // ... for this
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            nr.first = STREAM_A ? load_a(nst, 0) : load_b(nst, 0);
            if constexpr (!E8) {
#pragma unroll
                for (int k = NO * NI - LAG; k < NO * NI; ++k)
                    if (k >= 0) promote(k / NI, k % NI, ring[k % (LAG + 1)]);
            }
        }

        if (c + 1 == cur.c1) {
            // ---- end of the unit: BF16 to D, or the FP32 partial to the workspace ----
            // lane-derived offsets are recomputed here from an opaque copy of the lane id, so
            // that the compiler cannot hoist one register per store out of the main loop
            int el = lane;
            asm volatile("" : "+v"(el));
            if (p.splits == 1) {
                const int elj = el & 15;
                store_tile<TM, TN, WTM, WTN, LAYOUT, AMN>(p, cur.tl, acc, wm, wn, elj, el >> 4,
                                                          (TM > 1 && !AMN) ? (elj >> 3) : 0);
            } else {
                f32x4* ws = (f32x4*)(p.ws + ((int64_t)cur.t * p.splits + cur.s) * (BM * BN));
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j) ws[partial_index<TM, TN>(wave, i, j, el)] = acc[i][j];
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (!next_unit<BM, BN, LAYOUT>(p, cur.u + gridDim.x, cur, on_empty, pl)) break;
            c = cur.c0;
        } else {
            ++c;
        }
        sq = sn;
        si = si + 1 == NS ? 0 : si + 1;
        cr = nr;
    }
    // Copies issued past the end of the stream (repeats of the last chunk) may still be in
    // flight; the workgroup's LDS must not be released under them.
    wait_loads<0>();
}

// B-streaming kernel for few-row (decode) shapes.  Each workgroup computes one work
// unit -- K split s of one block_m x block_n tile -- with its NW wavefronts side by side
// along N: wavefront w owns columns n0 + w*WTN .. +WTN-1 and all block_m rows.
//
//   * B fragments are loaded from global memory straight into registers: every B byte
//     is used by exactly one wavefront, so staging it in LDS buys nothing, and vector
//     loads stream from HBM at a higher per-CU rate than direct-to-LDS copies.  Lane
//     (j = l%16, quarter q = l/16) of the instruction's first operand takes 16-byte
//     units q and q+4 of its B row's 128-byte chunk, so one load instruction covers 16
//     rows x 64 contiguous bytes.  Loads run NS-1 chunks ahead, into a ring of NS
//     register sets (the chunk loop is unrolled NS times so that ring slots are static).
//   * The A tile, its scales and the B-scale values of each chunk go through an LDS ring
//     of NS stages by direct-to-LDS copies, as in fp8bs_gemm_kernel; A fragments are
//     read with the same K-unit assignment (q, q+4) as the B fragments, which keeps the
//     chunk's dot products whole.
//   * Products, promotion, epilogue and split-K partials are those of fp8bs_gemm_kernel
//     with waves_m = 1, so fp8bs_splitk_reduce<BM, BN, 1, NW, LAYOUT> finishes a split.
template <int BM, int BN, int NW, int NS, int LAYOUT>
__global__ void __launch_bounds__(64 * NW) fp8bs_stream_kernel(GemmParams p) {
    constexpr int WTN = BN / NW;                      // columns per wavefront
    constexpr int TM = BM / 16, TN = WTN / 16;
    static_assert(BM % 16 == 0 && WTN % 16 == 0 && NW >= 2, "tile shape");
    static_assert(TM == 1 || TM == 2 || TM == 4 || TM == 8, "row blocks per wavefront");
    // stage: A tile, A scales (64 rows per copy instruction), 256 bytes of B scales
    constexpr int SA_OFF = BM * 128, SB_OFF = SA_OFF + stream_sa_bytes(BM);
    constexpr int STAGE = stream_stage_bytes(BM);
    constexpr int SA_COPIES = (BM + 63) / 64;         // wavefronts NW-1, NW-2 .. copy A scales
    static_assert(STAGE == SB_OFF + 256 && SA_COPIES < NW, "stage layout");
    static_assert(NS >= 2 && NS * STAGE <= kLdsBytesPerCu, "LDS ring");
    constexpr int A_INS = BM / 8;                     // 1 KB (8 rows) per wavefront copy
    constexpr int A_PER = (A_INS + NW - 1) / NW;
    static_assert(BN / 128 + 2 <= 64, "B-scale blocks per tile");
    constexpr int PD = NS - 1;                        // chunks in flight ahead
    // per chunk and wavefront: 2 B loads per column block, A copies, one scale copy
    constexpr int OPC = 2 * TN + A_PER + 1;
    static_assert((PD - 1) * OPC <= 63, "vmcnt range");
    constexpr bool UNIFORM_SB = (128 % WTN == 0) && (BN % 128 == 0 || 128 % BN == 0);

    // One LDS array per ring stage.  The compiler places its own waits before LDS reads
    // by which LDS variable they touch: with a single ring array, every read of chunk c
    // would wait for the copies of chunks c+1 .. c+NS-1 too (all in flight), which takes
    // the ring's depth away.  Stage indices are compile-time constants after unrolling.
    static_assert(NS <= 10, "ring stages");
    constexpr int S2 = NS > 2 ? STAGE : 1, S3 = NS > 3 ? STAGE : 1, S4 = NS > 4 ? STAGE : 1;
    constexpr int S5 = NS > 5 ? STAGE : 1, S6 = NS > 6 ? STAGE : 1, S7 = NS > 7 ? STAGE : 1;
    constexpr int S8 = NS > 8 ? STAGE : 1, S9 = NS > 9 ? STAGE : 1;
    __shared__ __attribute__((aligned(256))) uint8_t ring0[STAGE], ring1[STAGE], ring2[S2],
        ring3[S3], ring4[S4], ring5[S5], ring6[S6], ring7[S7], ring8[S8], ring9[S9];
    auto stage_at = [&](int s) -> uint8_t* {
        switch (s) {
            case 0: return ring0;
            case 1: return ring1;
            case 2: return ring2;
            case 3: return ring3;
            case 4: return ring4;
            case 5: return ring5;
            case 6: return ring6;
            case 7: return ring7;
            case 8: return ring8;
            default: return ring9;
        }
    };

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int kchunks = p.k / 128;
    const int K = p.k;
    const int nsb = (p.n + 127) / 128;

    Unit w;
    // one unit per workgroup (the grid has one workgroup per unit): a tile without valid
    // rows has nothing to do
    if (!next_unit<BM, BN, LAYOUT>(p, logical_block_id(), w)) return;
    const Tile tl = w.tl;
    const int nch = w.c1 - w.c0;

    // ---- A fragment addresses (as fp8bs_gemm_kernel with wm = 0; K units q and q+4) ----
    const int lj = lane & 15;
    const int kq = lane >> 4;
    const int flip = (TM > 1) ? (lj >> 3) : 0;
    int a_even[2], a_odd[2];
    {
        const int row0 = TM * lj;
        const int key = a_key<TM>(row0);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int base = row0 * 128 + (((kq + 4 * h) ^ key) << 4);
            a_even[h] = base + flip * 128;
            a_odd[h] = base - flip * 128;
        }
    }
    const int sa_rd = SA_OFF + TM * lj * 4;

    // ---- B fragment sources: row n0 + wave*WTN + 16j + lj (clamped into the matrix) ----
    const uint8_t* b_lane = p.b + (int64_t)tl.g * p.n * K + 16 * kq;
    uint32_t b_row_off[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int row = min(tl.n0 + wave * WTN + 16 * j + lj, p.n - 1);
        b_row_off[j] = (uint32_t)row * (uint32_t)K;
    }
    auto issue_b = [&](int c, i32x8 (&dst)[TN]) {
        const uint8_t* bc = b_lane + (int64_t)c * 128;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            // non-temporal: a tile's B rows are read by the few m-blocks of a decode shape
            // only (one when block_m covers M); measured on MI355X with the weights cold,
            // 2-18% faster than normal loads on the decode sweep, never slower than 3%
            const i32x4 lo = __builtin_nontemporal_load((const i32x4*)(bc + b_row_off[j]));
            const i32x4 hi = __builtin_nontemporal_load((const i32x4*)(bc + b_row_off[j] + 64));
            dst[j] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
    };

    // ---- A / scale copies of chunk c into stage s ----
    const int cp_row = lane >> 3, cp_slot = lane & 7;
    auto issue_a = [&](int c, int s) {
        uint8_t* st = stage_at(s);
        const uint8_t* a_base = p.a + (LAYOUT == kMasked ? (int64_t)tl.g * p.m * K : (int64_t)0) +
                                (int64_t)c * 128;
#pragma unroll
        for (int k = 0; k < A_PER; ++k) {
            const int ins = min(wave + k * NW, A_INS - 1);   // extra copies repeat the last one
            const int row = 8 * ins + cp_row;
            const int grow = min(tl.m0 + row, tl.row_limit - 1);
            const uint32_t off = (uint32_t)grow * (uint32_t)K + (uint32_t)((cp_slot ^ a_key<TM>(row)) << 4);
            dma16(a_base + off, (LDS_AS void*)(st + ins * 1024));
        }
        // One 4-byte copy per lane and no lane masking, so that every wavefront issues the
        // same number of memory operations per chunk on every path (the compiler counts
        // them to place its waits for the B registers).  Lanes past the tile's rows or
        // scale blocks copy a clamped in-range value into an unused LDS word.
        // A scales (wavefronts NW-1, NW-2, ..) or B scales (the others), chosen without a
        // branch: a data-dependent branch around a copy would hide the copy count from the
        // compiler's wait placement.
        const int part = NW - 1 - wave;                // A-scale rows 64*part .. 64*part+63
        const bool is_sa = part < SA_COPIES;
        const uint8_t* sa_c = (const uint8_t*)(p.sfa +
            (LAYOUT == kMasked ? (int64_t)tl.g * kchunks * p.sfa_ld : (int64_t)0) +
            (int64_t)c * p.sfa_ld);
        const uint8_t* sb_c = (const uint8_t*)(p.sfb + (int64_t)tl.g * nsb * kchunks + c);
        const uint32_t sa_off = (uint32_t)min(tl.m0 + 64 * part + lane, p.sfa_ld - 1) * 4u;
        const uint32_t sb_off = (uint32_t)min(tl.n0 / 128 + lane, nsb - 1) * (uint32_t)kchunks * 4u;
        const uint8_t* src = is_sa ? sa_c + sa_off : sb_c + sb_off;
        uint8_t* dst = st + (is_sa ? SA_OFF + 256 * part : SB_OFF);
        __builtin_amdgcn_global_load_lds((const GLOBAL_AS void*)src, (LDS_AS void*)dst, 4, 0, 0);
    };

    auto load_a = [&](const uint8_t* st, int i) {
        const int* base = (i & 1) ? a_odd : a_even;
        const i32x4 lo = *(const i32x4*)(st + base[0] + 128 * i);
        const i32x4 hi = *(const i32x4*)(st + base[1] + 128 * i);
        return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // multiply chunk in stage / ring slot `slot`
    auto compute = [&](int slot, const i32x8 (&bf)[TN]) {
        const uint8_t* st = stage_at(slot);
        float sa[TM];
        {
            const float* sap = (const float*)(st + sa_rd);
#pragma unroll
            for (int i = 0; i < TM; ++i) sa[i] = sap[i];
            if (TM > 1) {
#pragma unroll
                for (int i = 0; i < TM; i += 2) {
                    const float x = sa[i], y = sa[i + 1];
                    sa[i] = flip ? y : x;
                    sa[i + 1] = flip ? x : y;
                }
            }
        }
        float sb[UNIFORM_SB ? 1 : TN];
        {
            const float* sbl = (const float*)(st + SB_OFF);
            const int blk0 = tl.n0 / 128;
            if (UNIFORM_SB) {
                sb[0] = sbl[min(tl.n0 + wave * WTN, p.n - 1) / 128 - blk0];
            } else {
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    sb[j] = sbl[min(tl.n0 + wave * WTN + 16 * j, p.n - 1) / 128 - blk0];
            }
        }
        // products in the order (i, j); the result of product k is promoted after product
        // k+LAG has issued, so only LAG+1 partials are live
        constexpr int LAG = 2;
        f32x4 ring[LAG + 1];
        auto promote = [&](int k) {
            const int i = k / TN, j = k % TN;
            acc[i][j] += ring[k % (LAG + 1)] * (sa[i] * sb[UNIFORM_SB ? 0 : j]);
        };
        i32x8 fa = load_a(st, 0);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            i32x8 fn;
            if (i + 1 < TM) fn = load_a(st, i + 1);
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int k = i * TN + j;
                __builtin_amdgcn_s_setprio(1);
                ring[k % (LAG + 1)] = mfma_e4m3(bf[j], fa);
                __builtin_amdgcn_s_setprio(0);
                if (k >= LAG) promote(k - LAG);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // the MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // the promotion it covers
            }
            if (i + 1 < TM) fa = fn;
        }
#pragma unroll
        for (int k = TM * TN - LAG; k < TM * TN; ++k)
            if (k >= 0) promote(k);
        // Pin the promoted accumulators here: otherwise the compiler defers the promotions
        // of a whole unrolled group of chunks and holds all their partials live at once.
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) asm volatile("" : "+v"(acc[i][j]));
    };

    i32x8 breg[NS][TN];
    // prologue: chunks 0 .. PD-1 (the last one repeated when the unit is shorter)
#pragma unroll
    for (int q = 0; q < PD; ++q) {
        const int cq = w.c0 + min(q, nch - 1);
        issue_a(cq, q);
        issue_b(cq, breg[q]);
    }
    // Main loop over whole groups of NS chunks: straight-line code with the same memory
    // operations on every path, so that the compiler's own waits for the B registers
    // count exactly.  Chunk q sits in stage / register slot q % NS.
    const int nfull = nch - nch % NS;
    for (int base = 0; base < nfull; base += NS) {
#pragma unroll
        for (int ph = 0; ph < NS; ++ph) {
            // chunk base+ph has landed for this wavefront; after the barrier, for every
            // wavefront, and every wavefront is done with stage (ph + PD) % NS, which the
            // chunk PD ahead reuses
            wait_loads<(PD - 1) * OPC>();
            block_barrier();
            const int qi = min(base + ph + PD, nch - 1);
            issue_a(w.c0 + qi, (ph + PD) % NS);
            issue_b(w.c0 + qi, breg[(ph + PD) % NS]);
            compute(ph, breg[ph]);
        }
    }
    // Tail: the last nch % NS chunks are already in flight; nothing more is issued.
    const int rest = nch - nfull;
    static_for<0, NS - 1>([&](auto I) {
        constexpr int ph = decltype(I)::value;
        if (ph < rest) {
            wait_loads<(PD - 1 - ph) * OPC>();
            block_barrier();
            compute(ph, breg[ph]);
        }
    });
    wait_loads<0>();                                   // no copy may land after the exit

    int el = lane;
    asm volatile("" : "+v"(el));
    if (p.splits == 1) {
        const int elj = el & 15;
        store_tile<TM, TN, BM, WTN, LAYOUT>(p, tl, acc, 0, wave, elj, el >> 4,
                                            (TM > 1) ? (elj >> 3) : 0);
    } else {
        f32x4* ws = (f32x4*)(p.ws + ((int64_t)w.t * p.splits + w.s) * (BM * BN));
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) ws[partial_index<TM, TN>(wave, i, j, el)] = acc[i][j];
    }
}

// Split-K reduction, one thread per four outputs of a partial tile (every workgroup of
// 256 threads covers 1024 outputs of one tile, so the whole reduction runs on
// tiles * BM*BN/1024 workgroups): the FP32 partials of the tile's K splits are added in
// split order 0, 1, ..., S-1 (the same order whatever order the splits finished in, so
// results are reproducible), then written -- BF16, or FP32 for the K-grouped layout, with
// C added when given -- at valid rows and columns.  Partial element e of a tile is
// accumulator (i, j) of lane `lane` of wavefront `wave` in the GEMM kernel,
// e = ((wave * TM + i) * TN + j) * 64 + lane (partial_index), which fixes its row and
// columns exactly as store_tile does.
constexpr int kReduceThreads = 256;

template <int BM, int BN>
constexpr int reduce_groups_per_tile() {
    return (BM * BN / 4 + kReduceThreads - 1) / kReduceThreads;
}

template <int BM, int BN, int WM, int WN, int LAYOUT, bool AMN = false>
__global__ void __launch_bounds__(kReduceThreads) fp8bs_splitk_reduce(GemmParams p) {
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 16, TN = WTN / 16;
    constexpr int V = BM * BN / 4;                    // f32x4 per partial tile
    constexpr int PER_TILE = reduce_groups_per_tile<BM, BN>();
    const int t = blockIdx.x / PER_TILE;
    const int e = (blockIdx.x - t * PER_TILE) * kReduceThreads + threadIdx.x;
    if (t >= p.tiles || e >= V) return;
    Tile tl;
    if (!tile_at<BM, BN, LAYOUT>(p, t, tl)) return;
    const f32x4* ws = (const f32x4*)(p.ws + (int64_t)t * p.splits * (BM * BN)) + e;
    f32x4 acc = ws[0];
    for (int s = 1; s < p.splits; ++s) acc += ws[(int64_t)s * V];

    const int lane = e & 63, rest = e >> 6;
    const int j = rest % TN, i = (rest / TN) % TM, wave = rest / (TM * TN);
    const int wm = wave / WN, wn = wave % WN, lj = lane & 15, kq = lane >> 4;
    const int flip = (TM > 1 && !AMN) ? (lj >> 3) : 0;
    const int row = tl.m0 + wm * WTM + (AMN ? 16 * i + lj : TM * lj + (i ^ flip));
    const int col = tl.n0 + wn * WTN + 16 * j + 4 * kq;
    if (row >= tl.row_limit) return;
    if (LAYOUT == kContiguous && p.grouped_layout[row] != tl.g) return;
    const int64_t slot = (LAYOUT == kMasked || LAYOUT == kKGrouped)
                             ? (int64_t)tl.g * p.m * p.n : (int64_t)0;
    const int64_t off = slot + (int64_t)row * p.n + col;
    const bool vec = (p.n & 3) == 0 && col + 3 < p.n;
    if (p.c) {                                        // D = C + A B^T
        if (vec) {
            acc += *(const f32x4*)(p.c + off);
        } else {
#pragma unroll
            for (int v = 0; v < 4; ++v)
                if (col + v < p.n) acc[v] += p.c[off + v];
        }
    }
    if constexpr (LAYOUT == kKGrouped) {
        float* d = (float*)(void*)p.d + off;
        if (vec) {
            *(f32x4*)d = acc;
        } else {
#pragma unroll
            for (int v = 0; v < 4; ++v)
                if (col + v < p.n) d[v] = acc[v];
        }
    } else {
        uint16_t* d = p.d + off;
        if (vec) {
            *(uint2*)d = uint2{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
        } else {
#pragma unroll
            for (int v = 0; v < 4; ++v)
                if (col + v < p.n) d[v] = to_bf16(acc[v]);
        }
    }
}

typedef void (*KernelFn)(GemmParams);

struct InstanceEntry {
    KernelFn fn[3];            // FP32 scales, per layout
    KernelFn fn_e8[3];         // packed UE8M0 scales, per layout (null: not compiled)
    KernelFn reduce[3];
    int threads;
    KernelFn fn_form[4];       // dense, stored forms nt (unused), nn, tn, tt (null: not compiled)
    KernelFn fn_kg;            // K-grouped
    KernelFn reduce_amn;       // dense with an MN-major A (tn, tt)
    KernelFn reduce_kg;
    KernelFn fn_form_e8[4];    // the same with packed UE8M0 scales (null: not compiled)
    KernelFn fn_kg_e8;
    int reduce_groups;         // split-K reduction workgroups per tile
};

template <int KIND, int BM, int BN, int WM, int WN, int NS, int LAYOUT, int SCALE>
constexpr KernelFn gemm_fn() {
    if constexpr (KIND == kStreamB) {
        static_assert(WM == 1, "B-streaming instances have one wavefront along M");
        if constexpr (SCALE == kScaleF32) return fp8bs_stream_kernel<BM, BN, WN, NS, LAYOUT>;
        else return nullptr;
    } else {
        return fp8bs_gemm_kernel<BM, BN, WM, WN, NS, LAYOUT, SCALE>;
    }
}

template <int KIND, int BM, int BN, int WM, int WN, int NS, int LAYOUT, int E8>
constexpr KernelFn e8_fn() {
    if constexpr (E8) return gemm_fn<KIND, BM, BN, WM, WN, NS, LAYOUT, kScaleUE8M0>();
    else return nullptr;
}

// MN-major variants (staged kernel only): LAYOUT kDense with the form's operand majors, or
// kKGrouped; REDUCE picks the matching split-K reduction instead.
template <int KIND, int BM, int BN, int WM, int WN, int NS, int MN, int LAYOUT, bool AMN,
          bool BMN, bool REDUCE = false, int E8 = -1>
constexpr KernelFn mn_fn() {
    // E8 < 0: FP32 scales; 0 / 1: the instance's UE8M0 flag (packed power-of-two scales)
    if constexpr (!MN || KIND != kStaged || E8 == 0) {
        return nullptr;
    } else if constexpr (REDUCE) {
        return fp8bs_splitk_reduce<BM, BN, WM, WN, LAYOUT, AMN>;
    } else {
        return fp8bs_gemm_kernel<BM, BN, WM, WN, NS, LAYOUT, (E8 > 0 ? kScaleUE8M0 : kScaleF32),
                                 AMN, BMN>;
    }
}

#define FP8BS_INSTANCE(KIND, BM, BN, WM, WN, NS, OCC, CNS, TNS, SCNS, STNS, E8, MN, MNE8)  \
    {{gemm_fn<KIND, BM, BN, WM, WN, NS, kDense, kScaleF32>(),                              \
      gemm_fn<KIND, BM, BN, WM, WN, NS, kContiguous, kScaleF32>(),                         \
      gemm_fn<KIND, BM, BN, WM, WN, NS, kMasked, kScaleF32>()},                            \
     {e8_fn<KIND, BM, BN, WM, WN, NS, kDense, E8>(),                                       \
      e8_fn<KIND, BM, BN, WM, WN, NS, kContiguous, E8>(),                                  \
      e8_fn<KIND, BM, BN, WM, WN, NS, kMasked, E8>()},                                     \
     {fp8bs_splitk_reduce<BM, BN, WM, WN, kDense>,                                          \
      fp8bs_splitk_reduce<BM, BN, WM, WN, kContiguous>,                                     \
      fp8bs_splitk_reduce<BM, BN, WM, WN, kMasked>},                                        \
     64 * (WM) * (WN),                                                                      \
     {nullptr,                                                                              \
      mn_fn<KIND, BM, BN, WM, WN, NS, MN, kDense, false, true>(),                           \
      mn_fn<KIND, BM, BN, WM, WN, NS, MN, kDense, true, true>(),                            \
      mn_fn<KIND, BM, BN, WM, WN, NS, MN, kDense, true, false>()},                          \
     mn_fn<KIND, BM, BN, WM, WN, NS, MN, kKGrouped, true, true>(),                          \
     mn_fn<KIND, BM, BN, WM, WN, NS, MN, kDense, true, false, true>(),                      \
     mn_fn<KIND, BM, BN, WM, WN, NS, MN, kKGrouped, true, true, true>(),                    \
     {nullptr,                                                                              \
      mn_fn<KIND, BM, BN, WM, WN, NS, MN, kDense, false, true, false, E8>(),                \
      mn_fn<KIND, BM, BN, WM, WN, NS, MN, kDense, true, true, false, E8>(),                 \
      mn_fn<KIND, BM, BN, WM, WN, NS, MN, kDense, true, false, false, E8>()},               \
     mn_fn<KIND, BM, BN, WM, WN, NS, MN, kKGrouped, true, true, false, E8>(),               \
     reduce_groups_per_tile<BM, BN>()},
const InstanceEntry kEntries[] = {
#include "fp8bs_instances.inc"
};
#undef FP8BS_INSTANCE

}  // namespace

int launch_instance(const Plan& plan, int layout, int scale_mode, const GemmParams& p,
                    hipStream_t stream, int form) {
    if (plan.instance < 0 || plan.instance >= (int)(sizeof(kEntries) / sizeof(kEntries[0])))
        return (int)hipErrorInvalidValue;
    if (layout < kDense || layout > kKGrouped || form < kFormNT || form > kFormTT)
        return (int)hipErrorInvalidValue;
    const InstanceEntry& e = kEntries[plan.instance];
    KernelFn fn, reduce;
    const bool e8 = scale_mode == kScaleUE8M0;
    if (layout == kKGrouped) {
        fn = e8 ? e.fn_kg_e8 : e.fn_kg;
        reduce = e.reduce_kg;
    } else if (form != kFormNT) {
        fn = layout != kDense ? nullptr : e8 ? e.fn_form_e8[form] : e.fn_form[form];
        reduce = form_a_mn(form) ? e.reduce_amn : e.reduce[kDense];
    } else {
        fn = scale_mode == kScaleUE8M0 ? e.fn_e8[layout] : e.fn[layout];
        reduce = e.reduce[layout];
    }
    if (!fn || !reduce) return (int)hipErrorInvalidValue;
    GemmParams args = p;
    void* argv[] = {&args};
    hipError_t err = hipLaunchKernel((const void*)fn, dim3((unsigned)plan.grid),
                                     dim3(e.threads), argv, 0, stream);
    if (err != hipSuccess || p.splits == 1) return (int)err;
    // reduce_groups workgroups per tile (tiles without valid rows return at once)
    return (int)hipLaunchKernel((const void*)reduce,
                                dim3((unsigned)(p.tiles * (int64_t)e.reduce_groups)),
                                dim3(kReduceThreads), argv, 0, stream);
}

}  // namespace fp8bs
