// fp8bs_quant.hip -- the quantisers that produce the GEMM's operands on gfx950:
// FP32 / BF16 activations -> e4m3 with one FP32 scale per (row, 128-column group),
// written straight into the MN-major SFA layout, and weights -> e4m3 with one FP32
// scale per 128x128 block.
//
// The FP8-training recipe the pages describe ("deepseek开源周第三天：DeepGEMM深度分析",
// pxiaoer.blog, list "细粒度量化 / 在线量化": scaling factors computed online per 1x128
// activation block and per 128x128 weight block, values then converted to FP8); the
// pages leave the cast to the caller ("DeepGEMM: kernel FP8 GEMM sạch và hiệu quả nhờ
// scaling chi tiết", section "Giao diện GEMM và ràng buộc layout").  Per block:
//
//   a = max(max |x|, 1e-4); scale = a / 448; inv = 448 / a;
//   q = e4m3(clamp(x * inv, -448, 448))      (nearest value, ties to the even code)
//
// each step one IEEE FP32 operation, so codes and scales are reproducible bit for bit.
// Both kernels are HBM-bound streaming passes: each input byte is read once, each
// output byte written once.
#include <hip/hip_runtime.h>

#include "fp8bs_internal.h"

namespace fp8bs {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// OCP e4m3 code of an FP32 value of magnitude at most 448 (NaN -> the NaN code),
// nearest value with ties to the even code, sign kept.  Subnormal range (below 2^-6):
// the code is the value in units of 2^-9, rounded to the nearest integer (even on
// ties); normal range: keep 3 mantissa bits, rounding the 20 dropped ones to nearest
// even (a carry out of the mantissa bumps the exponent, which is the next code).
__device__ __forceinline__ uint32_t enc_e4m3(float v) {
    const uint32_t bits = __builtin_bit_cast(uint32_t, v);
    const uint32_t sign = (bits >> 24) & 0x80u;
    const float a = __builtin_fabsf(v);
    uint32_t code;
    if (a < 0x1p-6f) {
        code = (uint32_t)__builtin_rintf(a * 512.0f);
    } else {
        const uint32_t ab = bits & 0x7FFFFFFFu;
        const uint32_t exp = (ab >> 23) - 120u;          // 127 (FP32 bias) - 7 (e4m3 bias)
        const uint32_t mant = ab & 0x7FFFFFu;
        uint32_t r = mant >> 20;
        const uint32_t rem = mant & 0xFFFFFu;
        r += (rem > 0x80000u || (rem == 0x80000u && (r & 1u))) ? 1u : 0u;
        code = (exp << 3) + r;
    }
    if (!(a <= 448.0f)) code = 0x7Fu;                     // NaN
    return sign | code;
}

__device__ __forceinline__ float clamp448(float v) {
    // compare-and-select (not min/max) so that NaN stays NaN, as in the definition
    if (v > 448.0f) v = 448.0f;
    if (v < -448.0f) v = -448.0f;
    return v;
}

// scale and inverse of a block with largest magnitude amax
__device__ __forceinline__ float block_scale(float amax, float* inv) {
    const float a = amax < 1e-4f ? 1e-4f : amax;
    *inv = 448.0f / a;
    return a / 448.0f;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) {
    return __builtin_bit_cast(float, h << 16);
}

// 8 consecutive inputs starting at element e of x (FP32 or BF16), widened to FP32
template <bool BF16>
__device__ __forceinline__ void load8(const void* x, int64_t e, float (&v)[8]) {
    if (BF16) {
        const uint4 w = *(const uint4*)((const uint16_t*)x + e);
        const uint32_t h[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = bf16_to_f32(h[i] & 0xFFFFu);
            v[2 * i + 1] = bf16_to_f32(h[i] >> 16);
        }
    } else {
        const f32x4 lo = *(const f32x4*)((const float*)x + e);
        const f32x4 hi = *(const f32x4*)((const float*)x + e + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[i] = lo[i];
            v[4 + i] = hi[i];
        }
    }
}

// Four values to four e4m3 codes with gfx950's conversion instruction (v_cvt_pk_fp8_f32,
// OCP e4m3, round to nearest even).  For every finite input of magnitude at most 448 it
// gives the code enc_e4m3 gives -- checked on MI355X against every code value, every tie
// between neighbouring codes, the values one ulp either side of each tie and two million
// random values -- so the quantisers stay bit-exact with the definition.
__device__ __forceinline__ uint32_t cvt4_e4m3(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

__device__ __forceinline__ uint2 quantise8(const float (&v)[8], float inv) {
    float s[8];
    bool nan = false;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        s[i] = clamp448(v[i] * inv);
        nan |= s[i] != s[i];
    }
    uint2 out;
    if (!nan) {
        out.x = cvt4_e4m3(s[0], s[1], s[2], s[3]);
        out.y = cvt4_e4m3(s[4], s[5], s[6], s[7]);
        return out;
    }
    // a NaN input: the software encoder, which keeps the input's sign on the NaN code
    uint32_t c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = enc_e4m3(s[i]);
    out.x = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
    out.y = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
    return out;
}

__device__ __forceinline__ float absmax8(const float (&v)[8]) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float a = __builtin_fabsf(v[i]);
        m = a > m ? a : m;                                  // NaN never raises the maximum
    }
    return m;
}

// Activations.  Workgroup (4 wavefronts) = 64 rows x one 128-column group of one slot.
// Lane l of a wavefront holds 8 columns (16 lanes per row) of 4 rows at a time; the
// wavefront covers 16 rows in 4 steps, all loads issued before any arithmetic.
template <bool BF16>
__global__ void __launch_bounds__(256) quant_1x128_kernel(const void* __restrict__ x,
                                                          uint8_t* __restrict__ q,
                                                          float* __restrict__ sfa, int rows,
                                                          int k, int sfa_ld, int row_blocks) {
    const int kb = k / 128;
    const int blk = blockIdx.x;
    const int slot = blk / (row_blocks * kb);
    const int rest = blk - slot * row_blocks * kb;
    const int c = rest % kb;                               // column group
    const int rb = rest / kb;                              // 64-row block
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int seg = lane & 15, sub = lane >> 4;
    const int64_t slot_rows = (int64_t)slot * rows;
    float v[4][8];
    int row[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        row[i] = rb * 64 + wave * 16 + 4 * i + sub;
        const int r = row[i] < rows ? row[i] : rows - 1;   // out-of-range rows reread the last
        load8<BF16>(x, (slot_rows + r) * k + 128 * c + 8 * seg, v[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float m = absmax8(v[i]);
#pragma unroll
        for (int w = 8; w >= 1; w >>= 1) {
            const float o = __shfl_xor(m, w, 16);
            m = o > m ? o : m;
        }
        float inv;
        const float s = block_scale(m, &inv);
        if (row[i] < rows) {
            *(uint2*)(q + (slot_rows + row[i]) * k + 128 * c + 8 * seg) = quantise8(v[i], inv);
            if (seg == 0) sfa[((int64_t)slot * kb + c) * sfa_ld + row[i]] = s;
        }
    }
}

// Weights.  Workgroup (4 wavefronts) = one 128x128 block; thread t holds 8 columns
// (8 * (t % 16) ..) of 8 rows (t / 16 + 16 i); rows past N are not part of the block.
template <bool BF16>
__global__ void __launch_bounds__(256) quant_128x128_kernel(const void* __restrict__ x,
                                                            uint8_t* __restrict__ q,
                                                            float* __restrict__ sfb, int n,
                                                            int k) {
    __shared__ float wave_max[4];
    const int kb = k / 128, nb = (n + 127) / 128;
    const int blk = blockIdx.x;
    const int g = blk / (nb * kb);
    const int i_blk = (blk / kb) % nb, c = blk % kb;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int col = 128 * c + 8 * (t & 15);
    float v[8][8];
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = 128 * i_blk + (t >> 4) + 16 * i;
        const int rr = r < n ? r : n - 1;
        load8<BF16>(x, ((int64_t)g * n + rr) * k + col, v[i]);
        if (r < n) {
            const float mi = absmax8(v[i]);
            m = mi > m ? mi : m;
        }
    }
#pragma unroll
    for (int w = 32; w >= 1; w >>= 1) {
        const float o = __shfl_xor(m, w, 64);
        m = o > m ? o : m;
    }
    if (lane == 0) wave_max[wave] = m;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < 4; ++w) m = wave_max[w] > m ? wave_max[w] : m;
    float inv;
    const float s = block_scale(m, &inv);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = 128 * i_blk + (t >> 4) + 16 * i;
        if (r < n) *(uint2*)(q + ((int64_t)g * n + r) * k + col) = quantise8(v[i], inv);
    }
    if (t == 0) sfb[((int64_t)g * nb + i_blk) * kb + c] = s;
}

bool aligned16(const void* p) { return p && ((uintptr_t)p & 15u) == 0; }

}  // namespace
}  // namespace fp8bs

extern "C" int fp8bs_quantize_1x128(const void* x, int x_dtype, void* q, float* sfa, int groups,
                                    int rows, int k, hipStream_t stream) {
    using namespace fp8bs;
    if (k < 128 || k % 128 != 0 || rows < 0 || groups < 1) return FP8BS_ERR_SHAPE;
    if (x_dtype != FP8BS_DTYPE_F32 && x_dtype != FP8BS_DTYPE_BF16) return FP8BS_ERR_UNSUPPORTED;
    if ((double)groups * rows * k >= 9.0e15) return FP8BS_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(q) || !sfa || ((uintptr_t)sfa & 3u)) return FP8BS_ERR_POINTER;
    if (rows == 0) return FP8BS_OK;
    int row_blocks = (rows + 63) / 64;
    const int64_t grid = (int64_t)groups * row_blocks * (k / 128);
    if (grid > 0x7fffffff) return FP8BS_ERR_SHAPE;
    int ld = (int)fp8bs_get_sfa_ld(rows);
    uint8_t* qb = (uint8_t*)q;
    void* args[] = {(void*)&x, (void*)&qb, (void*)&sfa, (void*)&rows, (void*)&k, (void*)&ld,
                    (void*)&row_blocks};
    const void* fn = x_dtype == FP8BS_DTYPE_BF16 ? (const void*)quant_1x128_kernel<true>
                                                 : (const void*)quant_1x128_kernel<false>;
    return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(256), args, 0, stream) == hipSuccess
               ? FP8BS_OK : FP8BS_ERR_HIP;
}

extern "C" int fp8bs_quantize_128x128(const void* x, int x_dtype, void* q, float* sfb, int groups,
                                      int n, int k, hipStream_t stream) {
    using namespace fp8bs;
    if (k < 128 || k % 128 != 0 || n < 1 || groups < 1) return FP8BS_ERR_SHAPE;
    if (x_dtype != FP8BS_DTYPE_F32 && x_dtype != FP8BS_DTYPE_BF16) return FP8BS_ERR_UNSUPPORTED;
    if ((double)groups * n * k >= 9.0e15) return FP8BS_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(q) || !sfb || ((uintptr_t)sfb & 3u)) return FP8BS_ERR_POINTER;
    const int64_t grid = (int64_t)groups * ((n + 127) / 128) * (k / 128);
    if (grid > 0x7fffffff) return FP8BS_ERR_SHAPE;
    uint8_t* qb = (uint8_t*)q;
    void* args[] = {(void*)&x, (void*)&qb, (void*)&sfb, (void*)&n, (void*)&k};
    const void* fn = x_dtype == FP8BS_DTYPE_BF16 ? (const void*)quant_128x128_kernel<true>
                                                 : (const void*)quant_128x128_kernel<false>;
    return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(256), args, 0, stream) == hipSuccess
               ? FP8BS_OK : FP8BS_ERR_HIP;
}
