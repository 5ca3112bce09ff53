/*
 * fp8bs_oracle.c -- plain, slow CPU oracle for the block-scaled FP8 GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header, table or constant
 * generator with the HIP library; the two never include each other.
 *
 * Pages cited (titles as published):
 *   [README-zh]  DeepGEMM README repost, lqnn.cn/news/60274 (Chinese), sections
 *                "DeepGEMM" (library description) and "优化技术".
 *   [hada]       "DeepGEMM: kernel FP8 GEMM sạch và hiệu quả nhờ scaling chi
 *                tiết", vi.news.hada.io/topic?id=19459, sections "Giao diện
 *                GEMM và ràng buộc layout" and "Dense và Grouped GEMM".
 *   [pxiaoer]    "deepseek开源周第三天：DeepGEMM深度分析", pxiaoer.blog, the
 *                FP8-training list ("细粒度量化", "在线量化", "提高累加精度").
 *
 * What is computed (the plain definition, no blocking and no reordering
 * beyond what the definition states):
 *
 *   D[r][n] = bf16_rne( sum_{c=0}^{K/128-1}  P_c(r,n) * (SA[r][c] * SB[g][n/128][c]) )
 *   P_c(r,n) = sum_{k=128c}^{128c+127} dec(A[r][k]) * dec(B[g][n][k])
 *
 * - A is OCP e4m3 with one FP32 scale per row and per 128-wide K group
 *   ("1x128"), B is OCP e4m3 with one FP32 scale per 128x128 block
 *   ([pxiaoer] fine-grained / online quantisation list; [README-zh]
 *   "DeepGEMM" section: fine-grained scaling).
 * - The NT form D = A * B^T, A row-major [M][K], B stored [N][K] ([hada]
 *   "Giao diện GEMM và ràng buộc layout": fp8_gemm_nt computes D = C + A @ B.T,
 *   row-major x col-major).  The C term is taken by fp8bs_oracle_with_addend and
 *   the two functions further down; the other stored forms (nn, tn, tt) and the
 *   K-grouped weight-gradient product are defined next to their functions.
 * - Each 128-K chunk's partial product is scaled and promoted into a wider
 *   accumulator ([README-zh] "DeepGEMM" section, two-level accumulation;
 *   [pxiaoer] "提高累加精度").  Here the wider accumulator is FP64.
 *
 * Exactness: every e4m3 value is an integer multiple of 2^-9 of magnitude at
 * most 448, so each product is an integer multiple of 2^-18 below 2^36 * 2^-18
 * and each 128-term chunk sum stays below 2^43 * 2^-18: P_c is exact in FP64
 * whatever the order of summation.  SA*SB (two 24-bit significands) is exact
 * in FP64 too.  The only roundings are P_c*s_c and acc += ..., both in FP64
 * (compiled with -ffp-contract=off), and the final rounding to BF16, done
 * directly from FP64 with round-to-nearest-even.
 *
 * Layout-specific valid rows (rows that are not valid are never written):
 * - dense:       0 <= r < M, group 0.
 * - contiguous:  rows whose group index layout[r] satisfies 0 <= g < G; rows
 *                with a negative index (padding) or an index >= G are left
 *                untouched ([hada] "Dense và Grouped GEMM": expert segments
 *                concatenated along M, each aligned to the M block size).
 * - masked:      for group g, rows 0 <= r < min(max(masked_m[g], 0), max_m);
 *                the kernel "computes only the valid region" ([hada] "Dense
 *                và Grouped GEMM", masked grouped GEMM).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_API __attribute__((visibility("default")))

/* ---- element codecs ---------------------------------------------------- */

/* OCP e4m3 ("e4m3fn"): 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits,
 * no infinities, S.1111.111 is NaN, largest finite 448, exponent field 0 holds
 * subnormals m * 2^-9. */
ORACLE_API double fp8bs_oracle_dec_e4m3(uint8_t byte) {
    int s = byte >> 7;
    int e = (byte >> 3) & 15;
    int m = byte & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp((double)(8 + m), e - 10);
    return s ? -v : v;
}

/* Round an FP64 value straight to BF16 (8 significant bits, 8 exponent bits,
 * subnormals down to 2^-133) with round-to-nearest, ties to even.  No
 * intermediate FP32 rounding. */
ORACLE_API uint16_t fp8bs_oracle_bf16_rne(double x) {
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    double a = fabs(x);
    int e, q;
    double n, r, v;
    float f;
    uint32_t bits;
    if (isnan(x)) return 0x7FC0u;
    if (isinf(a)) return (uint16_t)(sign | 0x7F80u);
    if (a == 0.0) return sign;
    frexp(a, &e);          /* a = f * 2^e with 0.5 <= f < 1 */
    q = e - 8;             /* weight of the 8th significant bit */
    if (q < -133) q = -133;
    n = ldexp(a, -q);      /* exact: scaling by a power of two */
    r = rint(n);           /* default rounding mode: nearest, ties to even */
    v = ldexp(r, q);
    if (v >= 0x1p128) return (uint16_t)(sign | 0x7F80u);
    f = (float)v;          /* exact: v has at most 8 significant bits */
    memcpy(&bits, &f, sizeof bits);
    return (uint16_t)(sign | ((bits >> 16) & 0x7FFFu));
}

/* ---- the definition ---------------------------------------------------- */

static double dec_table[256];
static int dec_table_ready = 0;

static void init_dec_table(void) {
    int i;
    if (dec_table_ready) return;
    for (i = 0; i < 256; ++i) dec_table[i] = fp8bs_oracle_dec_e4m3((uint8_t)i);
    dec_table_ready = 1;
}

/* One output element before the final rounding.
 *   a:  the K bytes of one row of the product's left operand, a[k * a_step];
 *   sa: its K/128 scales, sa[c * sa_step];
 *   b:  the K bytes of the right operand for one output column n, b[k * b_step];
 *   sb: the K/128 scales that apply to that column, sb[c * sb_step].
 * Chunks are visited in increasing order c = 0, 1, ... */
static double element_acc(const uint8_t* a, ptrdiff_t a_step, const float* sa, ptrdiff_t sa_step,
                          const uint8_t* b, ptrdiff_t b_step, const float* sb, ptrdiff_t sb_step,
                          int64_t K) {
    double acc = 0.0;
    int64_t c, k;
    for (c = 0; c < K / 128; ++c) {
        double p = 0.0, s;
        for (k = 128 * c; k < 128 * c + 128; ++k)
            p += dec_table[a[k * a_step]] * dec_table[b[k * b_step]];
        s = (double)sa[c * sa_step] * (double)sb[c * sb_step];
        acc += p * s;
    }
    return acc;
}

/* Row r of A (logical [rows][K]) against column n of group g's B ([G][N][K]). */
static double dense_element(const uint8_t* A, const float* SA, const uint8_t* B,
                            const float* SB, int64_t r, int64_t g, int64_t n,
                            int64_t N, int64_t K) {
    int64_t kb = K / 128, nb = (N + 127) / 128;
    return element_acc(A + r * K, 1, SA + r * kb, 1,
                       B + (g * N + n) * K, 1, SB + (g * nb + n / 128) * kb, 1, K);
}

static int shape_ok(int64_t N, int64_t K) { return N > 0 && K >= 128 && K % 128 == 0; }

/* Dense: A[M][K], SA[M][K/128] (row-major, logical layout), B[N][K],
 * SB[ceil(N/128)][K/128], D[M][N] as BF16 bit patterns.  Returns 0, or -1 on
 * a shape the definition does not cover (K not a positive multiple of 128). */
ORACLE_API int fp8bs_oracle_dense(const uint8_t* A, const float* SA, const uint8_t* B,
                                  const float* SB, uint16_t* D, int64_t M, int64_t N,
                                  int64_t K) {
    int64_t r;
    if (!shape_ok(N, K) || M < 0) return -1;
    init_dec_table();
#pragma omp parallel for schedule(static)
    for (r = 0; r < M; ++r) {
        int64_t n;
        for (n = 0; n < N; ++n)
            D[r * N + n] = fp8bs_oracle_bf16_rne(dense_element(A, SA, B, SB, r, 0, n, N, K));
    }
    return 0;
}

/* Contiguous grouped: A[M][K], SA[M][K/128], B[G][N][K], SB[G][ceil(N/128)][K/128],
 * layout[M] (group index per row, negative = padding), D[M][N].  Only rows
 * with 0 <= layout[r] < G are written. */
ORACLE_API int fp8bs_oracle_contiguous(const uint8_t* A, const float* SA, const uint8_t* B,
                                       const float* SB, const int32_t* layout, uint16_t* D,
                                       int64_t M, int64_t N, int64_t K, int64_t G) {
    int64_t r;
    if (!shape_ok(N, K) || M < 0 || G <= 0) return -1;
    init_dec_table();
#pragma omp parallel for schedule(static)
    for (r = 0; r < M; ++r) {
        int64_t g = layout[r], n;
        if (g < 0 || g >= G) continue;
        for (n = 0; n < N; ++n)
            D[r * N + n] = fp8bs_oracle_bf16_rne(dense_element(A, SA, B, SB, r, g, n, N, K));
    }
    return 0;
}

/* Masked grouped: A[G][max_m][K], SA[G][max_m][K/128], B[G][N][K],
 * SB[G][ceil(N/128)][K/128], masked_m[G], D[G][max_m][N].  For group g only
 * rows r < min(max(masked_m[g], 0), max_m) are written. */
ORACLE_API int fp8bs_oracle_masked(const uint8_t* A, const float* SA, const uint8_t* B,
                                   const float* SB, const int32_t* masked_m, uint16_t* D,
                                   int64_t G, int64_t max_m, int64_t N, int64_t K) {
    int64_t i;
    if (!shape_ok(N, K) || G <= 0 || max_m < 0) return -1;
    init_dec_table();
#pragma omp parallel for schedule(static)
    for (i = 0; i < G * max_m; ++i) {
        int64_t g = i / max_m, r = i % max_m, n, valid = masked_m[g];
        if (valid < 0) valid = 0;
        if (valid > max_m) valid = max_m;
        if (r >= valid) continue;
        for (n = 0; n < N; ++n)
            D[i * N + n] = fp8bs_oracle_bf16_rne(dense_element(A, SA, B, SB, i, g, n, N, K));
    }
    return 0;
}

/* With an FP32 addend: D = bf16(C + A * B^T), the sum taken in FP64 before the single
 * rounding ([hada] "Giao diện GEMM và ràng buộc layout": fp8_gemm_nt computes
 * D = C + A @ B.T).  C has D's shape and layout ([rows][N], masked [G][max_m][N]); only
 * valid rows of C are read.  layout / masked_m / G select the layout exactly as in the
 * three functions above (kind 0 dense, 1 contiguous, 2 masked). */
ORACLE_API int fp8bs_oracle_with_addend(int kind, const uint8_t* A, const float* SA,
                                        const uint8_t* B, const float* SB, const int32_t* gdata,
                                        const float* C, uint16_t* D, int64_t G, int64_t rows,
                                        int64_t N, int64_t K) {
    int64_t i;
    if (!shape_ok(N, K) || rows < 0 || G <= 0 || kind < 0 || kind > 2) return -1;
    init_dec_table();
#pragma omp parallel for schedule(static)
    for (i = 0; i < (kind == 2 ? G * rows : rows); ++i) {
        int64_t g = 0, n;
        if (kind == 1) {
            g = gdata[i];
            if (!(g >= 0 && g < G)) continue;         /* padding row or unknown group */
        } else if (kind == 2) {
            int64_t valid = gdata[i / rows];
            if (valid < 0) valid = 0;
            if (valid > rows) valid = rows;
            g = i / rows;
            if (i % rows >= valid) continue;
        }
        for (n = 0; n < N; ++n)
            D[i * N + n] = fp8bs_oracle_bf16_rne((double)C[i * N + n] +
                                                 dense_element(A, SA, B, SB, i, g, n, N, K));
    }
    return 0;
}

/* Sampled outputs, for shapes too large to compute whole.  Point p names an
 * A row a_row[p] (an index into the flattened A / SA rows), the group whose B
 * it meets, group[p], and a column col[p].  The caller maps layout-specific
 * coordinates to these (contiguous: group = layout[row]; masked: a_row =
 * g*max_m + r).  Writes the FP64 value before rounding to acc[p] (if acc is
 * not NULL) and its BF16 rounding to d[p]. */
ORACLE_API int fp8bs_oracle_points(const uint8_t* A, const float* SA, const uint8_t* B,
                                   const float* SB, int64_t N, int64_t K, int64_t npts,
                                   const int64_t* a_row, const int64_t* group,
                                   const int64_t* col, double* acc, uint16_t* d) {
    int64_t p;
    if (!shape_ok(N, K) || npts < 0) return -1;
    init_dec_table();
#pragma omp parallel for schedule(static)
    for (p = 0; p < npts; ++p) {
        double v = dense_element(A, SA, B, SB, a_row[p], group[p], col[p], N, K);
        if (acc) acc[p] = v;
        d[p] = fp8bs_oracle_bf16_rne(v);
    }
    return 0;
}

/* ---- operand storage layouts: nt, nn, tn, tt ------------------------------
 *
 * [hada] "Giao diện GEMM và ràng buộc layout": the kernels are named for
 * D = C + A @ B with two letters saying whether A and B enter as stored ("n") or
 * transposed ("t") -- fp8_gemm_nt is D = C + A @ B.T -- and the newer kernels
 * accept all four of nt, tn, nn, tt ([hada] "Dense và Grouped GEMM":
 * fp8_gemm_{nt, nn, tn, tt}).  With every tensor stored row-major that reads:
 *
 *   nt: A [M][K], B [N][K]        nn: A [M][K], B [K][N]
 *   tn: A [K][M], B [K][N]        tt: A [K][M], B [N][K]
 *
 * Only where the bytes sit changes.  The scales keep their logical layouts
 * (SA [M][K/128], SB [ceil(N/128)][K/128]) and every output is the value defined
 * at the top of this file (plus C when C is given). */
ORACLE_API int fp8bs_oracle_dense_layout(int a_transposed, int b_transposed, const uint8_t* A,
                                         const float* SA, const uint8_t* B, const float* SB,
                                         const float* C, uint16_t* D, int64_t M, int64_t N,
                                         int64_t K) {
    int64_t r;
    if (!shape_ok(N, K) || M < 0) return -1;
    init_dec_table();
#pragma omp parallel for schedule(static)
    for (r = 0; r < M; ++r) {
        const int64_t kb = K / 128;
        /* row r of the left factor: stored as row r of A ("n") or column r ("t") */
        const uint8_t* a = a_transposed ? A + r : A + r * K;
        const ptrdiff_t a_step = a_transposed ? M : 1;
        int64_t n;
        for (n = 0; n < N; ++n) {
            /* column n of the right factor: row n of B ("t") or column n ("n") */
            const uint8_t* b = b_transposed ? B + n * K : B + n;
            const ptrdiff_t b_step = b_transposed ? 1 : N;
            double v = element_acc(a, a_step, SA + r * kb, 1, b, b_step, SB + (n / 128) * kb, 1, K);
            if (C) v += (double)C[r * N + n];
            D[r * N + n] = fp8bs_oracle_bf16_rne(v);
        }
    }
    return 0;
}

/* ---- K-grouped product for MoE weight gradients ---------------------------
 *
 * [hada] "Dense và Grouped GEMM": besides grouping along M, there is a grouping
 * along K for the MoE weight backward pass, with M and N fixed
 * (k_grouped_fp8_gemm_tn_contiguous).  The reading used here (the pages print
 * no formula):
 *
 * - tn form: A [K_total][M] and B [K_total][N], both stored with K outermost (the
 *   output gradient and the layer input, one row per token); group g owns the
 *   K rows [k_g, k_g + ks[g]), k_g = ks[0] + ... + ks[g-1], each ks[g] a multiple
 *   of 128 (zero allowed), so no 128-row chunk straddles two groups;
 * - both operands carry one FP32 scale per (row of the product, 128-K chunk), the
 *   1x128 activation granularity of [pxiaoer] "细粒度量化" taken along K:
 *   SA [M][K_total/128], SB [N][K_total/128] (logical layouts);
 * - D [G][M][N] is FP32 (a weight gradient), D[g] = C[g] + A_g^T B_g with the
 *   same per-chunk promotion as above, the sum taken in FP64 and rounded once to
 *   FP32 (nearest even); C may be NULL (zero).  An empty group gives D[g] = C[g]
 *   (or zeros).
 *
 * Returns 0, or -1 when a group size is negative or not a multiple of 128, or the
 * sizes do not add up to K_total. */
ORACLE_API int fp8bs_oracle_k_grouped(const uint8_t* A, const float* SA, const uint8_t* B,
                                      const float* SB, const int64_t* ks, const float* C,
                                      float* D, int64_t G, int64_t M, int64_t N,
                                      int64_t K_total) {
    int64_t g, sum = 0, i;
    if (G < 1 || M < 1 || N < 1 || K_total < 0 || K_total % 128 != 0) return -1;
    for (g = 0; g < G; ++g) {
        if (ks[g] < 0 || ks[g] % 128 != 0) return -1;
        sum += ks[g];
    }
    if (sum != K_total) return -1;
    init_dec_table();
#pragma omp parallel for schedule(static)
    for (i = 0; i < G * M; ++i) {
        const int64_t kbt = K_total / 128;
        int64_t gg = i / M, m = i % M, k0 = 0, j, n;
        for (j = 0; j < gg; ++j) k0 += ks[j];
        for (n = 0; n < N; ++n) {
            double v = element_acc(A + k0 * M + m, M, SA + m * kbt + k0 / 128, 1,
                                   B + k0 * N + n, N, SB + n * kbt + k0 / 128, 1, ks[gg]);
            if (C) v += (double)C[i * N + n];
            D[i * N + n] = (float)v;     /* one rounding, nearest even */
        }
    }
    return 0;
}

/* ---- quantisation (the step that produces A, SA, B and SB) ------------------
 *
 * [pxiaoer] FP8-training list ("细粒度量化", "在线量化"): activations are scaled per
 * 1x128 block and weights per 128x128 block, the factor computed online from the
 * block, and the values converted to FP8; [hada] "Giao diện GEMM và ràng buộc
 * layout": casting to FP8 is left to the caller.  The pages print no formula; the
 * reading used here (plainest maximum-abs scaling onto the e4m3 range):
 *
 *   a     = max(max_{block} |x|, 1e-4)                (FP32; the floor keeps an
 *                                                      all-zero block finite)
 *   scale = a / 448                                   (FP32 division, stored)
 *   inv   = 448 / a                                   (FP32 division, once per block)
 *   q     = e4m3(clamp(x * inv, -448, 448))           (FP32 product, then the
 *                                                      nearest e4m3 value, ties
 *                                                      to the even code)
 *
 * Every step is one IEEE FP32 operation (compiled with -ffp-contract=off), so the
 * GPU quantiser reproduces the codes and scales bit for bit. */

/* Nearest OCP e4m3 code of a value of magnitude at most 448, ties to the even code
 * (a code's last bit is its mantissa's last bit); the sign is kept (so -0 -> 0x80).
 * A plain search over the 127 non-negative finite codes, whose values increase
 * with the code.  NaN or magnitude above 448: the NaN code with x's sign. */
ORACLE_API uint8_t fp8bs_oracle_enc_e4m3(float x) {
    uint8_t sign = signbit(x) ? 0x80u : 0u;
    double a = fabs((double)x);
    int code, best = 0;
    double best_d;
    if (isnan(x) || a > 448.0) return (uint8_t)(sign | 0x7Fu);
    best_d = a;                                  /* distance to code 0 (value 0) */
    for (code = 1; code <= 126; ++code) {
        double d = fabs(a - fp8bs_oracle_dec_e4m3((uint8_t)code));
        if (d < best_d || (d == best_d && (code & 1) == 0)) {
            best = code;
            best_d = d;
        }
    }
    return (uint8_t)(sign | best);
}

static float block_scale_inputs(float amax, float* inv) {
    const float a = amax < 1e-4f ? 1e-4f : amax;
    *inv = 448.0f / a;
    return a / 448.0f;
}

static uint8_t quantise_one(float x, float inv) {
    float v = x * inv;
    if (v > 448.0f) v = 448.0f;
    if (v < -448.0f) v = -448.0f;
    return fp8bs_oracle_enc_e4m3(v);
}

/* Activations: X[rows][K] (FP32; BF16 inputs are widened exactly by the caller) ->
 * Q[rows][K] e4m3 bytes and S[rows][K/128] (logical layout).  Returns 0, or -1 when
 * K is not a positive multiple of 128. */
ORACLE_API int fp8bs_oracle_quant_1x128(const float* X, uint8_t* Q, float* S, int64_t rows,
                                        int64_t K) {
    int64_t r;
    if (K < 128 || K % 128 != 0 || rows < 0) return -1;
    init_dec_table();
#pragma omp parallel for schedule(static)
    for (r = 0; r < rows; ++r) {
        const int64_t groups = K / 128;
        int64_t c, k;
        for (c = 0; c < groups; ++c) {
            const float* x = X + r * K + 128 * c;
            float amax = 0.0f, inv;
            for (k = 0; k < 128; ++k)
                if (fabsf(x[k]) > amax) amax = fabsf(x[k]);
            S[r * groups + c] = block_scale_inputs(amax, &inv);
            for (k = 0; k < 128; ++k) Q[r * K + 128 * c + k] = quantise_one(x[k], inv);
        }
    }
    return 0;
}

/* Weights: X[G][N][K] -> Q[G][N][K] and S[G][ceil(N/128)][K/128]; the last row block
 * of an N that is not a multiple of 128 covers only its existing rows. */
ORACLE_API int fp8bs_oracle_quant_128x128(const float* X, uint8_t* Q, float* S, int64_t G,
                                          int64_t N, int64_t K) {
    int64_t nb = (N + 127) / 128, kb = K / 128, blk;
    if (K < 128 || K % 128 != 0 || N < 1 || G < 1) return -1;
    init_dec_table();
#pragma omp parallel for schedule(static)
    for (blk = 0; blk < G * nb * kb; ++blk) {
        int64_t g = blk / (nb * kb), i = (blk / kb) % nb, c = blk % kb, n, k;
        int64_t n1 = 128 * i + 128 < N ? 128 * i + 128 : N;
        float amax = 0.0f, inv, sc;
        for (n = 128 * i; n < n1; ++n)
            for (k = 128 * c; k < 128 * c + 128; ++k) {
                float v = fabsf(X[(g * N + n) * K + k]);
                if (v > amax) amax = v;
            }
        sc = block_scale_inputs(amax, &inv);
        S[(g * nb + i) * kb + c] = sc;
        for (n = 128 * i; n < n1; ++n)
            for (k = 128 * c; k < 128 * c + 128; ++k)
                Q[(g * N + n) * K + k] = quantise_one(X[(g * N + n) * K + k], inv);
    }
    return 0;
}

/* Threads an OpenMP parallel region of this library would use. */
ORACLE_API int fp8bs_oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
