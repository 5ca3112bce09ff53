/*
 * fp8bs.h -- C ABI of libfp8bs: block-scaled FP8 GEMM with BF16 output for
 * AMD Instinct MI355X (gfx950 / CDNA4).
 *
 * The operation (all three entry points):
 *
 *     D[r][n] = bf16( sum_c  P_c(r,n) * SFA(r,c) * SFB(n/128,c) )
 *     P_c(r,n) = sum_{k in [128c, 128c+128)} A[r][k] * B[n][k]
 *
 * A and B are OCP e4m3 (float8_e4m3fn: no infinities, max 448).  A carries one
 * FP32 scale per row and per 128-wide K group ("1x128"); B carries one FP32
 * scale per 128x128 block.  Each 128-K chunk's FP8 product is computed by the
 * matrix cores into an FP32 partial, multiplied by the two scales and added
 * into a separate FP32 accumulator (two-level accumulation), and the result is
 * rounded once to BF16 (round to nearest even).
 *
 * Sources (web pages, cited by title and section):
 *   - DeepGEMM README repost, lqnn.cn/news/60274, section "DeepGEMM": FP8
 *     GEMM with the fine-grained scaling of DeepSeek-V3, dense and MoE grouped
 *     GEMMs, two-level (promoted) accumulation on the CUDA cores.
 *   - "DeepGEMM: kernel FP8 GEMM sạch và hiệu quả nhờ scaling chi tiết",
 *     vi.news.hada.io/topic?id=19459:
 *       section "Giao diện GEMM và ràng buộc layout": the NT form
 *       D = C + A @ B.T (row-major A, column-major B), FP32 scale factors, the
 *       LHS scale factors in a TMA-aligned, transposed (MN-major) layout;
 *       section "Dense và Grouped GEMM": contiguous M-grouped layout (N, K fixed,
 *       expert segments concatenated along M, each aligned to the M block size)
 *       and the masked layout for graph-captured decoding, where the kernel
 *       computes only the valid region given a device mask tensor;
 *       section "Tiện ích và biến môi trường": set/get_num_sms,
 *       get_mk_alignment_for_contiguous_layout, get_tma_aligned_size,
 *       DG_PRINT_CONFIGS.
 *   - "deepseek开源周第三天：DeepGEMM深度分析", pxiaoer.blog: the FP8 training
 *     list (1x128 activation tiles, 128x128 weight blocks, FP32 accumulation).
 *   The "+ C" term of the pages' naming is available through the _c entry points;
 *   the nn / tn / tt stored forms and the K-grouped weight-gradient GEMM have entry
 *   points of their own (described next to them).
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers on the current HIP device; the
 *     caller owns every buffer (workspace included).  The library allocates
 *     nothing, keeps no pointer after returning and never synchronises `stream`.
 *   - Calls are asynchronous on `stream` (NULL = the default stream).  Buffers
 *     must stay alive until the stream work completes.
 *   - Inputs are read-only.  D is written only at valid rows (see each call)
 *     and columns n < N; every other byte of D is left untouched.
 *   - Pointers must be 16-byte aligned.  A call with no output rows (m, m_total
 *     or max_m == 0) checks its sizes, then returns FP8BS_OK without launching
 *     and without looking at any pointer (an empty buffer may be NULL).
 *     K must be a positive multiple of 128.
 *     One A slot (rows x K bytes: m, m_total or max_m rows) and one B group
 *     (N x K bytes) must each be smaller than 4 GiB.
 *   - SFA is stored MN-major ("transposed"): element (row r, K group c) lives at
 *     sfa[c * ld + r] with ld = fp8bs_get_sfa_ld(rows).  SFB is row-major
 *     [ceil(N/128)][K/128] per group.  D is row-major BF16 with row stride N.
 *   - Errors are reported by the return value before anything is launched;
 *     nothing is printed (unless FP8BS_PRINT_CONFIGS=1) and nothing aborts.
 *     A launch failure reported by the HIP runtime maps to FP8BS_ERR_HIP.
 *   - Thread-safe.  The only process-wide state is the CU cap
 *     (fp8bs_set_num_cus); the test pins (fp8bs_force_instance,
 *     fp8bs_force_splits) and the plan cache belong to the calling thread.
 *   - Graph-capturable: device-side group data (grouped_layout, masked_m) is
 *     never read on the host.
 */
#ifndef FP8BS_H
#define FP8BS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as HIP's stream handle. */
struct ihipStream_t;
typedef struct ihipStream_t* hipStream_t;

typedef enum {
    FP8BS_OK = 0,
    FP8BS_ERR_SHAPE = 1,        /* a size violates the preconditions          */
    FP8BS_ERR_POINTER = 2,      /* NULL or not 16-byte aligned                */
    FP8BS_ERR_UNSUPPORTED = 3,  /* no kernel instance covers the request      */
    FP8BS_ERR_HIP = 4           /* the HIP runtime reported an error          */
} fp8bs_status;

/* Layout codes for the planner queries (fp8bs_plan_query, fp8bs_workspace_size,
 * fp8bs_count_tiles, fp8bs_describe_config).  The first three are the NT entry
 * points; K_GROUPED is fp8bs_k_grouped_tn_contiguous (m = M, k = K_total, num_groups
 * groups); DENSE_NN / _TN / _TT are fp8bs_dense_nn / _tn / _tt.  OR-ing
 * FP8BS_LAYOUT_UE8M0 into a code asks about the packed power-of-two (_ue8m0) call of
 * that layout, which can only run the instances compiled for those scales. */
typedef enum {
    FP8BS_LAYOUT_DENSE = 0,
    FP8BS_LAYOUT_CONTIGUOUS = 1,
    FP8BS_LAYOUT_MASKED = 2,
    FP8BS_LAYOUT_K_GROUPED = 3,
    FP8BS_LAYOUT_DENSE_NN = 4,
    FP8BS_LAYOUT_DENSE_TN = 5,
    FP8BS_LAYOUT_DENSE_TT = 6,
    FP8BS_LAYOUT_UE8M0 = 16
} fp8bs_layout;

/*
 * Dense NT GEMM: D[m][n] = A[m][k] * B[n][k]^T with block scales.
 *   a    e4m3 [m][k] row-major          sfa  f32 [k/128][fp8bs_get_sfa_ld(m)]
 *   b    e4m3 [n][k] row-major          sfb  f32 [ceil(n/128)][k/128]
 *   d    bf16 [m][n] row-major          every row 0 <= r < m is valid.
 * m == 0 returns FP8BS_OK without launching.  (Section "Giao diện GEMM và
 * ràng buộc layout" of the hada page: fp8_gemm_nt.)
 */
int fp8bs_dense_nt(const void* a, const float* sfa, const void* b, const float* sfb, void* d,
                   int m, int n, int k, hipStream_t stream);

/*
 * M-grouped GEMM, contiguous layout: rows of several experts concatenated
 * along M; expert g multiplies its rows by B[g].
 *   a    e4m3 [m_total][k]              sfa  f32 [k/128][fp8bs_get_sfa_ld(m_total)]
 *   b    e4m3 [num_groups][n][k]        sfb  f32 [num_groups][ceil(n/128)][k/128]
 *   d    bf16 [m_total][n]
 *   grouped_layout  int32 [m_total] (device): expert index of each row, -1 for
 *        padding rows.  Each expert's segment starts at a multiple of
 *        fp8bs_get_mk_alignment() (128) rows and every 128-row block holds rows
 *        of a single expert followed only by padding.
 * Valid rows: 0 <= grouped_layout[r] < num_groups.  Padding rows and rows with
 * an index >= num_groups are not written.  m_total must be a multiple of 128.
 * (Section "Dense và Grouped GEMM" of the hada page: contiguous layout.)
 */
int fp8bs_grouped_contiguous_nt(const void* a, const float* sfa, const void* b, const float* sfb,
                                void* d, const int32_t* grouped_layout, int m_total, int n, int k,
                                int num_groups, hipStream_t stream);

/*
 * M-grouped GEMM, masked layout: each expert owns a slot of max_m rows of
 * which only the first masked_m[g] are valid; the host does not know
 * masked_m (it lives on the device, e.g. inside a captured graph).
 *   a    e4m3 [num_groups][max_m][k]    sfa  f32 [num_groups][k/128][fp8bs_get_sfa_ld(max_m)]
 *   b    e4m3 [num_groups][n][k]        sfb  f32 [num_groups][ceil(n/128)][k/128]
 *   d    bf16 [num_groups][max_m][n]
 *   masked_m  int32 [num_groups] (device); values are clamped to [0, max_m].
 *   expected_m  host hint of the typical masked_m (0 = unknown); it only
 *        steers the tile-shape choice and never changes results.
 * Valid rows: r < clamp(masked_m[g], 0, max_m) in slot g.  Other rows of D are
 * not written.  (Section "Dense và Grouped GEMM" of the hada page: masked
 * grouped GEMM for decoding under CUDA graphs.)
 */
int fp8bs_grouped_masked_nt(const void* a, const float* sfa, const void* b, const float* sfb,
                            void* d, const int32_t* masked_m, int num_groups, int max_m,
                            int expected_m, int n, int k, hipStream_t stream);

/*
 * Workspace variants.  The three calls below compute exactly what the call of
 * the same name without "_ws" computes; they differ only in that the caller
 * also lends `workspace` (device memory, 16-byte aligned, workspace_bytes long,
 * contents ignored and overwritten, not needed after the stream work ends).
 * With workspace the planner may split the K range of each output tile into S
 * ranges of whole 128-K chunks: every (tile, range) unit writes an FP32 partial
 * tile to the workspace, and a second kernel adds the S partials in the fixed
 * order 0..S-1 (so results do not depend on scheduling), rounds to BF16 and
 * stores the valid rows.  This fills the machine when M is small (decode):
 * output tiles alone then number far fewer than compute units.  Split-K is not
 * on the pages; it answers the under-filled-SM problem their block-size
 * discussion raises (DeepGEMM README repost, lqnn.cn/news/60274, section
 * "优化技术", unaligned block sizes).  Because the partial sums are added in a
 * different association than the unsplit kernel's, results may differ from the
 * workspace-free call in the last BF16 bit; both stay within the same bound of
 * the exact result.  workspace may be NULL when workspace_bytes is 0 (then no
 * split is used).  Two calls in flight at once must not share a workspace.
 */
int fp8bs_dense_nt_ws(const void* a, const float* sfa, const void* b, const float* sfb, void* d,
                      int m, int n, int k, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);
int fp8bs_grouped_contiguous_nt_ws(const void* a, const float* sfa, const void* b,
                                   const float* sfb, void* d, const int32_t* grouped_layout,
                                   int m_total, int n, int k, int num_groups, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream);
int fp8bs_grouped_masked_nt_ws(const void* a, const float* sfa, const void* b, const float* sfb,
                               void* d, const int32_t* masked_m, int num_groups, int max_m,
                               int expected_m, int n, int k, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);

/*
 * Addend variants: D = bf16(C + A * B^T) -- the full NT form of [hada] "Giao diện GEMM
 * và ràng buộc layout" (fp8_gemm_nt computes D = C + A @ B.T).  c is FP32 with D's
 * shape and layout ([rows][n], masked [num_groups][max_m][n], row stride n, 16-byte
 * aligned); it is read only at D's valid rows and columns, added to the FP32
 * accumulator once, after the last K chunk (after the split-K reduction when K is
 * split), and the sum is rounded once to BF16.  c may not overlap d.  Otherwise as
 * the _ws calls.
 */
int fp8bs_dense_nt_c(const void* a, const float* sfa, const void* b, const float* sfb,
                     const float* c, void* d, int m, int n, int k, void* workspace,
                     size_t workspace_bytes, hipStream_t stream);
int fp8bs_grouped_contiguous_nt_c(const void* a, const float* sfa, const void* b,
                                  const float* sfb, const float* c, void* d,
                                  const int32_t* grouped_layout, int m_total, int n, int k,
                                  int num_groups, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream);
int fp8bs_grouped_masked_nt_c(const void* a, const float* sfa, const void* b, const float* sfb,
                              const float* c, void* d, const int32_t* masked_m, int num_groups,
                              int max_m, int expected_m, int n, int k, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/*
 * Power-of-two scale variants (packed UE8M0).  The same operation with every scale a
 * power of two, given as an 8-bit biased exponent e (value 2^(e-127); E8M0, no sign,
 * no mantissa; e = 255 is not a number) packed four K groups per 32-bit word -- the
 * packed UE8M0 format [hada] "Giao diện GEMM và ràng buộc layout" describes for SM100
 * (four UE8M0 values in one int).  Byte j (least significant first) of word w holds
 * K group 4w + j:
 *   sfa  int32 [ceil(k/512)][fp8bs_get_sfa_ld(rows)] MN-major (masked: per slot,
 *        [num_groups][ceil(k/512)][ld(max_m)]); row r, group c at byte c%4 of
 *        sfa[(c/4)*ld + r]
 *   sfb  int32 [num_groups][ceil(n/128)][ceil(k/512)]; block (i, c) at byte c%4 of
 *        sfb[(g*ceil(n/128) + i)*ceil(k/512) + c/4]
 * Everything else (operands, D, valid rows, workspace and its split-K use, errors) is
 * as for the _ws calls.  gfx950's block-scaled matrix instructions apply the factors
 * and accumulate across K groups themselves, so there is no FP32 promotion step; the
 * result is within the same bound of the exact value.
 */
int fp8bs_dense_nt_ue8m0(const void* a, const int32_t* sfa, const void* b, const int32_t* sfb,
                         void* d, int m, int n, int k, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);
int fp8bs_grouped_contiguous_nt_ue8m0(const void* a, const int32_t* sfa, const void* b,
                                      const int32_t* sfb, void* d, const int32_t* grouped_layout,
                                      int m_total, int n, int k, int num_groups, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream);
int fp8bs_grouped_masked_nt_ue8m0(const void* a, const int32_t* sfa, const void* b,
                                  const int32_t* sfb, void* d, const int32_t* masked_m,
                                  int num_groups, int max_m, int expected_m, int n, int k,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Dense GEMM with the other stored operand forms ([hada] "Giao diện GEMM và ràng
 * buộc layout" and "Dense và Grouped GEMM": kernels named for D = C + A @ B, the
 * two letters saying whether A and B enter as stored or transposed; the newer
 * architecture accepts nt, tn, nn and tt).  Every tensor is row-major:
 *   nn:  a e4m3 [m][k],  b e4m3 [k][n]      (D = A B)
 *   tn:  a e4m3 [k][m],  b e4m3 [k][n]      (D = A^T B)
 *   tt:  a e4m3 [k][m],  b e4m3 [n][k]      (D = A^T B^T)
 * The value, the scales (sfa f32 [k/128][fp8bs_get_sfa_ld(m)] MN-major, sfb f32
 * [ceil(n/128)][k/128]) and D (bf16 [m][n]) are those of fp8bs_dense_nt_c: logical row
 * r of A and column n of B meet along K whatever their storage.  An operand stored
 * with M (or N) contiguous is staged in LDS as it lies and its MFMA fragments are read
 * with gfx950's transpose loads, so no transposed copy is made.
 * Preconditions on top of the NT ones: a stored [k][m] needs m % 16 == 0, a stored
 * [k][n] needs n % 16 == 0 (16-byte rows).  c (FP32 [m][n], may not overlap d) and
 * workspace (split-K, as for the _ws calls) may be NULL.
 */
int fp8bs_dense_nn(const void* a, const float* sfa, const void* b, const float* sfb,
                   const float* c, void* d, int m, int n, int k, void* workspace,
                   size_t workspace_bytes, hipStream_t stream);
int fp8bs_dense_tn(const void* a, const float* sfa, const void* b, const float* sfb,
                   const float* c, void* d, int m, int n, int k, void* workspace,
                   size_t workspace_bytes, hipStream_t stream);
int fp8bs_dense_tt(const void* a, const float* sfa, const void* b, const float* sfb,
                   const float* c, void* d, int m, int n, int k, void* workspace,
                   size_t workspace_bytes, hipStream_t stream);

/*
 * K-grouped GEMM for MoE weight gradients ([hada] "Dense và Grouped GEMM": grouping
 * along K for the MoE weight backward pass, M and N fixed,
 * k_grouped_fp8_gemm_tn_contiguous).  Groups run along K: group g owns K rows
 * [k_g, k_g + ks[g]), k_g = ks[0] + ... + ks[g-1], and
 *
 *     D[g][m][n] = fp32( C[g][m][n] + sum over group g's chunks c of
 *                        P_c(m,n) * SFA(m,c) * SFB(n,c) ),
 *     P_c(m,n) = sum_{k in [128c, 128c+128)} A[k][m] * B[k][n]
 *
 * (the tn form: both operands stored with K outermost, one row per token).
 *   a    e4m3 [k_total][m]     sfa  f32 [k_total/128][fp8bs_get_sfa_ld(m)]
 *   b    e4m3 [k_total][n]     sfb  f32 [k_total/128][fp8bs_get_sfa_ld(n)]
 *        (one scale per feature and 128-token chunk on both sides)
 *   c    f32 [num_groups][m][n] or NULL (zero); may be the same buffer as d
 *   d    f32 [num_groups][m][n], every element written
 *   ks   HOST int32 [num_groups]: tokens per group, each a multiple of 128 (0 allowed:
 *        D[g] = C[g] or zeros), adding up to k_total; read during the call only.
 * Preconditions: 1 <= num_groups <= 256; m and n multiples of 16 (>= 16); k_total a
 * multiple of 128 (0 allowed).  workspace (split-K) may be NULL.  The group sizes are
 * taken on the host and travel in the kernel arguments, so a captured graph replays
 * the sizes it was captured with.
 */
int fp8bs_k_grouped_tn_contiguous(const void* a, const float* sfa, const void* b,
                                  const float* sfb, const float* c, float* d, const int32_t* ks,
                                  int num_groups, int m, int n, int k_total, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/*
 * Power-of-two scale variants of the stored-form and K-grouped calls (the SM100 form of
 * the pages: packed UE8M0, [hada] "Giao diện GEMM và ràng buộc layout").  Scales are
 * packed four K groups per int32 exactly as for fp8bs_dense_nt_ue8m0:
 *   dense nn / tn / tt: sfa int32 [ceil(k/512)][fp8bs_get_sfa_ld(m)] (MN-major),
 *                       sfb int32 [ceil(n/128)][ceil(k/512)];
 *   K-grouped:          sfa int32 [ceil(k_total/512)][fp8bs_get_sfa_ld(m)],
 *                       sfb int32 [ceil(k_total/512)][fp8bs_get_sfa_ld(n)]
 *                       (one exponent per feature and 128-token chunk on both sides).
 * Everything else (operands, C, D, ks, workspace, preconditions, errors) is as for the
 * FP32-scale calls above; the matrix core applies both exponents and accumulates across
 * chunks, so the result has the promotion-free rounding of the UE8M0 NT calls.
 */
int fp8bs_dense_nn_ue8m0(const void* a, const int32_t* sfa, const void* b, const int32_t* sfb,
                         const float* c, void* d, int m, int n, int k, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);
int fp8bs_dense_tn_ue8m0(const void* a, const int32_t* sfa, const void* b, const int32_t* sfb,
                         const float* c, void* d, int m, int n, int k, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);
int fp8bs_dense_tt_ue8m0(const void* a, const int32_t* sfa, const void* b, const int32_t* sfb,
                         const float* c, void* d, int m, int n, int k, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);
int fp8bs_k_grouped_tn_contiguous_ue8m0(const void* a, const int32_t* sfa, const void* b,
                                        const int32_t* sfb, const float* c, float* d,
                                        const int32_t* ks, int num_groups, int m, int n,
                                        int k_total, void* workspace, size_t workspace_bytes,
                                        hipStream_t stream);

/*
 * No-allocation dense call, for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.  It computes
 * what fp8bs_dense_nt_ws computes, with the split-K workspace taken from a library-owned
 * device array of FP8BS_NOALLOC_SCRATCH_BYTES (32 MiB) instead of from the caller: each GPU
 * the library runs on holds one such array from its first use until the process ends.
 * The call allocates nothing (no hipMalloc, no allocating library routine); the caller
 * still owns and passes a, sfa, b, sfb and d (same layouts as fp8bs_dense_nt).  The planner
 * only picks plans whose FP32 partial tiles fit the array, so every valid size is accepted;
 * a pinned split count (fp8bs_force_splits) that would need more is refused with
 * FP8BS_ERR_UNSUPPORTED before anything is launched.  The array keeps the last call's
 * partials; nothing in it has to start at zero.  Every call on one GPU shares that GPU's
 * array: two calls that may overlap on one GPU (different streams, or a graph replayed
 * while another call runs) race on it and must be ordered by the caller.  Returns
 * FP8BS_ERR_HIP if the array's device address cannot be obtained.
 */
#define FP8BS_NOALLOC_SCRATCH_BYTES (32u << 20)
int fp8bs_dense_nt_noalloc(const void* a, const float* sfa, const void* b, const float* sfb,
                           void* d, int m, int n, int k, hipStream_t stream);
/* Size of that array in bytes (FP8BS_NOALLOC_SCRATCH_BYTES). */
size_t fp8bs_noalloc_scratch_bytes(void);

/* Workspace bytes the planner's preferred plan uses for a request on the current
 * device (CU cap respected; `m` as in fp8bs_plan_query).  0 means the best plan
 * splits nothing.  Passing at least this much to a _ws call lets it use that
 * plan; less makes it pick the best plan that fits.  On an invalid request, a
 * pin the request cannot use, or a HIP error it returns the negated status
 * (-FP8BS_ERR_SHAPE, -FP8BS_ERR_UNSUPPORTED, -FP8BS_ERR_HIP). */
int64_t fp8bs_workspace_size(int layout, int64_t m, int n, int k, int num_groups,
                             int expected_m);

/* Element types of quantiser inputs. */
typedef enum {
    FP8BS_DTYPE_F32 = 0,
    FP8BS_DTYPE_BF16 = 1
} fp8bs_dtype;

/*
 * Quantisers: produce the GEMM operands from FP32 or BF16 values, with the
 * fine-grained online scaling of the FP8-training list in
 * "deepseek开源周第三天：DeepGEMM深度分析" (pxiaoer.blog: one factor per 1x128
 * activation block and per 128x128 weight block, computed from the block, values
 * converted to FP8); the pages leave this cast to the caller ([hada] "Giao diện
 * GEMM và ràng buộc layout").  Per block, each step one IEEE FP32 operation:
 *
 *     a = max(max_block |x|, 1e-4);  scale = a / 448;  inv = 448 / a;
 *     q = e4m3(clamp(x * inv, -448, 448))   (nearest e4m3 value, ties to even;
 *                                            a negative value rounding to zero
 *                                            gives 0x80)
 *
 * NaN inputs never raise a block's maximum and quantise to the NaN code.
 *
 * fp8bs_quantize_1x128 -- activations, `groups` slots of `rows` rows:
 *   x    f32 or bf16 [groups][rows][k] row-major (16-byte aligned)
 *   q    e4m3 [groups][rows][k] (written; 16-byte aligned)
 *   sfa  f32 [groups][k/128][fp8bs_get_sfa_ld(rows)] MN-major, the layout the GEMM
 *        entry points read (groups = 1: dense / contiguous A; groups = G: masked A).
 *        Entries for rows r < rows are written; the alignment padding is not.
 * fp8bs_quantize_128x128 -- weights:
 *   x    f32 or bf16 [groups][n][k];  q  e4m3 [groups][n][k]
 *   sfb  f32 [groups][ceil(n/128)][k/128]; the last row block of an n that is not a
 *        multiple of 128 covers only its existing rows.
 * k must be a positive multiple of 128.  Asynchronous on `stream`, no allocation;
 * returns FP8BS_ERR_SHAPE / _POINTER / _UNSUPPORTED (unknown x_dtype) before
 * launching, FP8BS_ERR_HIP if the launch fails; rows == 0 is a no-op.
 */
int fp8bs_quantize_1x128(const void* x, int x_dtype, void* q, float* sfa, int groups, int rows,
                         int k, hipStream_t stream);
int fp8bs_quantize_128x128(const void* x, int x_dtype, void* q, float* sfb, int groups, int n,
                           int k, hipStream_t stream);

/* Row alignment of expert segments in the contiguous layout (128).  Analogue
 * of get_mk_alignment_for_contiguous_layout (hada page, section "Tiện ích và
 * biến môi trường"). */
int fp8bs_get_mk_alignment(void);

/* Leading dimension, in floats, of the MN-major SFA for `rows` rows: rows
 * rounded up to a multiple of 4 (16 bytes).  Analogue of get_tma_aligned_size
 * (same section).  Returns -1 for rows < 0. */
int64_t fp8bs_get_sfa_ld(int64_t rows);

/* Cap on the compute units the persistent grid may occupy (0 = all).  It
 * changes the launch shape, never the results.  Analogue of set_num_sms.
 * Returns the previous cap, or -1 for n < 0. */
int fp8bs_set_num_cus(int n);
/* The current cap (0 = no cap). */
int fp8bs_get_num_cus(void);

/* Pins every later call of the calling thread to compiled instance i (see
 * fp8bs_instance_info); -1 restores the planner's choice.  Other threads' calls are
 * not affected.  For testing and measuring tile shapes:
 * the choice of instance changes speed, never results.  Returns the previous
 * setting, or -2 for an index out of range. */
int fp8bs_force_instance(int i);

/* Pins the K split count of the calling thread's later _ws calls to s >= 1 (1 = no
 * split); 0 restores the planner's choice.  Without a pinned instance the planner then
 * picks the best instance that runs with s splits (fp8bs_workspace_size reports that
 * plan's workspace).  A pinned count that the request cannot use (s > K/128, s x K/128
 * of 2^32 or more, or more workspace than lent) makes the call fail with
 * FP8BS_ERR_UNSUPPORTED.  For testing and measuring; changes speed, and
 * results only within the bound stated for the _ws calls.  Returns the previous
 * setting, or -1 for s < 0. */
int fp8bs_force_splits(int s);

/* Planner result for one request, as chosen by the entry points. */
typedef struct {
    int block_m;        /* rows per output tile                               */
    int block_n;        /* columns per output tile (may be non-power-of-two)  */
    int waves_m;        /* wavefronts along M in a workgroup                  */
    int waves_n;        /* wavefronts along N                                 */
    int threads;        /* threads per workgroup                              */
    int lds_bytes;      /* LDS per workgroup                                  */
    int wg_per_cu;      /* workgroups resident per CU the planner assumes     */
    int stages;         /* 128-K chunks the LDS ring holds                    */
    int64_t tiles;      /* upper bound of output tiles in the schedule        */
    int64_t grid;       /* persistent workgroups launched                     */
    int raster;         /* m-blocks per raster group                          */
    int instance;       /* index of the compiled kernel instance              */
    int splits;         /* K ranges per tile (1: no split, no workspace)      */
    int64_t workspace_bytes; /* workspace the plan uses (0 when splits == 1)  */
    int kind;           /* 0: A and B tiles staged in LDS, persistent grid;
                           1: B streamed into registers, one workgroup per unit */
    int ue8m0;          /* 1: the instance is also compiled for packed UE8M0 scales */
    int mn;             /* 1: the instance is also compiled for MN-major operands
                           (dense nn / tn / tt, K-grouped) */
} fp8bs_plan;

/*
 * Host-only planner query (no device access): the configuration the entry
 * point for `layout` would use for these sizes on a device with `num_cus`
 * compute units when lent `workspace_bytes` of workspace (0: the call without
 * "_ws").  For FP8BS_LAYOUT_DENSE `m` is M; for CONTIGUOUS it is m_total; for
 * MASKED it is max_m (num_groups groups, expected_m hint).  Returns FP8BS_OK
 * and fills *out, or an error status.  Pins (fp8bs_force_instance,
 * fp8bs_force_splits) are not applied here.
 */
int fp8bs_plan_query(int layout, int64_t m, int n, int k, int num_groups, int expected_m,
                     int num_cus, int64_t workspace_bytes, fp8bs_plan* out);

/* Output tiles a (block_m x block_n) tiling has for a request: m-blocks x
 * n-blocks (x num_groups for MASKED, where m is max_m).  Plain tile
 * arithmetic, no device access; -1 on invalid arguments. */
int64_t fp8bs_count_tiles(int layout, int64_t m, int n, int num_groups, int block_m, int block_n);

/* Number of compiled kernel instances, and the shape of instance i (fields
 * tiles, grid, raster and workspace_bytes are 0, splits is 1).  fp8bs_instance_info returns FP8BS_OK or
 * FP8BS_ERR_UNSUPPORTED for an index out of range. */
int fp8bs_num_instances(void);
int fp8bs_instance_info(int i, fp8bs_plan* out);

/* Human-readable summary of the plan a _ws call lent fp8bs_workspace_size
 * bytes would use for a request on the current device's CU count (respecting
 * the cap and the pins), written to buf (NUL-terminated, truncated to len).  Analogue of DG_PRINT_CONFIGS; FP8BS_PRINT_CONFIGS=1 prints the same
 * line to stderr at every call.  Returns the status of the planner. */
int fp8bs_describe_config(int layout, int64_t m, int n, int k, int num_groups, int expected_m,
                          char* buf, size_t len);

/* Static description of a status code. */
const char* fp8bs_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FP8BS_H */
