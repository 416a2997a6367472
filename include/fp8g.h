/*
 * fp8g -- FP8 (E4M3) groupwise-scaled NT GEMM for MoE expert layers, native to AMD MI355X (gfx950).
 *
 * C ABI of libfp8g.so. Every entry point takes plain device pointers and sizes and returns a status;
 * no PyTorch (or any other framework) type appears here.
 *
 * Conventions shared by every call (flashmla-rs README, section "Design Notes"; flashinfer-rs
 * README, section "Additional Notes"):
 *   - Memory is owned by the caller. Every pointer argument is a DEVICE pointer on the current HIP
 *     device unless it is documented otherwise. The library never allocates, frees or keeps a
 *     pointer after the call returns; scratch space comes in as a workspace argument, except for
 *     fp8_moe_build_permutation_noalloc, which uses a fixed array of the library's own.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream) and the call returns
 *     without synchronising. No call reads device memory from the host.
 *   - Arguments are validated before anything is launched; C++ exceptions never cross the ABI. A
 *     failing call returns a non-zero status, launches nothing and leaves a message that
 *     fp8g_last_error() returns (thread-local, valid until the thread's next fp8g call).
 *   - An unsupported device (anything but gfx950) is an error (FP8G_NOT_SUPPORTED), never a fallback.
 *   - Tensors are dense and row-major ("contiguous"); E4M3 means OCP E4M3FN (bias 7, max 448,
 *     NaN = S.1111.111, no infinities), one byte per element. BF16 and FP16 outputs are
 *     round-to-nearest-even.
 *   - Pointers must be 16-byte aligned (E4M3 operands, outputs) or 4-byte aligned (scales, indices).
 *   - Output rows that the operation leaves unspecified are not written.
 *
 * Scale granularity: only (gran_m, gran_n, gran_k) = (1, 128, 128) -- one FP32 scale per row and
 * 128-wide K block of `a`, one per 128x128 block of `b` -- is implemented; any other value returns
 * FP8G_NOT_SUPPORTED. k must be a multiple of 128 in every form; n must be a multiple of 128 in the
 * grouped and masked forms (the plain form takes any n: its last b-scale block may cover fewer than
 * 128 rows of b).
 *
 * Arithmetic (MATE FlashInfer-API page, section "GEMM"): for every output element
 *     out[i][j] = cvt( sum_kb  sa(i,kb) * sb(j/128,kb) * sum_{k in block kb} a[i][k] * b[j][k] )
 * where each 128-wide block sum is one FP8 matrix-core product accumulated in FP32 and the scale
 * product is applied by one FP32 multiply-add per K block; cvt rounds the FP32 sum to the output
 * type (out_dtype: BF16 by default, or FP16 -- the page's out_dtype). Results do not depend on
 * `expected_m` or on the tile configuration the library picks.
 */
#ifndef FP8G_H_
#define FP8G_H_

#include <stdint.h>

#if defined(__GNUC__)
#define FP8G_API __attribute__((visibility("default")))
#else
#define FP8G_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FP8G_OK = 0,
  FP8G_INVALID_ARGUMENT = 1, /* null pointer, bad size, misalignment, bad enum value */
  FP8G_NOT_SUPPORTED = 2,    /* unsupported granularity, or the device is not gfx950 */
  FP8G_HIP_ERROR = 3,        /* the HIP runtime reported an error (message has hipGetErrorString) */
  FP8G_INTERNAL = 4          /* an unexpected C++ exception inside the library */
} fp8g_status_t;

typedef enum {
  FP8G_OUT_BF16 = 0, /* bfloat16 */
  FP8G_OUT_FP16 = 1  /* IEEE binary16; values beyond its range become +-inf */
} fp8g_out_dtype_t;

typedef enum {
  FP8G_SCALE_K_MAJOR = 0,  /* a_scale (m, k/128), b_scale (n/128, k/128) */
  FP8G_SCALE_MN_MAJOR = 1  /* a_scale (k/128, m), b_scale (k/128, n/128) */
} fp8g_scale_major_t;

/* Message of the calling thread's last failing call ("" after a successful one). */
FP8G_API const char* fp8g_last_error(void);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
FP8G_API int32_t fp8g_version(void);

/*
 * Measurement aid (not part of the method): the shader clock the device runs at. Enqueues on
 * `stream` one single-wave kernel that spins for about spin_us (0 .. 100000) microseconds of the
 * device's constant-rate wall clock and writes to out (device memory, two uint64, 8-byte aligned)
 * the shader-clock cycles and the wall-clock ticks that passed. The average shader clock in kHz is
 * out[0] / out[1] * fp8g_wall_clock_khz(). Enqueued right after a timed region it reads the clock
 * the part settled at under that load.
 */
FP8G_API fp8g_status_t fp8g_clock_probe(unsigned long long* out, int64_t spin_us, void* stream);

/*
 * Measurement aid (not part of the method): the clock the most recent GEMM launch on the current
 * device ran at. Every GEMM kernel's first workgroup stamps the shader-clock counter and the
 * constant-rate wall clock when it starts and when it leaves; this copies the four stamps (start
 * cycles, start ticks, end cycles, end ticks) to host_out (HOST memory, four uint64). The average
 * shader clock in kHz is (end cycles - start cycles) / (end ticks - start ticks) * fp8g_wall_clock_khz().
 * Synchronous (a device-to-host copy); launches overlapping on several streams overwrite each other's
 * stamps.
 */
FP8G_API fp8g_status_t fp8g_gemm_clock_record(unsigned long long* host_out);

/* Rate of the current device's wall clock (hipDeviceAttributeWallClockRate) in kHz; -1 on error. */
FP8G_API int64_t fp8g_wall_clock_khz(void);

/*
 * Plain form: out = a @ b.T with groupwise scales.
 * MATE FlashInfer-API page, section "GEMM", gemm_fp8_nt_groupwise.
 *   a        (m, k)  E4M3, row-major
 *   b        (n, k)  E4M3, row-major (the product is a @ b.T)
 *   a_scale  FP32, (m, k/128) when scale_major = K-major, (k/128, m) when MN-major
 *   b_scale  FP32, (NB, k/128) when K-major, (k/128, NB) when MN-major, NB = ceil(n/128)
 *   out      (m, n)  BF16 or FP16 (out_dtype), fully written
 * m >= 0 and n >= 0 are arbitrary (output column j uses b-scale block j/128, so the last block may
 * cover fewer than 128 rows of b); k is a multiple of 128. m == 0 or n == 0 is a no-op; k == 0
 * writes zeros. scale_major applies to both scale tensors.
 */
FP8G_API fp8g_status_t fp8_gemm_nt_groupwise(const void* a, const void* b, const float* a_scale,
                                    const float* b_scale, void* out, int32_t out_dtype, int64_t m,
                                    int64_t n, int64_t k, int32_t scale_major, int32_t gran_m,
                                    int32_t gran_n, int32_t gran_k, void* stream);

/*
 * Plain form with FP8 output: gemm_fp8_nt_groupwise's output_scale (MATE FlashInfer-API page,
 * section "GEMM"), an FP32 scale for E4M3 output. Read here as one per-tensor dequantisation
 * scale s = output_scale[0] (a device pointer):
 *   out[i][j] = E4M3_RNE(saturate(acc[i][j] / s))   (FP32 IEEE division; beyond +-448 the code
 *                                                    is +-448, NaN stays NaN)
 * where acc is the FP32 value the plain form would round to BF16. Arguments and sizes as for
 * fp8_gemm_nt_groupwise; out (m, n) holds E4M3 codes.
 */
FP8G_API fp8g_status_t fp8_gemm_nt_groupwise_fp8_out(const void* a, const void* b, const float* a_scale,
                                            const float* b_scale, void* out,
                                            const float* output_scale, int64_t m, int64_t n,
                                            int64_t k, int32_t scale_major, int32_t gran_m,
                                            int32_t gran_n, int32_t gran_k, void* stream);

/*
 * Contiguous grouped form: out[i] = a[i] @ b[m_indices[i]].T for every row with m_indices[i] >= 0.
 * MATE FlashInfer-API page, section "GEMM", group_deepgemm_fp8_nt_groupwise.
 *   a          (m, k)              E4M3; m is a multiple of 128
 *   b          (num_groups, n, k)  E4M3 expert weights
 *   a_scale    FP32, (m, k/128) K-major, or (k/128, m) MN-major
 *   b_scale    FP32, (num_groups, n/128, k/128) K-major, or (num_groups, k/128, n/128) MN-major
 *   m_indices  (m,) int32 expert of every row; -1 marks a padding row. Each expert's rows occupy a
 *              contiguous, 128-row-aligned region, so every aligned 128-row tile holds one expert
 *              and padding. The tile's expert is the largest index among its rows.
 *   out        (m, n) BF16 or FP16 (out_dtype); rows whose m_indices is -1 (or is not the tile's
 *              expert) are not written.
 * Indices outside [-1, num_groups) are treated as padding. The MN-major layout is an extension
 * (the page defines the grouped forms with K-major scales only).
 */
FP8G_API fp8g_status_t fp8_group_gemm_contiguous(const void* a, const void* b, const float* a_scale,
                                        const float* b_scale, const int32_t* m_indices, void* out,
                                        int32_t out_dtype, int64_t m, int64_t n, int64_t k,
                                        int64_t num_groups,
                                        int32_t scale_major, int32_t gran_m, int32_t gran_n,
                                        int32_t gran_k, void* stream);

/*
 * Contiguous grouped form with gathered rows of a: row r of the product reads row a_rows[r] of a
 * (and of a_scale), i.e. out[r] = a[a_rows[r]] @ b[m_indices[r]].T for every r with
 * m_indices[r] >= 0. This is the contiguous form of the MATE FlashInfer-API page (section "GEMM")
 * applied to the permuted token rows of the expert FFN (flashinfer-rs README, section "API
 * Example: Fused MoE FP8 (cudarc)"), without materialising the permuted copy of the tokens.
 *   a          (a_rows_total, k) E4M3; a_scale (a_rows_total, k/128) K-major or
 *              (k/128, a_rows_total) MN-major
 *   a_rows     (m,) int32 device array; entries of rows with m_indices[r] >= 0 must lie in
 *              [0, a_rows_total) (other rows are never stored; an out-of-range entry there reads
 *              row 0)
 *   everything else as fp8_group_gemm_contiguous.
 */
FP8G_API fp8g_status_t fp8_group_gemm_contiguous_gather(const void* a, const float* a_scale,
                                               int64_t a_rows_total, const int32_t* a_rows,
                                               const void* b, const float* b_scale,
                                               const int32_t* m_indices, void* out, int32_t out_dtype,
                                               int64_t m, int64_t n, int64_t k, int64_t num_groups,
                                               int32_t scale_major, int32_t gran_m, int32_t gran_n,
                                               int32_t gran_k, void* stream);

/*
 * Masked batched form: out[g, :masked_m[g]] = a[g, :masked_m[g]] @ b[g].T.
 * MATE FlashInfer-API page, section "GEMM", batch_deepgemm_fp8_nt_groupwise.
 *   a          (num_groups, max_m, k)  E4M3
 *   b          (num_groups, n, k)      E4M3
 *   a_scale    FP32, (num_groups, max_m, k/128) K-major, or (num_groups, k/128, max_m) MN-major
 *   b_scale    FP32, (num_groups, n/128, k/128) K-major, or (num_groups, k/128, n/128) MN-major
 *   masked_m   (num_groups,) int32 valid rows per group, read on the device; values are clamped
 *              into [0, max_m]
 *   expected_m host-side hint of the typical masked_m, used only to pick a tile configuration
 *   out        (num_groups, max_m, n) BF16 or FP16 (out_dtype); rows at or beyond masked_m[g] are
 *              not written
 */
FP8G_API fp8g_status_t fp8_batch_gemm_masked(const void* a, const void* b, const float* a_scale,
                                    const float* b_scale, const int32_t* masked_m,
                                    int64_t expected_m, void* out, int32_t out_dtype,
                                    int64_t num_groups,
                                    int64_t max_m, int64_t n, int64_t k, int32_t scale_major,
                                    int32_t gran_m, int32_t gran_n, int32_t gran_k, void* stream);

/*
 * Batched FP8 GEMM with per-tensor or per-channel scales (MATE FlashInfer-API page, section "GEMM",
 * bmm_fp8):
 *   out[g] = sa_g * sb_g * (a[g] @ b[g])    for g < batch
 *   a        (batch, m, k) E4M3, row-major
 *   b        (batch, k, n) E4M3, row-major (n contiguous: the product is a @ b, not a @ b.T)
 *   a_scale  FP32: one value (a_scale_per_row = 0) or (batch, m), one per row (= 1)
 *   b_scale  FP32: one value (b_scale_per_col = 0) or (batch, n), one per column (= 1)
 *   out      (batch, m, n) BF16 or FP16 (out_dtype), fully written
 * b is read in place (no copy, no workspace). The k-sum is accumulated in FP32 over all of k, then
 * multiplied by the FP32 product of the two scales. k is a multiple of 128 and n of 16; m is
 * arbitrary; batch <= 65535. E4M3 only.
 */
FP8G_API fp8g_status_t fp8_bmm(const void* a, const void* b, const float* a_scale, int32_t a_scale_per_row,
                      const float* b_scale, int32_t b_scale_per_col, void* out, int32_t out_dtype,
                      int64_t batch, int64_t m, int64_t n, int64_t k, void* stream);

/* ---------------------------------------------------------------------------------------------
 * Producers of the a operand (1x128 E4M3 rows with FP32 scales).
 * ------------------------------------------------------------------------------------------- */

/*
 * 1x128 activation quantiser: for every row r and 128-column block c of x,
 *   scale[r][c] = amax / 448 (FP32 IEEE division; 1 when the block is all zero)
 *   out[r][c*128 + t] = E4M3_RNE(x[r][c*128 + t] / scale[r][c])   (FP32 IEEE division)
 * The a_scale layout of the MATE FlashInfer-API page (section "GEMM"): K-major (rows, cols/128) or
 * MN-major (cols/128, rows).
 *   x         (rows, cols) BF16; out (rows, cols) E4M3; scale_out FP32 in scale_major layout
 * cols must be a multiple of 128.
 */
FP8G_API fp8g_status_t fp8_quantize_1x128(const void* x, int64_t rows, int64_t cols, void* out,
                                 float* scale_out, int32_t scale_major, void* stream);

/*
 * Fused add-RMSNorm with 1x128 FP8 quantisation (MATE FlashInfer-API page, section "norm",
 * fused_add_rmsnorm_fp8_block_quant; arguments in its order):
 *   residual[r]   <- bf16(input[r] + residual[r])                 (in place; FP32 sum, RNE)
 *   normed_out[r] <- bf16(residual[r] * (1/sqrt(mean_j residual[r][j]^2 + eps)) * weight)
 *   out[r], block_scale[r]  <- the 1x128 quantisation above of normed_out[r]
 * All arithmetic is FP32 (the mean is an FP32 sum of squares over hidden divided by hidden).
 *   input, residual, normed_out  (rows, hidden) BF16;  weight (hidden,) BF16
 *   out (rows, hidden) E4M3;  block_scale FP32, (rows, hidden/128) K-major or (hidden/128, rows)
 *   MN-major
 * hidden must be a multiple of 128; normed_out may be input; residual must be distinct from the
 * other tensors.
 */
FP8G_API fp8g_status_t fp8_fused_add_rmsnorm_quant(void* out, float* block_scale, void* normed_out,
                                          const void* input, void* residual, const void* weight,
                                          float eps, int64_t rows, int64_t hidden,
                                          int32_t scale_major, void* stream);

/* ---------------------------------------------------------------------------------------------
 * Expert-FFN steps around the grouped GEMM (flashinfer-rs README, section "API Example: Fused MoE
 * FP8 (cudarc)", DeepSeek FP8 block-scale mode: BF16 tokens, int32 token_selected
 * (num_tokens, top_k), fc1 weights (num_experts, 2*inter, hidden) holding gate then up rows, fc2
 * weights (num_experts, hidden, inter), hidden and inter multiples of 128).
 * ------------------------------------------------------------------------------------------- */

/*
 * Group the (token, slot) entries of topk_ids by expert into the contiguous grouped layout (the
 * m_indices of the MATE FlashInfer-API page's group_deepgemm_fp8_nt_groupwise, section "GEMM").
 *   topk_ids      (num_tokens, top_k) int32 expert ids in [0, num_experts); other values are
 *                 dropped (routed nowhere)
 *   m_indices     (m_alloc,) int32 out: expert e owns rows [off_e, off_e + ceil(c_e/128)*128) in
 *                 expert order (off_0 = 0), where c_e is its entry count; the first c_e rows hold
 *                 its entries in ascending (token, slot) order, the rest and every row past the
 *                 last region are -1
 *   src_token     (m_alloc,) int32 out: token of each row, -1 for padding
 *   row_of_entry  (num_tokens, top_k) int32 out: row of each entry, -1 if the entry was dropped
 *   workspace     device scratch of at least fp8_moe_permutation_workspace_size(num_tokens, top_k,
 *                 num_experts) bytes, 4-byte aligned (may be NULL when that size is 0); it holds
 *                 per-chunk expert counts between the call's kernels, needs no initialisation, and
 *                 must not be used by another call until this one has finished on `stream`
 * m_alloc must be at least num_tokens*top_k + num_experts*127 (rounded up to 128) so that every
 * routing fits; it must be a multiple of 128. num_experts <= 1024. Deterministic; the work is linear
 * in num_tokens*top_k (three kernels: per-chunk counts, one scan, per-chunk placement).
 */
FP8G_API int64_t fp8_moe_permutation_workspace_size(int64_t num_tokens, int64_t top_k, int64_t num_experts);
FP8G_API fp8g_status_t fp8_moe_build_permutation(const int32_t* topk_ids, int64_t num_tokens,
                                        int64_t top_k, int64_t num_experts, int64_t m_alloc,
                                        int32_t* m_indices, int32_t* src_token,
                                        int32_t* row_of_entry, void* workspace, int64_t workspace_bytes,
                                        void* stream);

/*
 * fp8_moe_build_permutation without a workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). Same
 * arguments, result and errors as fp8_moe_build_permutation, except that the per-chunk counts live in
 * the library's own device array of 4 MiB (1048576 int32), one copy per device, held until the process
 * ends. Sizes whose counts do not fit -- ceil(num_tokens*top_k / 1024) * num_experts > 1048576, e.g.
 * more than 16.7 M entries over 64 experts or 1 M entries over 1024 experts -- return
 * FP8G_INVALID_ARGUMENT. The call allocates nothing and needs no initialisation of the array (every
 * count it reads is written earlier in the same call). Calls that overlap on one device (on different
 * streams, or from different threads, before the previous one has finished) share that array and race.
 */
FP8G_API fp8g_status_t fp8_moe_build_permutation_noalloc(const int32_t* topk_ids, int64_t num_tokens,
                                                         int64_t top_k, int64_t num_experts, int64_t m_alloc,
                                                         int32_t* m_indices, int32_t* src_token,
                                                         int32_t* row_of_entry, void* stream);

/*
 * Quantise BF16 token rows per 1x128 block into the permuted layout:
 *   for every row r with s = src_token[r] >= 0 and every 128-column block c of x[s]:
 *     scale[r][c] = amax / 448 (FP32 IEEE division; 1 when the block is all zero)
 *     a_out[r][c*128 + t] = E4M3_RNE(x[s][c*128 + t] / scale[r][c])
 *   x        (num_tokens, hidden) BF16
 *   a_out    (m_alloc, hidden) E4M3 out; a_scale_out (m_alloc, hidden/128) FP32 out (K-major)
 * Rows with src_token = -1 are not written. src_token may be null: row r then quantises token r
 * (m_alloc <= num_tokens), which, with fp8_group_gemm_contiguous_gather, replaces the gathered
 * copy of the tokens by one quantised copy read through src_token.
 */
FP8G_API fp8g_status_t fp8_moe_gather_quant(const void* x, const int32_t* src_token, int64_t num_tokens,
                                   int64_t hidden, int64_t m_alloc, void* a_out,
                                   float* a_scale_out, void* stream);

/*
 * h = silu(y[:, :inter]) * y[:, inter:] in FP32 (silu(g) = g / (1 + exp(-g))), then the 1x128
 * quantisation above applied to h.
 *   y        (rows, 2*inter) BF16 (the fc1 output: gate columns, then up columns)
 *   m_indices (rows,) int32; rows with m_indices < 0 are skipped (not written)
 *   a_out    (rows, inter) E4M3 out; a_scale_out (rows, inter/128) FP32 out (K-major)
 */
FP8G_API fp8g_status_t fp8_moe_silu_mul_quant(const void* y, const int32_t* m_indices, int64_t rows,
                                     int64_t inter, void* a_out, float* a_scale_out,
                                     void* stream);

/*
 * The expert FFN's fc1 and its activation in one pass: the bytes fp8_group_gemm_contiguous_gather
 * (a_rows non-null) or fp8_group_gemm_contiguous (a_rows null) would write to y = fc1 output
 * (BF16, gate columns then up columns) followed by fp8_moe_silu_mul_quant(y), bit for bit, without
 * writing y (flashinfer-rs README, section "API Example: Fused MoE FP8 (cudarc)": the fused FP8
 * MoE; the GEMM itself is the contiguous form of the MATE FlashInfer-API page, section "GEMM").
 *   a, a_scale, a_rows_total, a_rows   as fp8_group_gemm_contiguous_gather (a_rows may be null:
 *                                      then a has m rows)
 *   w1          (num_experts, 2*inter, hidden) E4M3, gate rows then up rows; w1_scale FP32
 *               (num_experts, 2*inter/128, hidden/128) K-major or (num_experts, hidden/128,
 *               2*inter/128) MN-major (the same mode as a_scale)
 *   m_indices   (m,) int32, 128-row-aligned expert regions, -1 padding
 *   q_out       (m, inter) E4M3 out; q_scale_out (m, inter/128) FP32 out (K-major); rows with
 *               m_indices < 0 are not written
 * inter must be a multiple of 128, hidden of 128.
 */
FP8G_API fp8g_status_t fp8_moe_fc1_silu_quant(const void* a, const float* a_scale, int64_t a_rows_total,
                                     const int32_t* a_rows, const void* w1, const float* w1_scale,
                                     const int32_t* m_indices, void* q_out, float* q_scale_out,
                                     int64_t m, int64_t inter, int64_t hidden, int64_t num_experts,
                                     int32_t scale_major, int32_t gran_m, int32_t gran_n,
                                     int32_t gran_k, void* stream);

/*
 * out[t] = round( sum_s w[t][s] * y[row_of_entry[t][s]] ), summed in FP32 in slot order, rounded to
 * BF16 or FP16 (out_dtype); entries with row_of_entry = -1 contribute nothing.
 *   y             (m_alloc, hidden) BF16 (the fc2 output)
 *   row_of_entry  (num_tokens, top_k) int32
 *   topk_weights  (num_tokens, top_k) FP32 routing weights, or null for weight 1 (the per-tensor
 *                 fused-MoE call of the flashinfer-rs README takes no routing weights)
 *   out           (num_tokens, hidden) BF16 or FP16, fully written
 */
FP8G_API fp8g_status_t fp8_moe_combine(const void* y, const int32_t* row_of_entry,
                              const float* topk_weights, int64_t num_tokens, int64_t top_k,
                              int64_t hidden, int64_t m_alloc, void* out, int32_t out_dtype,
                              void* stream);

/* ---------------------------------------------------------------------------------------------
 * Per-tensor FP8 expert FFN (flashinfer-rs README, section "API Example: Fused MoE FP8 (cudarc)",
 * per-tensor FP8 mode): FP8 tokens, one dequantisation scale per expert and GEMM, one (or one per
 * expert) quantisation scale for fc2's input. The permutation and the combine are the calls above.
 * ------------------------------------------------------------------------------------------- */

/*
 * out[i] = round( b_dequant[e] * (a[r_i] @ b[e].T) ) for every row with e = m_indices[i] >= 0,
 * where r_i = a_rows[i] (a_rows non-null) or i; the sum is FP32 over all of k, one multiply by the
 * expert's scale, BF16 or FP16 output (out_dtype). Rows with m_indices < 0 are not written.
 *   a (a_rows_total, k) E4M3 (a_rows_total = m without a_rows); b (num_groups, n, k) E4M3;
 *   b_dequant (num_groups,) FP32; m_indices (m,) int32 in 128-row-aligned regions; out (m, n)
 * m, n and k are multiples of 128.
 */
FP8G_API fp8g_status_t fp8_group_gemm_contiguous_per_tensor(const void* a, int64_t a_rows_total,
                                                   const int32_t* a_rows, const void* b,
                                                   const float* b_dequant, const int32_t* m_indices,
                                                   void* out, int32_t out_dtype, int64_t m, int64_t n,
                                                   int64_t k, int64_t num_groups, void* stream);

/*
 * fc1 of the per-tensor FFN with the activation and fc2's input quantisation in its epilogue:
 *   g, u = fc1_dequant[e] * (a[r_i] @ w1[e][0:inter].T),  fc1_dequant[e] * (a[r_i] @ w1[e][inter:].T)
 *   q_out[i] = E4M3_RNE(saturate(silu(g) * u * fc2_quant[e or 0]))     (all FP32; +-448, NaN kept)
 * fc2_quant holds one value (fc2_quant_per_expert = 0) or one per expert (= 1): a multiplicative
 * quantisation scale, the convention of the MATE page's quant_scale (section "Attention",
 * mla_rope_quantize_fp8). Rows with m_indices < 0 are not written.
 *   a (a_rows_total, hidden) E4M3 tokens; w1 (num_experts, 2*inter, hidden) E4M3, gate then up;
 *   fc1_dequant (num_experts,) FP32; q_out (m, inter) E4M3
 * inter and hidden are multiples of 128; m of 128.
 */
FP8G_API fp8g_status_t fp8_moe_fc1_silu_quant_per_tensor(const void* a, int64_t a_rows_total,
                                                 const int32_t* a_rows, const void* w1,
                                                 const float* fc1_dequant, const float* fc2_quant,
                                                 int32_t fc2_quant_per_expert,
                                                 const int32_t* m_indices, void* q_out, int64_t m,
                                                 int64_t inter, int64_t hidden,
                                                 int64_t num_experts, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8G_H_ */
