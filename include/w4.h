/*
 * w4.h -- C ABI of the MI355X (gfx950) 4-bit-weight mixed-precision GEMM library.
 *
 * The library computes out = A . dequant(W)^T for a 4-bit weight W [N, K] and
 * activations A [M, K]:
 *
 *   W4A8  : int4 weights with per-channel or group-128 scales; activations
 *           quantised dynamically per token (row) to int8 or fp8-e4m3
 *           (QQQ-style; "[Kernel] Initial Machete W4A8 support + Refactors",
 *           summary; "support W4A8 Marlin kernel", summary).
 *   W4A16 : unsigned 4-bit weights with group scales and raw zero-points,
 *           fp16/bf16 activations ("...mixed_precision.rdna_hybrid_w4a16"
 *           API page, triton_w4a16_skinny_fmt_gemm docstring).
 *
 * Entry points: w4_prepack_B (and w4_prepack_B_from_exllama), the activation
 * quantisers (w4_quant_act_per_token, w4_quant_act_per_tensor,
 * w4_rmsnorm_quant_per_token), the GEMMs (w4a8_gemm, w4a8_gemm_zp,
 * w4a8_gemm_quant_fused, w4a8_gemm_no_alloc, w4a16_gemm,
 * w4a16_gemm_prescaled_zeros), their
 * verification variants
 * (w4a8_gemm_partials, w4a16_gemm_partials), and the planning helpers
 * (w4_gemm_workspace_bytes, w4_gemm_plan, w4_schedule_add / _clear,
 * w4_set_option / w4_get_option).
 *
 * General conventions (every entry point):
 *   - All pointers named as device pointers must point to device memory of
 *     the current HIP device; all arrays are dense and row-major.  Every device
 *     pointer must be 16-byte aligned.
 *   - The caller owns every buffer.  The library never allocates, frees or
 *     synchronises; it keeps no per-call state and may be called concurrently
 *     from several threads (on distinct output/workspace buffers; the one
 *     exception is w4a8_gemm_no_alloc, whose workspace is a buffer built into
 *     the library and shared by every call on a GPU).  The
 *     tuning options and the run-time schedule entries are process-wide.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued on it and the call returns without waiting.
 *   - Arguments are validated on the host before anything is enqueued.  On a
 *     validation error nothing is enqueued and a non-zero w4_status is
 *     returned; w4_last_error() then holds a message (thread-local).
 *   - Errors of the HIP runtime while enqueueing return W4_E_HIP.  Faults of
 *     enqueued work surface at the caller's next synchronisation, as usual
 *     for HIP.
 *   - M = 0 is valid and enqueues nothing.
 *   - Size limits of the GEMMs (and of w4_gemm_plan / w4_gemm_workspace_bytes),
 *     from their 32-bit buffer offsets: K <= 2^22, and at most 2^29 - 4
 *     weight scales (N x K / group_size, or N per channel); larger problems
 *     return W4_E_SHAPE.  Per-channel int8 also needs K <= 131072 (its int32
 *     accumulators).
 */
#ifndef W4_H_
#define W4_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define W4_API __attribute__((visibility("default")))
#else
#define W4_API
#endif

#define W4_ABI_VERSION 1
#define W4_LAYOUT_VERSION 1 /* PB-v1 */

typedef enum w4_status {
  W4_OK = 0,
  W4_E_NULL = 1,        /* a required pointer is NULL                        */
  W4_E_SHAPE = 2,       /* a size is negative or violates N%16, K%128, ...   */
  W4_E_DTYPE = 3,       /* unsupported dtype / wtype / operand combination   */
  W4_E_ALIGN = 4,       /* a device pointer is not 16-byte aligned           */
  W4_E_GROUP = 5,       /* group_size not in {K, -1, 128} (W4A16 also 64, 32) or does not divide K */
  W4_E_WORKSPACE = 6,   /* workspace missing or smaller than required        */
  W4_E_UNSUPPORTED = 7, /* valid request outside what this version implements */
  W4_E_HIP = 8          /* the HIP runtime returned an error                 */
} w4_status;

typedef enum w4_dtype {
  W4_F16 = 0,
  W4_BF16 = 1,
  W4_F32 = 2,
  W4_I8 = 3,
  W4_FP8_E4M3 = 4, /* OCP e4m3fn: bias 7, no infinities, max 448 */
  W4_I32 = 5
} w4_dtype;

/* How a 4-bit code c (0..15) stored in the weight is read. */
typedef enum w4_wtype {
  W4_INT4 = 0,    /* two's complement nibble, value in [-8, 7]                  */
  W4_UINT4 = 1,   /* value c in [0, 15]; W4A16 with explicit zero-points        */
  W4_UINT4B8 = 2  /* value c - 8 ("uint4b8" of the Machete W4A8 PR; the W4A16
                     kernel page subtracts the same constant 8 when no
                     zero-points are given)                                     */
} w4_wtype;

/* The MFMA operand class a prepacked weight is laid out for. */
typedef enum w4_operand {
  W4_OPERAND_I8 = 0, /* consumed by w4a8_gemm (int8 and fp8 activations) */
  W4_OPERAND_F16 = 1 /* consumed by w4a16_gemm (fp16 and bf16 activations) */
} w4_operand;

W4_API int w4_abi_version(void);
W4_API int w4_layout_version(void);
W4_API const char* w4_status_string(int status);
/* Detail of the last error returned on this thread ("" if none). */
W4_API const char* w4_last_error(void);

/* ---------------------------------------------------------------------------
 * Weight prepack.
 *
 * Follows the Machete README, "API": the weight is reordered once, before any
 * GEMM call, into a layout that matches the matrix-core operand so that the
 * GEMM reads it with wide loads; and the Machete W4A8 PR summary: the prepack
 * is a pure data shuffle, so one kernel serves every 4-bit weight type.
 *
 * w_logical : device, [N][K/2] bytes; byte (n, j) holds the code of k = 2j in
 *             bits 0..3 and of k = 2j+1 in bits 4..7.
 * w_packed  : device, w4_prepack_B_bytes(N, K) bytes, written entirely.
 *             PB-v1 layout: 16 (n) x 128 (k) blocks of 1 KiB, n-block major;
 *             inside a block lane l = 16*kq + (n%16) holds k in
 *             [32 kq, 32 kq + 32) as four little-endian 32-bit words, word kw
 *             holding k in [8 kw, 8 kw + 8) of that range.  The nibble of
 *             k-offset j (0..7) sits at bit 8j (j < 4) / 8(j-4)+4 (j >= 4) for
 *             W4_OPERAND_I8 and at bit 4(j/2) + 16(j%2) (the ExLlama order of
 *             the W4A16 page) for W4_OPERAND_F16.
 * Requires N % 16 == 0, K % 128 == 0, N, K > 0, N * K < 2^43.  Input and
 * output must not overlap.  Errors: W4_E_NULL, W4_E_SHAPE, W4_E_DTYPE (operand), W4_E_ALIGN,
 * W4_E_HIP.
 * ------------------------------------------------------------------------- */
W4_API size_t w4_prepack_B_bytes(int64_t N, int64_t K);
W4_API int w4_prepack_B(const void* w_logical, void* w_packed, int64_t N, int64_t K, int operand,
                 void* stream);

/* ---------------------------------------------------------------------------
 * Prepack from ExLlama-shuffled int32 words.
 *
 * vLLM API page "...mixed_precision.rdna_hybrid_w4a16", docstring of
 * _triton_w4a16_skinny_fmt_kernel: the weight as [N][K/8] int32 words, each
 * holding 8 consecutive k (k = 8 w + j) with k-offset j at bit
 * (j / 2) * 4 + (j % 2) * 16.  Writes the same PB-v1 bytes as w4_prepack_B
 * of the equivalent logical weight, in one pass (for W4_OPERAND_F16 the
 * words move unchanged: the two orders coincide).  Codes are taken as they
 * are (raw 4-bit values; their signedness is chosen by the GEMM's wtype).
 *
 * w_words  : device, [N][K/8] 32-bit words, N*K/2 bytes, 16-byte aligned.
 * w_packed : device, N*K/2 bytes, 16-byte aligned, not overlapping w_words.
 * Requirements and errors as w4_prepack_B.
 * ------------------------------------------------------------------------- */
W4_API int w4_prepack_B_from_exllama(const void* w_words, void* w_packed, int64_t N, int64_t K, int operand,
                              void* stream);

/* ---------------------------------------------------------------------------
 * Dynamic per-token activation quantisation.
 *
 * Follows "[ Kernel ] Enable Dynamic Per Token fp8", summary and review
 * discussion: one scale per row (token), computed at run time.  Per row m:
 *   amax = max_k |x[m,k]|;  s[m] = fp32(amax / qmax)   (qmax 127 int8, 448 fp8)
 *   q = round-half-even(fp32(x / s[m])) clamped to [-127, 127]   (int8)
 *   q = e4m3fn(round-half-even(clamp(fp32(x / s[m]), -448, 448)))   (fp8)
 * with a correctly rounded fp32 division.  A row of zeros gets s = 0, q = 0.
 *
 * x       : device, [M][K] of x_dtype (W4_F16 or W4_BF16); finite values.
 * xq      : device, [M][K] of q_dtype (W4_I8, or W4_FP8_E4M3 as raw bytes).
 * scales  : device, [M] fp32.
 * Requires 0 < K <= 2^29, K % 8 == 0, M >= 0.  Errors: W4_E_NULL, W4_E_SHAPE,
 * W4_E_DTYPE, W4_E_ALIGN, W4_E_HIP.
 * ------------------------------------------------------------------------- */
W4_API int w4_quant_act_per_token(const void* x, int x_dtype, void* xq, int q_dtype, float* scales,
                           int64_t M, int64_t K, void* stream);

/* ---------------------------------------------------------------------------
 * Dynamic per-tensor activation quantisation.
 *
 * "[ Kernel ] Enable Dynamic Per Token fp8", results and review discussion:
 * the per-tensor alternative to per-token scales, one scale for the whole
 * [M][K] tensor computed at run time:
 *   amax = max_{m,k} |x[m,k]|;  s = fp32(amax / qmax)   (qmax 127 int8, 448 fp8)
 *   q = as w4_quant_act_per_token, with s in place of every row's s[m]
 * s is written to each of scales[0..M), so that the GEMMs, which take one
 * scale per row, consume the result unchanged.  An all-zero tensor gets
 * s = 0, q = 0.  x is read twice (its row maxima, then the codes): three
 * launches on the stream, with scales holding the row maxima in between.
 *
 * Arguments, requirements and errors as w4_quant_act_per_token.
 * ------------------------------------------------------------------------- */
W4_API int w4_quant_act_per_tensor(const void* x, int x_dtype, void* xq, int q_dtype, float* scales,
                            int64_t M, int64_t K, void* stream);

/* ---------------------------------------------------------------------------
 * Fused RMSNorm + dynamic per-token activation quantisation.
 *
 * "[ Kernel ] Enable Dynamic Per Token fp8", review discussion: per-token
 * scales make it easy to fuse the RMSNorm before a linear layer with the
 * quantisation of its output.  The result is exactly that of an RMSNorm whose
 * output is in x_dtype, followed by w4_quant_act_per_token.  Per row m:
 *   ss   = sum_k x[m,k]^2, exact, rounded once to fp64 (no dependence on
 *          summation order)
 *   r    = fp32( 1 / sqrt( ss / K + eps ) )        (fp64 arithmetic)
 *   y    = x_dtype( fp32( fp32(x[m,k] * r) * gamma[k] ) )   (round to nearest even)
 *   xq, scales = w4_quant_act_per_token(y)
 * x and gamma are read once; y is never stored.
 *
 * x       : device, [M][K] of x_dtype (W4_F16 or W4_BF16); finite values.
 * gamma   : device, [K] of x_dtype; every y must be finite in x_dtype.
 * eps     : positive, finite.
 * xq      : device, [M][K] of q_dtype (W4_I8, or W4_FP8_E4M3 as raw bytes).
 * scales  : device, [M] fp32.
 * Requires 0 < K <= 2^29, K % 8 == 0, M >= 0; x, gamma, xq 16-byte aligned.
 * Errors: W4_E_NULL, W4_E_SHAPE (shape or eps), W4_E_DTYPE, W4_E_ALIGN, W4_E_HIP.
 * ------------------------------------------------------------------------- */
W4_API int w4_rmsnorm_quant_per_token(const void* x, int x_dtype, const void* gamma, float eps, void* xq,
                               int q_dtype, float* scales, int64_t M, int64_t K, void* stream);

/* ---------------------------------------------------------------------------
 * Workspace.
 *
 * Some (M, N, K) are split along K across workgroups; the partial results go
 * through a caller-provided workspace.  w4_gemm_workspace_bytes returns the
 * bytes the GEMM entry points need for this problem (0 when no split is
 * used).  The workspace needs no initialisation and is not used after the
 * call's work has finished; concurrent calls need distinct workspaces.
 * a_dtype: the activation dtype of the GEMM (W4_I8, W4_FP8_E4M3, W4_F16,
 * W4_BF16).  Returns 0 for invalid arguments.
 * ------------------------------------------------------------------------- */
W4_API size_t w4_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t group_size, int a_dtype);

/* ---------------------------------------------------------------------------
 * W4A8 GEMM.
 *
 * Follows the Machete README, "Overview" (out = activations times the
 * dequantised weight, with the weight [N, K] and the output [M, N]), the
 * Machete W4A8 PR summary (QQQ-style W4A8 with int8 or fp8 activations) and
 * "support W4A8 Marlin kernel" (int4 weights, symmetric, per-channel or
 * per-group scales):
 *
 *   out[m,n] = RNE_out( s_a[m] * sum_g s_w[n,g] * sum_{k in g} a[m,k] * w[n,k]
 *                       + bias[n] )
 *
 * where a is the int8 code, or the fp8 value, of the quantised activation.
 *
 * aq        : device, [M][K] int8 codes or e4m3fn bytes (a_dtype W4_I8 / W4_FP8_E4M3).
 * a_scales  : device, [M] fp32 per-token scales.
 * b_packed  : device, PB-v1 bytes from w4_prepack_B(..., W4_OPERAND_I8).
 * wtype     : W4_INT4 or W4_UINT4B8.
 * b_scales  : device; [N] when group_size is K or -1 (per channel), else
 *             [N][K/group_size]; dtype s_dtype (W4_F32, W4_F16 or W4_BF16).
 * group_size: K, -1 (= K) or 128.
 * bias      : device, [N] of out_dtype, or NULL.
 * out       : device, [M][N] of out_dtype (W4_F16 or W4_BF16).
 * workspace : device, at least w4_gemm_workspace_bytes(M, N, K, group_size,
 *             a_dtype) bytes (may be NULL when that is 0).
 * Requires N % 16 == 0, K % 128 == 0, N, K > 0, M >= 0.  Errors: W4_E_NULL,
 * W4_E_SHAPE, W4_E_DTYPE, W4_E_ALIGN, W4_E_GROUP, W4_E_WORKSPACE, W4_E_HIP.
 * ------------------------------------------------------------------------- */
W4_API int w4a8_gemm(const void* aq, int a_dtype, const float* a_scales, const void* b_packed,
              int wtype, const void* b_scales, int s_dtype, int64_t group_size,
              const void* bias, void* out, int out_dtype, int64_t M, int64_t N, int64_t K,
              void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * W4A8 GEMM that allocates nothing.
 *
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): w4a8_gemm
 * with the split-K workspace taken from a buffer built into the library, one
 * 64 MiB copy per GPU, held until the process ends.  Same arguments, results
 * and errors as w4a8_gemm without workspace / workspace_bytes; problems
 * whose workspace (w4_gemm_workspace_bytes) exceeds 64 MiB return
 * W4_E_WORKSPACE (use w4a8_gemm with a workspace of your own).  No
 * allocation, free or memset.  Every call on a GPU shares that GPU's buffer:
 * calls that overlap on one GPU (other streams, other threads) race.
 * ------------------------------------------------------------------------- */
W4_API int w4a8_gemm_no_alloc(const void* aq, int a_dtype, const float* a_scales, const void* b_packed,
                              int wtype, const void* b_scales, int s_dtype, int64_t group_size,
                              const void* bias, void* out, int out_dtype, int64_t M, int64_t N, int64_t K,
                              void* stream);

/* ---------------------------------------------------------------------------
 * W4A16 GEMM with pre-scaled zero-points.
 *
 * Machete README, "Overview": the dequantised weight is the code times its
 * scale minus a zero term to which the scale is already applied (so that one
 * FMA dequantises):
 *
 *   out[m,n] = RNE_a( sum_k a[m,k] * (c[n,k] * s[n,g] - zs[n,g]) + bias[n] )
 *
 * c are raw uint4 codes; s and zs [N][K/128] are in a_dtype (any values).
 * The kernels take sum(a c) per group from the MFMAs and zs * sum(a) from a
 * second MFMA with a ones-operand, both in fp32.
 * group_size: 128 (K > 128).  Other arguments as w4a16_gemm (the workspace is
 * the one w4_gemm_workspace_bytes reports for a_dtype and group size 128).
 * Errors as w4a16_gemm.
 * ------------------------------------------------------------------------- */
W4_API int w4a16_gemm_prescaled_zeros(const void* a, int a_dtype, const void* b_packed, const void* scales,
                                      const void* zeros_scaled, int64_t group_size, const void* bias, void* out,
                                      int64_t M, int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
                                      void* stream);

/* ---------------------------------------------------------------------------
 * W4A8 GEMM with the per-token quantisation fused into the small-M kernel.
 *
 * "[ Kernel ] Enable Dynamic Per Token fp8", review discussion: per-token
 * scales make it easy to fuse the quantisation with its neighbours.  Returns
 * what w4_quant_act_per_token followed by w4a8_gemm returns (the same codes,
 * scales and output bits), in one launch: every workgroup of the small-M
 * kernel quantises the M rows into its LDS before its main loop.
 *
 * x           : device, [M][K] of x_dtype (W4_F16 or W4_BF16), finite values.
 * q_dtype     : W4_I8 or W4_FP8_E4M3 (the activation codes).
 * a_scales_out: device, [M] fp32, receives the per-token scales, or NULL.
 * Other arguments as w4a8_gemm.  Supported where the problem takes the
 * small-M kernel (M <= 16) and the M*K codes fit its LDS (M*K codes plus the
 * scale tables and the reduction buffer at most 64 KiB); otherwise
 * W4_E_UNSUPPORTED, and the two calls are the way.
 * No workspace.  Errors as w4a8_gemm, plus W4_E_UNSUPPORTED.
 * ------------------------------------------------------------------------- */
W4_API int w4a8_gemm_quant_fused(const void* x, int x_dtype, int q_dtype, const void* b_packed, int wtype,
                                 const void* b_scales, int s_dtype, int64_t group_size, const void* bias,
                                 void* out, int out_dtype, int64_t M, int64_t N, int64_t K, float* a_scales_out,
                                 void* stream);

/* ---------------------------------------------------------------------------
 * Asymmetric W4A8 GEMM (weights with zero-points).
 *
 * "support W4A8 Marlin kernel", limitations comment: QQQ's W4A8 handles
 * symmetric weights only.  This entry point takes raw uint4 codes u with an
 * integer zero-point per (column, group), as the W4A16 API page does for
 * W4A16 (raw zero-points, subtracted before the scale):
 *
 *   out[m,n] = RNE_out( s_a[m] * sum_g s_w[n,g] * sum_{k in g} a[m,k] * (u[n,k] - z[n,g])
 *                       + bias[n] )
 *
 * with int8 activation codes a.  The inner sums are exact (int32).
 *
 * zeros   : device, [N][K/group_size] (per channel: [N]) of z_dtype (W4_F16,
 *           W4_BF16 or W4_F32), integer values 0..15.
 * b_packed: PB-v1 bytes of the raw codes (w4_prepack_B, W4_OPERAND_I8).
 * Other arguments as w4a8_gemm with a_dtype W4_I8.  The workspace is the
 * one w4_gemm_workspace_bytes(M, N, K, group_size, W4_I8) reports.  Per
 * channel needs K <= 65536.  Errors as w4a8_gemm.
 * ------------------------------------------------------------------------- */
W4_API int w4a8_gemm_zp(const void* aq, const float* a_scales, const void* b_packed, const void* b_scales,
                        int s_dtype, const void* zeros, int z_dtype, int64_t group_size, const void* bias,
                        void* out, int out_dtype, int64_t M, int64_t N, int64_t K, void* workspace,
                        size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * W4A16 GEMM.
 *
 * Follows the "...mixed_precision.rdna_hybrid_w4a16" API page
 * (triton_w4a16_skinny_fmt_gemm and its kernel's docstring): the weight code
 * minus a raw per-group zero-point, times a per-group scale, with scales and
 * zero-points [N, K/G] in the activation dtype, the constant 8 subtracted
 * when no zero-points are given, and the output in the activation dtype:
 *
 *   out[m,n] = RNE_a( sum_g s[n,g] * sum_{k in g} a[m,k] * (c[n,k] - z[n,g]) + bias[n] )
 *
 * a         : device, [M][K] of a_dtype (W4_F16 or W4_BF16).
 * b_packed  : device, PB-v1 bytes from w4_prepack_B(..., W4_OPERAND_F16).
 * wtype     : W4_UINT4 (zeros given or NULL) or W4_UINT4B8 (zeros must be NULL).
 * scales    : device, [N][K/group_size] of a_dtype.
 * zeros     : device, [N][K/group_size] of a_dtype, integer values 0..15, or
 *             NULL for z = 8.
 * group_size: K, -1 (= K), 128, 64 or 32.  Groups smaller than the kernels'
 *             128-deep K block follow the W4A16 API page's kernel, which
 *             narrows its K tile to the group size: each block then holds 2
 *             or 4 groups, each with its own scale and zero-point.
 * bias      : device, [N] of a_dtype, or NULL.
 * out       : device, [M][N] of a_dtype.
 * workspace : as for w4a8_gemm.
 * Requires N % 16 == 0, K % 128 == 0.  Errors as for w4a8_gemm.
 * ------------------------------------------------------------------------- */
W4_API int w4a16_gemm(const void* a, int a_dtype, const void* b_packed, int wtype, const void* scales,
               const void* zeros, int64_t group_size, const void* bias, void* out, int64_t M,
               int64_t N, int64_t K, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Group partial sums (verification entry points).
 *
 * Run the same kernels and main loops as w4a8_gemm / w4a16_gemm on the same
 * arguments, but instead of the scale epilogue store, for the output window
 * rows [m0, m1) x columns [n0, n1), the per-group dot products
 *   W4A8 int8 : P[g][m-m0][n-n0] = sum_{k in g} a[m,k] w[n,k]   as int32
 *   W4A8 fp8  : the same sum of fp8 values times w, as fp32
 *   W4A16     : sum_{k in g} a[m,k] (c[n,k] - z[n,g]), as fp32
 * into `partials` (device, G * (m1-m0) * (n1-n0) elements, G = K/group_size).
 * Requires 0 <= m0 <= m1 <= M, 0 <= n0 <= n1 <= N.  The kernel and K split
 * are the ones the GEMM would use for the same problem (including the
 * "force_path" / "splitk" overrides below), and so is the workspace size.
 * No output, scales or bias are touched.
 * ------------------------------------------------------------------------- */
W4_API int w4a8_gemm_partials(const void* aq, int a_dtype, const void* b_packed, int wtype,
                       int64_t group_size, int64_t M, int64_t N, int64_t K, int64_t m0,
                       int64_t m1, int64_t n0, int64_t n1, void* partials, void* workspace,
                       size_t workspace_bytes, void* stream);
W4_API int w4a16_gemm_partials(const void* a, int a_dtype, const void* b_packed, int wtype,
                        const void* zeros, int64_t group_size, int64_t M, int64_t N, int64_t K,
                        int64_t m0, int64_t m1, int64_t n0, int64_t n1, void* partials,
                        void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Tuning / test overrides (process-wide, not synchronised with running
 * calls; set them before issuing work).
 *   "force_path" : 0 = automatic, 1 = small-M kernel, 2 = tiled kernel,
 *                  3 = streaming kernel (int8 / fp8 activations, symmetric
 *                  weights), 4 = ping-pong kernel (symmetric int8 per channel)
 *   "splitk"     : 0 = automatic, else the number of K splits (tiled and
 *                  streaming kernels, 1..64) or waves splitting K (small-M
 *                  kernel: 1..16 for ungrouped int8 / fp8, 1..8 otherwise)
 *   "skinny_strips": 0 = automatic, else 16-column blocks per wave: 1 or 2
 *                  strips of the small-M kernel (2 needs N % 32 == 0); 2 or 4
 *                  for the tiled and streaming kernels with int8 / fp8
 *                  activations (tiles of 128 or 256 columns; 16-bit
 *                  activations take 2; 128-row tiles of 256 columns exist for
 *                  symmetric int8 per channel only, and not in the streaming
 *                  kernel)
 *   "tiled_bm"   : 0 = automatic, 64 or 128 rows per tile of the tiled kernel
 *                  (128 only for int8 and fp8 activations; by default its tile
 *                  is 128 x 256 for int8 per channel, 128 x 128 otherwise), 32,
 *                  64 or 128 for the streaming kernel, 128 or 256 for the
 *                  ping-pong kernel (tiles of 256 columns; 256 alone selects
 *                  that kernel)
 *   "norm_exact_sum": 1 = w4_rmsnorm_quant_per_token always re-sums the squares
 *                  with error-free pair arithmetic (the path it otherwise takes
 *                  only when the fast sum cannot decide r); same results
 *   "schedule_table": 1 (default) = consult the schedule table below; 0 = the
 *                  heuristic alone
 * When any of force_path, splitk, skinny_strips or tiled_bm is nonzero, those
 * fields are forced and the schedule table is not consulted.
 * Returns W4_OK, or W4_E_UNSUPPORTED for an unknown key / W4_E_SHAPE for an
 * out-of-range value.
 * ------------------------------------------------------------------------- */
W4_API int w4_set_option(const char* key, int64_t value);
W4_API int64_t w4_get_option(const char* key);

/* ---------------------------------------------------------------------------
 * Schedule table.
 *
 * [Machete README] *Code generation*: each type pair carries a default
 * heuristic that maps problem shapes to schedules (tile shapes and the like),
 * since no one schedule suits every shape, and a caller may name the schedule
 * instead.  Here a schedule is (path, K split, tile rows, strips per wave)
 * and the table maps (activation dtype, grouping, N, K, M range) to one.  The
 * GEMM entry points look a problem up in the run-time entries (newest first),
 * then in the built-in entries (measured on MI355X for the benchmark shapes,
 * kept only where they beat the heuristic), and otherwise use the heuristic.
 * An entry whose schedule does not fit the problem is passed over.
 *
 * w4_schedule_add registers a run-time entry: problems with this a_dtype
 * (W4_I8, W4_FP8_E4M3, W4_F16, W4_BF16), group_mode (0 = one group over K,
 * 1 = group size 128), N, K and m_lo <= M <= m_hi take path (0 = heuristic,
 * 1 = small-M, which needs m_hi <= 16, 2 = tiled, 3 = streaming,
 * 4 = ping-pong), splitk
 * (0 = heuristic, 1..64), tile_m (0, 32, 64, 128 or 256) and strips (0, 1, 2 or
 * 4; the meanings of the options above).  This is also the
 * per-shape override of the heuristic.  The workspace size the GEMM needs
 * follows the schedule in force (w4_gemm_workspace_bytes and w4_gemm_plan
 * consult the same table).  Errors: W4_E_DTYPE, W4_E_SHAPE.
 * w4_schedule_clear removes every run-time entry.
 * Both take a lock; calls racing with GEMM launches on other threads are safe.
 * ------------------------------------------------------------------------- */
W4_API int w4_schedule_add(int a_dtype, int group_mode, int64_t N, int64_t K, int64_t m_lo, int64_t m_hi,
                           int path, int splitk, int tile_m, int strips);
W4_API int w4_schedule_clear(void);

/* The kernel the GEMM entry points would choose for this problem under the
 * current options, for logging and tests: *path (1 = small-M, 2 = tiled,
 * 3 = streaming, 4 = ping-pong), its
 * K split (*splitk), and the output tile one workgroup computes (*tile_m rows
 * x *tile_n columns; for the small-M kernel tile_m is 16).  Any out pointer
 * may be NULL.  Errors as for the GEMM's shape checks. */
W4_API int w4_gemm_plan(int64_t M, int64_t N, int64_t K, int64_t group_size, int a_dtype, int* path,
                        int* splitk, int* tile_m, int* tile_n);

#ifdef __cplusplus
}
#endif

#endif /* W4_H_ */
