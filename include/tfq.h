/*
 * tfq.h -- C ABI of the MI355X (gfx950) W8A8 scaled-quantized Linear.
 *
 * The method (web pages, cited by title and section):
 *   - TeleFuser "Quantization", "Core ideas": symmetric INT8,
 *     s = max|x| / 127, q = clamp(round(x / s), -128, 127), x_hat = s q; one
 *     scale may cover a tensor, an output channel, a token or a block.
 *   - TeleFuser "Quantization", "Scaled FP8 checkpoints: W8A8": every input
 *     row quantised to E4M3FN with s = max|x| / max(E4M3FN),
 *     q = cast_E4M3FN(clamp(x / s)); then a scaled GEMM back to BF16.
 *   - TeleFuser "Quantization", "tf-kernel FP8: online W8A8": activations
 *     quantised per token at each forward, weights per output channel and
 *     cached on first use, BF16 output; single GPU.
 *   - LightX2V "模型量化技术", "MiniMax-H3 FP8 FP16 累加": row-dynamic
 *     activation scale = max(abs(x)) / qmax with reduced qmax (14, 12, 7);
 *     table "量化模式", fp8-b128-deepgemm: block-symmetric FP8 weights and
 *     group-symmetric FP8 activations.
 *   - vLLM-Omni "FP8 Quantization", "Parameters": weight_block_size.
 *
 * Arithmetic contract (readings of what the pages leave open):
 *   s = RN32(amax / qmax); t = RN32(x / s) (correctly rounded division);
 *   FP8: code = E4M3FN_RNE(clamp(t, -qmax, qmax)), sign of zero kept;
 *   INT8: code = clamp(round_half_even(t), -128, 127);
 *   an all-zero row/group stores s = 0 and signed-zero codes;
 *   GEMM: y[m,n] = s_a[m] * s_b[n] * sum_k a[m,k] b[n,k] accumulated in
 *   FP32 (FP8) or exactly in INT32 (INT8), rounded once to BF16 (RNE);
 *   INT8 BF16 output is bf16(RN(RN(float(acc) * s_a[m]) * s_b[n]) [+ bias]);
 *   block mode: y = sum_kb s_a[m,kb] s_b[n/128,kb] (sum_{k in kb} a b).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the
 *     library never allocates or frees memory and keeps no pointer after a
 *     call returns.  Matrices are row-major.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued asynchronously; no call synchronises the host.
 *   - Arguments are validated on the host before any HIP call; a failed
 *     check returns a status and enqueues nothing.  Nothing throws or aborts
 *     across the ABI.  Calls are thread-safe (per-device state is set up
 *     once under a lock).
 *   - The current HIP device must be a gfx950; otherwise
 *     TFQ_ERR_UNSUPPORTED_DEVICE.  There is no fallback path.
 *   - Inputs must be finite (behaviour for NaN/Inf inputs is unspecified).
 */
#ifndef TFQ_H
#define TFQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 9: MXFP6 codes are stored group-major, [cols/128, rows, 96] */
#define TFQ_ABI_VERSION 9

typedef enum tfq_status {
    TFQ_OK = 0,
    TFQ_ERR_NULL_POINTER = 1,       /* a required pointer is NULL */
    TFQ_ERR_BAD_SHAPE = 2,          /* a size is out of range or not a multiple it must be */
    TFQ_ERR_MISALIGNED = 3,         /* a pointer or leading dimension breaks 16-byte alignment */
    TFQ_ERR_BAD_QMAX = 4,           /* qmax not finite, <= 0, too large, or not on the code grid */
    TFQ_ERR_WORKSPACE_TOO_SMALL = 5,/* fused Linear workspace smaller than required */
    TFQ_ERR_ALIAS = 6,              /* an output overlaps an input or another output */
    TFQ_ERR_UNSUPPORTED = 7,        /* an enum value or option combination that is not provided */
    TFQ_ERR_UNSUPPORTED_DEVICE = 8, /* no HIP device, or the current device is not gfx950 */
    TFQ_ERR_HIP = 9                 /* a HIP runtime call failed; see tfq_last_hip_error() */
} tfq_status;

typedef enum tfq_qtype {
    TFQ_QTYPE_E4M3FN = 0,  /* OCP FP8 E4M3FN codes (uint8), qmax on the E4M3FN grid, <= 448 */
    TFQ_QTYPE_INT8 = 1     /* symmetric INT8 codes (int8), integer qmax in [1, 127] */
} tfq_qtype;

typedef enum tfq_epilogue {
    TFQ_EPI_NONE = 0,      /* y = scaled product (+ bias) */
    TFQ_EPI_GELU_TANH = 1  /* y = gelu_tanh(scaled product (+ bias)), computed in FP32 */
} tfq_epilogue;

/*
 * Per-token (row-wise) dynamic absmax quantisation of BF16 activations.
 * TeleFuser "Quantization", "Scaled FP8 checkpoints: W8A8" (FP8 rows) and
 * "Core ideas" (INT8); LightX2V "模型量化技术", "MiniMax-H3 FP8 FP16 累加"
 * (reduced qmax); group_cols = 128 is the 1x128 token-group scaling of
 * fp8-b128-deepgemm (LightX2V, table "量化模式").
 *
 *   x_bf16    [rows, cols] BF16, row stride ld_x elements (ld_x >= cols,
 *             ld_x % 8 == 0), 16-byte aligned.
 *   qtype     TFQ_QTYPE_E4M3FN or TFQ_QTYPE_INT8; qmax as in tfq_qtype.
 *   group_cols 0 = one scale per row; 128 = one scale per 1x128 group
 *             (cols % 128 == 0).
 *   q_out     [rows, cols] codes, dense (row stride cols), 16-byte aligned.
 *   scale_out [rows] FP32, or [rows, cols/128] for group_cols = 128.
 *   rows >= 1; cols >= 16, cols % 16 == 0.
 */
tfq_status tfq_quantize_rows(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                             int32_t qtype, float qmax, int32_t group_cols, void* q_out,
                             float* scale_out, void* stream);

/*
 * Routed (gathered) per-token quantisation for a MoE layer: output row r
 * quantises row row_index[r] of x, exactly as tfq_quantize_rows would.
 * TeleFuser "Quantization", "Other quantized data paths" (LingBot-Video MoE
 * FP8: the routed activations are quantised per row); the router's token
 * order (e.g. tokens sorted by expert, a token repeated once per chosen
 * expert) is the caller's.
 *
 *   x_bf16    [src_rows, cols] BF16, row stride ld_x (as tfq_quantize_rows).
 *   row_index [rows] int32 device array, 4-byte aligned; an index outside
 *             [0, src_rows) quantises a row of zeros (codes 0, scale 0).
 *   q_out [rows, cols], scale_out [rows] or [rows, cols/128]: as
 *   tfq_quantize_rows.  rows, src_rows >= 1.
 */
tfq_status tfq_quantize_rows_gather(const void* x_bf16, int64_t src_rows, int64_t cols,
                                    int64_t ld_x, const int32_t* row_index, int64_t rows,
                                    int32_t qtype, float qmax, int32_t group_cols, void* q_out,
                                    float* scale_out, void* stream);

/*
 * Weight quantisation, one absmax scale per output channel (row of W) or per
 * 128x128 block.  TeleFuser "Quantization", "Offline conversion" (one absmax
 * scale per output row for int8 and fp8) and "tf-kernel FP8: online W8A8"
 * (weights quantised per output channel, cached by the caller on first use);
 * LightX2V table "量化模式" (fp8-b128-deepgemm block-symmetric weights) and
 * vLLM-Omni "Parameters" (weight_block_size).
 *
 *   w_bf16    [n, k] BF16, dense, 16-byte aligned.
 *   block     0 = per output channel (scale_out [n]);
 *             128 = per 128x128 block (scale_out [n/128, k/128]; n % 128 == 0
 *             and k % 128 == 0).
 *   q_out     [n, k] codes, 16-byte aligned.
 *   n >= 1; k >= 16, k % 16 == 0.
 */
tfq_status tfq_quantize_weight_per_channel(const void* w_bf16, int64_t n, int64_t k, int32_t qtype,
                                           float qmax, int32_t block, void* q_out,
                                           float* scale_out, void* stream);

/*
 * Scaled FP8 (E4M3FN x E4M3FN, FP32 accumulation) GEMM with the scale
 * epilogue fused into the BF16 store: y = a . b^T scaled per row and column.
 * TeleFuser "Quantization", "tf-kernel FP8: online W8A8" (fp8_scaled_mm
 * produces BF16) and "Scaled FP8 checkpoints: W8A8"; block mode follows
 * LightX2V table "量化模式" (fp8-b128-deepgemm).
 *
 *   a_q [m, k] codes (activations), b_q [n, k] codes (weights, one output
 *   channel per row): both K-contiguous, 16-byte aligned.
 *   scale_block 0:   a_scale [m], b_scale [n].
 *   scale_block 128: a_scale [m, k/128] (1x128 groups), b_scale [n/128, k/128]
 *                    (128x128 blocks); k % 128 == 0, n % 128 == 0,
 *                    k <= 131072 (else TFQ_ERR_BAD_SHAPE).
 *   bias_bf16  [n] BF16 or NULL (16-byte aligned), added after scaling
 *              (before GELU).
 *   epi        tfq_epilogue.
 *   y_bf16     [m, n] BF16, 16-byte aligned.
 *   m >= 1; n >= 8, n % 8 == 0; k >= 16, k % 16 == 0.
 */
tfq_status tfq_scaled_mm_fp8(const uint8_t* a_q, const float* a_scale, const uint8_t* b_q,
                             const float* b_scale, int64_t m, int64_t n, int64_t k,
                             int32_t scale_block, const void* bias_bf16, int32_t epi, void* y_bf16,
                             void* stream);

/*
 * Scaled INT8 GEMM (INT32 accumulation, exact): symmetric INT8 of TeleFuser
 * "Quantization", "Core ideas", per-token activations and per-channel
 * weights.
 *
 *   a_q [m, k], b_q [n, k] int8 codes, 16-byte aligned; a_scale [m],
 *   b_scale [n]; bias_bf16 [n] or NULL (16-byte aligned); epi tfq_epilogue.
 *   y_bf16  [m, n] BF16 output or NULL.
 *   acc_i32 [m, n] raw INT32 accumulators or NULL (16-byte aligned).
 *   At least one of y_bf16 / acc_i32 must be given.
 *   m >= 1; n >= 8, n % 8 == 0; 16 <= k <= 131071, k % 16 == 0 (so no INT32
 *   sum can overflow: 131071 * 128 * 128 < 2^31).
 */
tfq_status tfq_scaled_mm_int8(const int8_t* a_q, const float* a_scale, const int8_t* b_q,
                              const float* b_scale, int64_t m, int64_t n, int64_t k,
                              const void* bias_bf16, int32_t epi, void* y_bf16, int32_t* acc_i32,
                              void* stream);

/*
 * Grouped (MoE) scaled FP8 GEMM: rows group_offsets[g] .. group_offsets[g+1]
 * of a_q are multiplied by expert g's weights, y[m,:] = the scaled product
 * of a_q[m] with b_q[g] as in tfq_scaled_mm_fp8 (per-row a_scale, per-output-
 * channel b_scale[g], optional bias[g], epilogue).  TeleFuser "Quantization",
 * "Other quantized data paths" (LingBot-Video MoE FP8: expert weights per
 * output channel, routed activations per row, a scaled matmul per expert).
 *
 *   a_q [m, k] E4M3FN codes, a_scale [m] (e.g. from
 *   tfq_quantize_rows_gather, rows sorted by expert).
 *   b_q [groups, n, k] codes, b_scale [groups, n] FP32, bias_bf16
 *   [groups, n] BF16 or NULL (16-byte aligned).
 *   group_offsets [groups + 1] int32 DEVICE array, 4-byte aligned, read by
 *   the kernel: non-decreasing, group_offsets[0] >= 0, group_offsets[groups]
 *   <= m.  Rows in no group are not written.  Offsets that break these rules
 *   are clamped to [0, m] (every access stays in bounds) but give unspecified
 *   results.
 *   y_bf16 [m, n] BF16, 16-byte aligned.
 *   1 <= groups <= 256; m >= 1; n >= 8, n % 8 == 0; 16 <= k <= 4194304,
 *   k % 16 == 0.
 */
tfq_status tfq_grouped_scaled_mm_fp8(const uint8_t* a_q, const float* a_scale, const uint8_t* b_q,
                                     const float* b_scale, const int32_t* group_offsets,
                                     int32_t groups, int64_t m, int64_t n, int64_t k,
                                     const void* bias_bf16, int32_t epi, void* y_bf16, void* stream);

/*
 * Bytes of workspace tfq_quant_linear_fused needs: the activation codes
 * [m, k] followed (at a 256-byte boundary) by the activation scales.
 * Returns 0 for invalid arguments.
 */
size_t tfq_quant_linear_workspace_bytes(int64_t m, int64_t k, int32_t qtype, int32_t scale_block);

/*
 * The W8A8 Linear forward: quantise the BF16 activations per token (or per
 * 1x128 group when scale_block = 128) into the workspace, then run the scaled
 * GEMM against already-quantised weights, on one stream.  TeleFuser
 * "Quantization", "tf-kernel FP8: online W8A8" and "Scaled FP8 checkpoints:
 * W8A8" (LinearFP8: quantise each input row every forward, scaled GEMM, BF16
 * out).
 *
 *   x_bf16 [m, k] (row stride ld_x) BF16 activations; w_q [n, k] codes and
 *   w_scale ([n], or [n/128, k/128] for scale_block 128) from
 *   tfq_quantize_weight_per_channel; qtype applies to both operands;
 *   act_qmax the activation qmax; bias_bf16 [n] or NULL (16-byte aligned);
 *   epi tfq_epilogue;
 *   block mode (scale_block = 128) is FP8 only;
 *   y_bf16 [m, n]; workspace of at least
 *   tfq_quant_linear_workspace_bytes(m, k, qtype, scale_block) bytes,
 *   256-byte aligned, owned by the caller and not used concurrently by
 *   another call.
 */
tfq_status tfq_quant_linear_fused(const void* x_bf16, int64_t m, int64_t k, int64_t ld_x,
                                  const void* w_q, const float* w_scale, int64_t n, int32_t qtype,
                                  float act_qmax, int32_t scale_block, const void* bias_bf16,
                                  int32_t epi, void* y_bf16, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* Size of the device scratch of tfq_quant_linear_fused_noalloc (per GPU). */
#define TFQ_NOALLOC_WORKSPACE_BYTES ((size_t)64 << 20)

/*
 * tfq_quant_linear_fused for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same quantise + scaled GEMM kernels, with the activation
 * codes and scales in a device array of TFQ_NOALLOC_WORKSPACE_BYTES that the
 * library holds on each GPU it runs on until the process ends, instead of a
 * caller workspace.  The call allocates nothing (no hipMalloc, no host or
 * device allocation by any library it uses) and never tunes: it launches the
 * GEMM configuration already cached for the shape (tfq_set_autotune) or the
 * heuristic one.  Arguments as for tfq_quant_linear_fused without the
 * workspace.
 *
 * Limit: tfq_quant_linear_workspace_bytes(m, k, qtype, scale_block) must not
 * exceed TFQ_NOALLOC_WORKSPACE_BYTES, else TFQ_ERR_WORKSPACE_TOO_SMALL (e.g.
 * 64 MiB holds m * k up to about 66e6 activation codes).
 *
 * Calls on one GPU share its array and each call leaves its codes there:
 * calls that overlap in time on one GPU (two streams, two threads) race and
 * give unspecified results; calls ordered on one stream are safe.
 */
tfq_status tfq_quant_linear_fused_noalloc(const void* x_bf16, int64_t m, int64_t k, int64_t ld_x,
                                          const void* w_q, const float* w_scale, int64_t n,
                                          int32_t qtype, float act_qmax, int32_t scale_block,
                                          const void* bias_bf16, int32_t epi, void* y_bf16,
                                          void* stream);

/*
 * MXFP8 quantisation: E4M3FN codes with one E8M0 scale byte per 32
 * consecutive elements of a row.  TeleFuser "Quantization", converter
 * section (MXFP8 uses 32-value blocks with E8M0 scales); the pages print no
 * block rule, so the OCP Microscaling (MX) v1.0 one is used: shared exponent
 * floor(log2(amax)) - 8 (8 = the exponent of E4M3FN's largest normal),
 * clamped to [-127, 127], scale byte = shared + 127 (an all-zero block gets
 * byte 0); codes = E4M3FN_RNE(clamp(x * 2^-shared, -448, 448)), an exact
 * power-of-two scaling.
 *
 *   x_bf16    [rows, cols] BF16, row stride ld_x elements (ld_x >= cols,
 *             ld_x % 8 == 0), 16-byte aligned.
 *   q_out     [rows, cols] E4M3FN codes, dense, 16-byte aligned.
 *   scale_out [cols/128, rows] 32-bit scale words, 4-byte aligned: bytes
 *             0, 1, 2, 3 (little-endian) of word (g, r) are the scales of
 *             blocks 4 g, 4 g + 2, 4 g + 1, 4 g + 3 of row r -- the four
 *             block scales of a 128-wide K group, stored group-major so that
 *             the GEMM reads a tile's scales for one K group in one piece,
 *             in the byte order its matrix instructions take them.
 *   rows >= 1; cols >= 128, cols % 128 == 0; rows * cols / 32 <= 2^30.
 * Quantising weights [n, k] with this call gives the MXFP8 weight operand.
 */
tfq_status tfq_quantize_mx(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                           void* q_out, uint32_t* scale_out, void* stream);

/*
 * MXFP8 GEMM: y[m,n] = sum over 32-blocks kb of 2^(ea[m,kb] - 127)
 * 2^(eb[n,kb] - 127) sum_{k in kb} a[m,k] b[n,k], accumulated in FP32 (the
 * matrix cores apply the E8M0 scales), rounded once to BF16 (RNE), bias
 * and epilogue as for tfq_scaled_mm_fp8.  TeleFuser "Quantization",
 * converter section (MXFP8 block format).
 *
 *   a_q [m, k], b_q [n, k] E4M3FN codes, K-contiguous, 16-byte aligned.
 *   a_scale [k/128, m], b_scale [k/128, n] scale words in the layout
 *   tfq_quantize_mx writes, 4-byte aligned (byte 255, NaN in the MX format,
 *   gives unspecified results).
 *   bias_bf16 [n] BF16 or NULL (16-byte aligned); epi tfq_epilogue;
 *   y_bf16 [m, n] BF16, 16-byte aligned.
 *   m >= 1; n >= 8, n % 8 == 0; 128 <= k <= 4194304, k % 128 == 0;
 *   m * k / 32 <= 2^30 and n * k / 32 <= 2^30.
 */
tfq_status tfq_scaled_mm_mxfp8(const uint8_t* a_q, const uint32_t* a_scale, const uint8_t* b_q,
                               const uint32_t* b_scale, int64_t m, int64_t n, int64_t k,
                               const void* bias_bf16, int32_t epi, void* y_bf16, void* stream);

/*
 * MXFP4 quantisation: E2M1 codes (1 sign, 2 exponent bits with bias 1, 1
 * mantissa bit: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6) with one E8M0 scale
 * byte per 32 consecutive elements of a row.  TeleFuser "Quantization",
 * converter section (MXFP4 uses 32-value blocks with E8M0 scales); OCP MX
 * v1.0 block rule: shared exponent floor(log2(amax)) - 2 (6 = 1.5 * 2^2),
 * clamped to [-127, 127], scale byte = shared + 127; codes = nearest E2M1
 * value of clamp(x * 2^-shared, +-6), ties to the even code, sign kept.
 *
 *   x_bf16    [rows, cols] BF16 as tfq_quantize_mx.
 *   q_out     [rows, cols/2] bytes, two codes each, the element with the
 *             lower index in the low nibble; 16-byte aligned.
 *   scale_out [cols/128, rows] scale words in the layout of
 *             tfq_quantize_mx.
 *   rows >= 1; cols >= 128, cols % 128 == 0; rows * cols / 32 <= 2^30.
 */
tfq_status tfq_quantize_mxfp4(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                              void* q_out, uint32_t* scale_out, void* stream);

/*
 * MXFP4 GEMM: y[m,n] = sum over 32-blocks kb of 2^(ea[m,kb] - 127)
 * 2^(eb[n,kb] - 127) sum_{k in kb} a[m,k] b[n,k] over E2M1 values,
 * accumulated in FP32 by the matrix cores, rounded once to BF16, bias and
 * epilogue as for tfq_scaled_mm_fp8.  TeleFuser "Quantization", converter
 * section (MXFP4 block format).
 *
 *   a_q [m, k/2], b_q [n, k/2] packed E2M1 codes (as tfq_quantize_mxfp4
 *   writes them), 16-byte aligned; a_scale [k/128, m], b_scale [k/128, n]
 *   scale words as for tfq_scaled_mm_mxfp8.
 *   bias_bf16 [n] or NULL (16-byte aligned); epi tfq_epilogue; y_bf16
 *   [m, n] BF16.
 *   m >= 1; n >= 8, n % 8 == 0; 128 <= k <= 8388608, k % 128 == 0;
 *   m * k / 32 <= 2^30 and n * k / 32 <= 2^30.
 */
tfq_status tfq_scaled_mm_mxfp4(const uint8_t* a_q, const uint32_t* a_scale, const uint8_t* b_q,
                               const uint32_t* b_scale, int64_t m, int64_t n, int64_t k,
                               const void* bias_bf16, int32_t epi, void* y_bf16, void* stream);

/*
 * MXFP6 quantisation: 6-bit codes with one E8M0 scale byte per 32
 * consecutive elements of a row.  TeleFuser "Quantization", converter
 * section (MXFP6 uses 32-value blocks with E8M0 scales); OCP MX v1.0.
 *   fmt 0: E2M3 (2 exponent bits with bias 1, 3 mantissa bits, largest 7.5,
 *          shared exponent floor(log2(amax)) - 2);
 *   fmt 1: E3M2 (3 exponent bits with bias 3, 2 mantissa bits, largest 28,
 *          shared exponent floor(log2(amax)) - 4).
 * Scale byte = shared + 127 (clamped to [0, 254]); codes = nearest value of
 * x * 2^-shared clamped to the largest, ties to the even code, sign in bit 5
 * (kept for zero).
 *   q_out     [cols/128, rows, 96] bytes, group-major: the 128 codes of
 *             group g (elements 128 g .. 128 g + 127) of row r are the 96
 *             bytes at (g rows + r) 96, a little-endian bit stream with
 *             element 128 g + i in bits 6 i .. 6 i + 5; 16-byte aligned.
 *             (A GEMM stage of 128 elements then reads one contiguous panel
 *             of rows, whole cache lines.)
 *   scale_out [cols/128, rows] scale words as for tfq_quantize_mx.
 *   rows >= 1; cols >= 128, cols % 128 == 0; rows * cols / 32 <= 2^30.
 */
tfq_status tfq_quantize_mxfp6(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                              int32_t fmt, void* q_out, uint32_t* scale_out, void* stream);

/*
 * MXFP6 GEMM, as tfq_scaled_mm_mxfp8 over 6-bit codes of format fmt (both
 * operands): a_q [k/128, m, 96], b_q [k/128, n, 96] as tfq_quantize_mxfp6
 * writes them, a_scale [k/128, m], b_scale [k/128, n] scale words.
 * TeleFuser "Quantization", converter section (MXFP6 block format).
 *   m >= 1; n >= 8, n % 8 == 0; 128 <= k <= 4194304, k % 128 == 0;
 *   m * k / 32 <= 2^30 and n * k / 32 <= 2^30.
 */
tfq_status tfq_scaled_mm_mxfp6(const uint8_t* a_q, const uint32_t* a_scale, const uint8_t* b_q,
                               const uint32_t* b_scale, int64_t m, int64_t n, int64_t k, int32_t fmt,
                               const void* bias_bf16, int32_t epi, void* y_bf16, void* stream);

/*
 * FP8 KV cache.  TeleFuser "Quantization", "Other quantized data paths"
 * (LiveAct FP8 KV cache: K/V stored as E4M3FN with one FP32 scale per
 * last-dimension vector, dequantised to the requested attention dtype on
 * load).  A cache holds `slots` rows of [heads, head_dim] E4M3FN codes
 * (uint8 [slots, heads, head_dim], 16-byte aligned) and their scales
 * (FP32 [slots, heads]); K and V are two such caches.
 *
 * Store: each vector kv[t, h, :] is quantised exactly as an FP8 row of
 * tfq_quantize_rows (s = RN32(amax / qmax), codes E4M3FN_RNE(clamp(RN32(x /
 * s), ±qmax))) into cache row slot_index[t], head h.
 *   kv_bf16    [tokens, heads, head_dim] BF16, token stride ld_token elements
 *              (ld_token >= heads * head_dim, ld_token % 8 == 0), heads
 *              contiguous, 16-byte aligned.
 *   slot_index [tokens] int32 DEVICE array; a slot outside [0, slots) is
 *              not written.  Slots must be distinct (else which token's
 *              vector a slot keeps is unspecified).
 *   qmax       E4M3FN grid value <= 448 (448 = the full range).
 *   8 <= head_dim <= 512, head_dim % 8 == 0.
 */
tfq_status tfq_kv_cache_store(const void* kv_bf16, int64_t tokens, int64_t heads, int64_t head_dim,
                              int64_t ld_token, const int32_t* slot_index, int64_t slots,
                              float qmax, uint8_t* cache, float* cache_scale, void* stream);

/*
 * Load (dequantise): out[i, h, :] = cache_scale[j, h] * value(cache[j, h, :])
 * for j = slot_index[i]: the E4M3FN value is exact, the product one binary32
 * multiplication (RNE), then one conversion (RNE) to out_dtype: 0 = BF16,
 * 1 = FP16, 2 = FP32.  A slot outside [0, slots) gives a zero vector.
 *   slot_index [n] int32 DEVICE array; out [n, heads, head_dim], 16-byte
 *   aligned.
 */
tfq_status tfq_kv_cache_load(const uint8_t* cache, const float* cache_scale, int64_t slots,
                             int64_t heads, int64_t head_dim, const int32_t* slot_index, int64_t n,
                             int32_t out_dtype, void* out, void* stream);

/*
 * Per-exact-shape autotuning of the GEMM launch configuration.  LightX2V
 * "模型量化技术", "MiniMax-H3 FP8 FP16 累加" (tile and swizzle tuned per exact
 * GEMM shape on first sight, winner kept in an in-process C++ cache, warm-up
 * absorbing the first call, nothing written to disk).
 *
 * mode 0 (default): every GEMM entry point uses a fixed heuristic
 * configuration.  mode 1: the first call of each (device, kind, m, n, k,
 * epilogue, groups) shape times every candidate configuration (tile order
 * band height; for per-channel FP8 / INT8 also the tile shape) on the
 * caller's buffers and stream, caches the fastest and uses it from then on.
 * That first call waits for the stream; a stream being captured into a
 * graph is never tuned (the cached or the heuristic configuration is used).
 * Every configuration produces the same result bits.  Other values:
 * TFQ_ERR_UNSUPPORTED.
 */
tfq_status tfq_set_autotune(int32_t mode);

/*
 * The cached configuration of a shape, if any: returns 1 and writes kernel
 * (0 = 256x256 tiles, 1 = 256x128 tiles two per CU, 2 = 256x192 tiles; 1
 * and 2 for per-channel FP8 and INT8 only) and band (tile rows per band of
 * the tile order), else 0.  kind: 0 FP8 per channel (tfq_scaled_mm_fp8,
 * scale_block 0, and the fused FP8 Linear), 1 INT8, 2 FP8 block-scaled,
 * 3 MXFP8, 4 grouped FP8 (with `groups`), 5 MXFP4, 6 MXFP6 E2M3, 7 MXFP6
 * E3M2.  Looks up the current device's entries.
 */
int32_t tfq_autotune_lookup(int32_t kind, int64_t m, int64_t n, int64_t k, int32_t epi,
                            int32_t groups, int32_t* kernel, int32_t* band);

/*
 * Put a launch configuration for one shape into the current device's cache
 * (the same cache tuning fills, with the same key as tfq_autotune_lookup):
 * a tuning table saved from an earlier run can be loaded this way instead of
 * tuning again.  The configuration is used while autotuning is on
 * (tfq_set_autotune(1)).  It must be one of the configurations the tuner
 * would try for that shape, all of which give the same result bits;
 * otherwise TFQ_ERR_UNSUPPORTED (also for an unknown kind or epilogue).
 * TFQ_ERR_BAD_SHAPE for non-positive sizes or groups outside 1..256 (kind 4).
 */
tfq_status tfq_autotune_set(int32_t kind, int64_t m, int64_t n, int64_t k, int32_t epi,
                            int32_t groups, int32_t kernel, int32_t band);

/* Forget every cached configuration. */
void tfq_autotune_clear(void);

/*
 * The device's own E4M3FN encoder (round-to-nearest-even, saturating to
 * +-448, sign of zero kept) applied to n FP32 values: the cast of TeleFuser
 * "Quantization", "Scaled FP8 checkpoints: W8A8", exposed on its own so that
 * the conversion the quantiser uses can be checked over all binary32 inputs.
 *   x [n] FP32, q [n] codes, both 16-byte aligned; n >= 1, n % 4 == 0.
 */
tfq_status tfq_e4m3fn_encode_f32(const float* x, uint8_t* q, int64_t n, void* stream);

/* Static, NUL-terminated description of a status code. */
const char* tfq_status_string(tfq_status s);
/* hipError_t of the last TFQ_ERR_HIP returned on the calling thread (0 if none). */
int tfq_last_hip_error(void);
/* TFQ_ABI_VERSION of the library. */
int tfq_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TFQ_H */
