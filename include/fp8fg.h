/*
 * fp8fg — fine-grained FP8 (OCP E4M3) quantization and block-scaled GEMMs for MI355X (gfx950).
 *
 * C ABI. Every pointer argument is DEVICE memory owned by the caller; the library never allocates, frees
 * or synchronises. All work is enqueued asynchronously on `stream` (0 = the null stream), and the calls
 * can be captured in a HIP graph (no memset or host synchronisation is enqueued). The library keeps no
 * state between calls beyond per-device facts cached on first use (compute-unit count, the GEMM kernels'
 * LDS limit), and is safe to call from several threads. Arguments are checked on the host
 * before any HIP call; a failed check returns a status and enqueues nothing. A launch failure returns
 * FG_ERR_HIP and fg_last_hip_error() gives the hipError_t on the calling thread.
 *
 * Sources (web pages quoting the FP8 training section of the DeepSeek-V3 report):
 *   [W1] "5 Ways You can get More Deepseek While Spending Less"
 *   [W2] untitled page, why-be.why-be.co.kr board "as_center", post 65967
 *   [W3] untitled page, cameseeing.com board "community", post 22576
 *   [W4] "Three Fast Methods To Study Deepseek"
 *   [W5] untitled page, gnrental.net board "free", post 15227
 *
 * Number formats.
 *   bf16 inputs: IEEE bfloat16 bit patterns (2 bytes). Inputs must be finite (NaN/Inf: undefined result).
 *   codes: OCP E4M3 ("E4M3FN"), 1 byte: bias 7, max 448 (0x7E), no infinities, 0x7F/0xFF are NaN
 *          (E4M3 on all tensors: [W4]/[W5], the passage contrasting it with the hybrid E4M3/E5M2 format).
 *   scales: fp32. Dequantized value = decode(code) * scale.
 *
 * Quantization rule (identical for every quantizer): for each group (1x128 tile or 128x128 block),
 *   amax  = max |x| over the group, computed from the data being quantized ("online"; [W3], passage next
 *           to Figure 7 (a));
 *   scale = amax / 448 in fp32 (IEEE division): the max-abs is aligned to the largest E4M3 value ([W1],
 *           passage on scaling the maximum absolute value to the maximum representable FP8 value);
 *           amax == 0 gives scale 1; a scale below FLT_MIN is raised to FLT_MIN;
 *           FG_SCALE_POW2 then rounds the scale up to the next integral power of two ([W1], opening
 *           paragraph: scaling factors that are integral powers of 2);
 *   code  = E4M3 round-to-nearest-even of the fp32 quotient x / scale (correctly rounded division).
 *   Codes and scales are bit-exact against a plain CPU statement of this rule.
 *
 * GEMM rule ([W1]: per-group scaling factors along the inner dimension; partial sums promoted into FP32
 * every 128 elements of K, the "128 elements, equal to four WGMMAs" interval; [W5]: GEMMs take FP8
 * inputs and produce BF16 or FP32): for every output element and every 128-element block b of the
 * contraction dimension, in ascending order,
 *   P_b  = sum over the block of decode(a) * decode(b)          (matrix-core partial sum)
 *   acc  = fma(P_b, scale_a * scale_b, acc)                     (FP32 promotion in registers)
 * and the output is acc (FP32) or acc rounded to nearest-even BF16.
 * The matrix core's summation inside a block is hardware-defined; results agree with the exact value to
 * within a max relative error of 1e-3 (FP32 output) / 1e-2 (BF16 output), normwise.
 *
 * Every GEMM takes `scales`, the mode its operands were quantized in. FG_SCALE_FP32 accepts any fp32
 * scales and promotes with a VALU FMA per element and block, as above. FG_SCALE_POW2 declares that every
 * scale is an exact power of two in [2^-126, 2^127] (what the quantizers write in that mode): the matrix
 * core then applies the scales itself (E8M0 block-scale operands of v_mfma_scale_f32_16x16x128_f8f6f4) and
 * adds 2^(ea+eb) * P_b straight into the FP32 accumulator, which is the same promotion with an exact
 * scale product and no VALU work. Passing FG_SCALE_POW2 with a scale that has sign or mantissa bits set
 * makes the outputs NaN (every output of each 64-column wave tile whose contraction read such a scale;
 * fg_fp8_gemm_fprop_quant then writes NaN codes 0x7F and NaN scales for those rows). A zero scale reads as
 * 2^-127 in this mode.
 *
 * Size limits of every GEMM (the kernels address operand rows with 32-bit offsets from the tile base):
 * the contraction length is at most 2^24, and Dgrad's output width (its K) at most 2^25. A launch has at
 * most 2^31 - 1 workgroups: a GEMM with more than 2^31 - 1 tiles of 256 x 128 outputs, or a grouped GEMM
 * with more than 2^31 - 1 in (total_rows / 256 + G + 7) x (output width / 128), is refused. Larger shapes
 * return FG_ERR_UNSUPPORTED_SHAPE.
 *
 * Every GEMM picks one of two workgroup tiles per launch (256x192 or 256x256 outputs) from the problem size
 * and the device's compute-unit count, and fg_fp8_gemm_fprop a third (256x288) where it covers the output
 * in fewer rounds of tiles over the compute units; the results are bit-identical whichever is used (every
 * output element goes through the same instructions in the same order). The environment variable
 * FG_GEMM_TILE=256x192, 256x256 or 256x288 (Fprop only) forces one (read at every launch).
 *
 * Layouts are row-major. "ld" arguments are row strides in elements.
 * Activation scales are MN-major: scale[group][row] (rows contiguous), so one 128-deep K step of a GEMM
 * reads its rows' scales as one contiguous run.
 */
#ifndef FP8FG_H
#define FP8FG_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FG_OK = 0,
    FG_ERR_INVALID_ARG = 1,        /* null pointer, negative size, bad enum, ld smaller than the row   */
    FG_ERR_UNSUPPORTED_SHAPE = 2,  /* a size that the operation's tiling requires to be a multiple    */
    FG_ERR_MISALIGNED = 3,         /* a pointer or leading dimension breaks the 16-byte row alignment */
    FG_ERR_HIP = 4                 /* the HIP runtime reported an error at launch                     */
} fg_status;

typedef enum { FG_SCALE_FP32 = 0, FG_SCALE_POW2 = 1 } fg_scale_mode;
typedef enum { FG_OUT_F32 = 0, FG_OUT_BF16 = 1 } fg_out_dtype;
typedef enum {
    FG_ALONG_COLS = 0,   /* 1x128 tiles along the columns (per token, per 128 channels)               */
    FG_ALONG_ROWS = 1    /* 1x128 tiles along the rows (per channel, per 128 tokens), codes transposed */
} fg_tile_axis;

/* 1x128 activation quantization ([W2]/[W3]/[W4], Figure 7 (a): activations are grouped and scaled per
 * token per 128 channels; the forward activations are kept as 1x128 FP8 tiles for the backward pass,
 * [W1] Figure 6 passage).
 *
 *   x       bf16 [rows][cols], row stride ld_x (elements).
 *   FG_ALONG_COLS: requires cols % 128 == 0. Writes q u8 [rows][cols] (row stride cols) and
 *                  scales f32 [cols/128][rows]. Any rows >= 0.
 *   FG_ALONG_ROWS: the token-dimension tiling used by the weight-gradient GEMM, which contracts over
 *                  tokens. Requires rows % 128 == 0 and cols % 8 == 0. Writes q u8 [cols][rows]
 *                  (transposed, row stride rows) and scales f32 [rows/128][cols].
 *   Alignment: x, q 16-byte aligned; ld_x % 8 == 0; scales 4-byte aligned.
 *   rows == 0 or cols == 0 is a no-op returning FG_OK. */
fg_status fg_quantize_act_1x128(const void* x, int64_t rows, int64_t cols, int64_t ld_x,
                                fg_tile_axis axis, fg_scale_mode mode,
                                uint8_t* q, float* scales, hipStream_t stream);

/* Both 1x128 tilings of one activation from a single read ([W1] Figure 6 passage: activations are kept in
 * FP8 for the backward pass, where the Wgrad GEMM consumes them tiled along the tokens; [W5] passage on
 * the transposed reads that the backward pass needs): writes exactly what fg_quantize_act_1x128 writes
 * with FG_ALONG_COLS into (q_cols, scales_cols) and with FG_ALONG_ROWS into (q_rows, scales_rows),
 * bit for bit, reading x once instead of twice.
 *   x       bf16 [rows][cols], row stride ld_x; rows % 128 == 0 and cols % 128 == 0.
 *   q_cols  u8 [rows][cols], scales_cols f32 [cols/128][rows]   (tiles along the columns)
 *   q_rows  u8 [cols][rows], scales_rows f32 [rows/128][cols]   (tiles along the rows, transposed)
 *   Alignment: x, q_cols, q_rows 16-byte aligned; ld_x % 8 == 0; scales 4-byte aligned.
 *   rows == 0 or cols == 0 is a no-op returning FG_OK. */
fg_status fg_quantize_act_1x128_both(const void* x, int64_t rows, int64_t cols, int64_t ld_x, fg_scale_mode mode,
                                     uint8_t* q_cols, float* scales_cols, uint8_t* q_rows, float* scales_rows,
                                     hipStream_t stream);

/* Token tiles from cached FP8 activations. The activations Wgrad needs are kept in FP8 for the backward
 * pass ([W4]/[W5], Figure 6 passage), as 1x128 tiles along the channels; Wgrad contracts over tokens and
 * needs tiles along the tokens, so the cached codes are read, dequantized, transposed and quantized
 * again ([W5], the chip-design passage on transposed reads that would spare these memory operations).
 *   q_in  u8 [rows][cols], s_in f32 [cols/128][rows]: codes and scales of fg_quantize_act_1x128 along
 *         the columns (row stride cols).
 *   Each element is taken as the bf16 activation bf16(RN_f32(decoded code * its row scale)), and that
 *   tensor is quantized as fg_quantize_act_1x128(.., FG_ALONG_ROWS, mode) would quantize it:
 *   q_out u8 [cols][rows] (transposed), s_out f32 [rows/128][cols].
 *   With power-of-2 scales in and out, the dequantized values lie on the E4M3 grid of every power-of-2
 *   scale, so re-quantizing rounds nothing except values that leave E4M3's normal range; with fp32
 *   scales each value is rounded a second time.
 *   rows % 128 == 0, cols % 128 == 0. q_in, s_in, q_out 16-byte aligned; s_out 4-byte aligned.
 *   rows == 0 or cols == 0 is a no-op. */
fg_status fg_requantize_1x128_to_tokens(const uint8_t* q_in, const float* s_in, int64_t rows, int64_t cols,
                                        fg_scale_mode mode, uint8_t* q_out, float* s_out, hipStream_t stream);

/* 128x128 weight-block quantization ([W2]/[W3]/[W4], Figure 7 (a): per 128 input channels per 128
 * output channels).
 *   w       bf16 [n][k], row stride ld_w; k % 128 == 0; any n >= 0 (a short last block row-group takes
 *           the max over the rows it has).
 *   q       u8 [n][k] (row stride k);  scales f32 [ceil(n/128)][k/128] row-major.
 *   Alignment: w, q 16-byte aligned; ld_w % 8 == 0; scales 4-byte aligned. */
fg_status fg_quantize_w_128x128(const void* w, int64_t n, int64_t k, int64_t ld_w,
                                fg_scale_mode mode, uint8_t* q, float* scales, hipStream_t stream);

/* The Linear operator's two forward operands in one launch ([W1]/[W3]/[W4], Figure 6: the Fprop takes X
 * and W in FP8, and the backward pass keeps X's FP8 tiles for Wgrad; Figure 7 (a): 1x128 activation tiles
 * and 128x128 weight blocks): writes exactly what fg_quantize_act_1x128_both(x, rows, k, ld_x, mode,
 * q_cols, scales_cols, q_rows, scales_rows) and fg_quantize_w_128x128(w, n, k, ld_w, mode, qw, sw) write,
 * bit for bit, from a single kernel launch. Both tensors share the contraction width k.
 *   x   bf16 [rows][k], row stride ld_x; rows % 128 == 0, k % 128 == 0.
 *   q_cols u8 [rows][k], scales_cols f32 [k/128][rows]; q_rows u8 [k][rows], scales_rows f32 [rows/128][k].
 *   w   bf16 [n][k], row stride ld_w; any n >= 0.   qw u8 [n][k], sw f32 [ceil(n/128)][k/128].
 *   Alignment: x, w, q_cols, q_rows, qw 16-byte aligned; ld_x % 8 == 0, ld_w % 8 == 0; scales 4-byte
 *   aligned. A tensor with rows == 0 (x) or n == 0 (w) is not read and its pointers and row stride are
 *   ignored; the launch covers the other one (nothing when both are empty or k == 0).
 *   FG_ERR_UNSUPPORTED_SHAPE when the two tensors' blocks exceed 2^31 - 1 workgroups in all. */
fg_status fg_quantize_fprop_operands(const void* x, int64_t rows, int64_t ld_x, const void* w, int64_t n, int64_t ld_w,
                                     int64_t k, fg_scale_mode mode, uint8_t* q_cols, float* scales_cols,
                                     uint8_t* q_rows, float* scales_rows, uint8_t* qw, float* sw, hipStream_t stream);

/* Fprop ([W1]/[W3]/[W4]/[W5], Figure 6, forward pass): Y[M][N] = X[M][K] . W[N][K]^T.
 *   xq u8 [M][K], sx f32 [K/128][M]   (from fg_quantize_act_1x128, FG_ALONG_COLS)
 *   wq u8 [N][K], sw f32 [ceil(N/128)][K/128]   (from fg_quantize_w_128x128)
 *   y  [M][N] f32 or bf16 (row stride N).  K % 128 == 0; any M, N >= 0 (M == 0 or N == 0: no-op;
 *   K == 0 writes zeros). xq, wq, y 16-byte aligned; sx, sw 4-byte aligned. */
fg_status fg_fp8_gemm_fprop(const uint8_t* xq, const float* sx, const uint8_t* wq, const float* sw,
                            int64_t M, int64_t N, int64_t K, void* y, fg_out_dtype out,
                            fg_scale_mode scales, hipStream_t stream);

/* Fprop with the output quantized on chip: the BF16 Y of fg_fp8_gemm_fprop, quantized 1x128 along its
 * columns (per token per 128 output channels, as the next layer's Fprop input needs it) before it leaves
 * the GEMM. [W5], the passage of chip-design suggestions, describes the round trip this removes: BF16
 * activations written to HBM, read back for quantization, FP8 codes written and read again for the next
 * MMA. Here only the codes and scales reach HBM.
 *   xq, sx, wq, sw as for fg_fp8_gemm_fprop (scales: their scale mode).
 *   yq u8 [M][N], sy f32 [N/128][M]: bit-identical to fg_quantize_act_1x128(Y_bf16, FG_ALONG_COLS,
 *   out_scales) applied to the BF16 output of fg_fp8_gemm_fprop on the same operands.
 *   N % 128 == 0, K % 128 == 0, any M (M == 0 or N == 0: no-op; K == 0 quantizes zeros: codes 0,
 *   scales 1). xq, wq, yq 16-byte aligned; scales 4-byte aligned. Always the 256x256 output tile. */
fg_status fg_fp8_gemm_fprop_quant(const uint8_t* xq, const float* sx, const uint8_t* wq, const float* sw,
                                  int64_t M, int64_t N, int64_t K, uint8_t* yq, float* sy,
                                  fg_scale_mode scales, fg_scale_mode out_scales, hipStream_t stream);

/* Dgrad (Figure 6, activation backward pass): dX[M][K] = dY[M][N] . W[N][K], contracting over N.
 *   dyq u8 [M][N], sdy f32 [N/128][M]   (dY quantized FG_ALONG_COLS)
 *   wq  u8 [N][K], sw f32 [N/128][K/128] (the same codes and 128x128 block scales as Fprop; the block
 *       is a 128-group along both axes, so it serves the transposed contraction unchanged; the kernel
 *       reads W transposed on chip, the transposed read the pages ask of future hardware, [W5])
 *   dx  [M][K] f32 or bf16.  N % 128 == 0, K % 128 == 0, any M.
 *   dyq, wq, dx 16-byte aligned; sdy, sw 4-byte aligned. */
fg_status fg_fp8_gemm_dgrad(const uint8_t* dyq, const float* sdy, const uint8_t* wq, const float* sw,
                            int64_t M, int64_t N, int64_t K, void* dx, fg_out_dtype out,
                            fg_scale_mode scales, hipStream_t stream);

/* Wgrad (Figure 6, weight backward pass): dW[N][K] (+)= dY[M][N]^T . X[M][K], contracting over the M
 * tokens, from token-dimension quantized operands:
 *   dytq u8 [N][M], sdyt f32 [M/128][N]   (dY quantized FG_ALONG_ROWS)
 *   xtq  u8 [K][M], sxt  f32 [M/128][K]   (X quantized FG_ALONG_ROWS)
 *   dw   f32 [N][K]; weight gradients stay FP32 ([W5], passage on master weights and gradients).
 *        accumulate != 0: the FP32 accumulation of each element starts from the value already in dw.
 *   M % 128 == 0; any N, K >= 0 with K % 4 == 0. dytq, xtq, dw, sxt 16-byte aligned; sdyt 4-byte
 *   aligned. */
fg_status fg_fp8_gemm_wgrad(const uint8_t* dytq, const float* sdyt, const uint8_t* xtq, const float* sxt,
                            int64_t M, int64_t N, int64_t K, float* dw, int accumulate,
                            fg_scale_mode scales, hipStream_t stream);

/* Grouped Fprop for the routed experts of one GPU ([W4]: MoE layers of 256 routed experts with expert
 * intermediate dimension 2048, 8 active per token; [W5]: each GPU hosts 8 experts). For each group g:
 *   Y[off[g]:off[g+1]][:] = X[off[g]:off[g+1]][:] . W[g]^T
 *   xq u8 [T][K], sx f32 [K/128][T]; wq u8 [G][N][K], sw f32 [G][ceil(N/128)][K/128]; y [T][N].
 *   d_offsets: DEVICE int32 [G+1], non-decreasing, d_offsets[0] == 0, d_offsets[G] == T (precondition,
 *   not re-checked on the host). The kernel clamps each offset into [0, T] and treats a decreasing pair as
 *   an empty group, so malformed offsets give wrong results but no access outside the operands.
 *   K % 128 == 0, G >= 1. xq, wq, y 16-byte aligned; sx, sw, d_offsets 4-byte aligned. */
fg_status fg_fp8_grouped_gemm(const uint8_t* xq, const float* sx, const uint8_t* wq, const float* sw,
                              const int32_t* d_offsets, int32_t G, int64_t total_rows,
                              int64_t N, int64_t K, void* y, fg_out_dtype out, fg_scale_mode scales,
                              hipStream_t stream);

/* Grouped Dgrad of the routed experts (the backward of fg_fp8_grouped_gemm, the MoE backward pass of
 * [W1]/[W5], Figure 6 applied per expert). For each group g:
 *   dX[off[g]:off[g+1]][:] = dY[off[g]:off[g+1]][:] . W[g]
 *   dyq u8 [T][N], sdy f32 [N/128][T]        (dY quantized FG_ALONG_COLS over all T rows)
 *   wq  u8 [G][N][K], sw f32 [G][N/128][K/128] (the experts' weight codes and blocks, as in Fprop)
 *   dx  [T][K] f32 or bf16.  N % 128 == 0, K % 128 == 0. dyq, wq, dx 16-byte aligned; sdy, sw,
 *   d_offsets 4-byte aligned.
 *   d_offsets: DEVICE int32 [G+1] as for fg_fp8_grouped_gemm (precondition, not re-checked; clamped into
 *   [0, T] on the device as there). */
fg_status fg_fp8_grouped_gemm_dgrad(const uint8_t* dyq, const float* sdy, const uint8_t* wq, const float* sw,
                                    const int32_t* d_offsets, int32_t G, int64_t total_rows, int64_t N, int64_t K,
                                    void* dx, fg_out_dtype out, fg_scale_mode scales, hipStream_t stream);

/* Grouped Wgrad of the routed experts: for each group g, over the group's tokens,
 *   dW[g][N][K] (+)= dY[tokens of g][N]^T . X[tokens of g][K]
 *   dytq u8 [N][T], sdyt f32 [T/128][N]   (dY quantized FG_ALONG_ROWS over all T tokens)
 *   xtq  u8 [K][T], sxt  f32 [T/128][K]   (X quantized FG_ALONG_ROWS)
 *   dw   f32 [G][N][K]; accumulate != 0 starts each element from the value already in dw.
 *   The 1x128 token tiles must not straddle two groups: every d_offsets[g] is a multiple of 128 (a
 *   routed layout padded per expert; precondition, not re-checked; offsets are clamped into [0, T] on the
 *   device as for fg_fp8_grouped_gemm). T % 128 == 0, K % 4 == 0. dytq, xtq, dw, sxt 16-byte aligned;
 *   sdyt, d_offsets 4-byte aligned.
 *   An empty group writes zeros (or leaves dw unchanged with accumulate). */
fg_status fg_fp8_grouped_gemm_wgrad(const uint8_t* dytq, const float* sdyt, const uint8_t* xtq, const float* sxt,
                                    const int32_t* d_offsets, int32_t G, int64_t total_rows, int64_t N, int64_t K,
                                    float* dw, int accumulate, fg_scale_mode scales, hipStream_t stream);

/* ---- Accuracy study: accumulation without promotion ------------------------------------------------
 * Fprop as fg_fp8_gemm_fprop computes it but WITHOUT the FP32 promotion: every 32-element chunk of the
 * contraction is one matrix-core partial sum, scaled by its tile and block scales and added to an FP32
 * accumulator that keeps only `mantissa_bits` explicit mantissa bits (truncated toward zero) after every
 * addition. It emulates the limited accumulation width that [W1]/[W2] blame for an error of nearly 2% at
 * K = 4096 (the passage on increasing accumulation precision), for comparison with the promoted GEMMs.
 * Not part of the training path; written for clarity, not speed.
 *   xq, sx, wq, sw as for fg_fp8_gemm_fprop; y f32 [M][N].  K % 128 == 0; 1 <= mantissa_bits <= 23
 *   (23: an ordinary FP32 accumulator). xq, wq 8-byte aligned; y, scales 4-byte aligned. */
fg_status fg_fp8_gemm_fprop_limited_accum(const uint8_t* xq, const float* sx, const uint8_t* wq, const float* sw,
                                          int64_t M, int64_t N, int64_t K, int mantissa_bits, float* y,
                                          hipStream_t stream);

/* ---- E5M6 storage of cached activations -------------------------------------------------------------
 * [W1] keeps some cached activations (those entering the Linear after the attention operator) in a
 * customized E5M6 format with power-of-2 scaling factors, and stores forward activations as 1x128 tiles.
 * Format (a reading; the pages name it only): sign, 5 exponent bits with bias 15, 6 fraction bits;
 * exponent 31 holds infinities and NaN as in E5M2 and binary16; largest finite value 65024; subnormals
 * down to 2^-20. Encoding rounds to nearest even and saturates at +-65024, keeping the sign.
 * Packing: two 12-bit codes c0, c1 per 3 bytes, little-endian: byte0 = c0 & 0xFF,
 * byte1 = (c0 >> 8) | ((c1 & 0xF) << 4), byte2 = c1 >> 4; a row of cols values takes cols * 3 / 2 bytes. */

/* x bf16 [rows][cols] (row stride ld_x) -> packed u8 [rows][cols * 3 / 2] and scales f32 [cols/128][rows].
 * Per 1x128 tile: s = the smallest power of two >= RN_f32(max-abs / 65024) (max-abs 0 gives 1; scales
 * below FLT_MIN become FLT_MIN); codes encode x / s (exact). cols % 128 == 0, any rows.
 * x 16-byte aligned, ld_x % 8 == 0; packed 4-byte aligned; scales 4-byte aligned. rows == 0: no-op. */
fg_status fg_quantize_e5m6_1x128(const void* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* packed,
                                 float* scales, hipStream_t stream);

/* packed, scales as written by fg_quantize_e5m6_1x128 -> y bf16 [rows][cols] (row stride ld_y):
 * y = bf16(RN_f32(decoded code * s)), exact for every value inside bf16's range.
 * cols % 128 == 0; y 16-byte aligned, ld_y % 8 == 0, ld_y >= cols; packed, scales 4-byte aligned. */
fg_status fg_dequantize_e5m6_1x128(const uint8_t* packed, const float* scales, int64_t rows, int64_t cols, void* y,
                                   int64_t ld_y, hipStream_t stream);

/* ---- Per-tensor scaling: the contrast baseline ----------------------------------------------------
 * The usual FP8 recipe that the fine-grained tiles replace ([W1], the passage on aligning a whole
 * tensor's max-abs to the largest FP8 value and on its sensitivity to activation outliers) and its
 * delayed variant ([W4], the passage on delayed quantization, which infers the current max-abs from a
 * history kept over earlier iterations). */

/* Max-abs of a bf16 tensor.
 *   x     bf16 [rows][cols], row stride ld_x; cols % 8 == 0, ld_x % 8 == 0, x 16-byte aligned;
 *         rows * cols < 2^34.
 *   amax  DEVICE float, 4-byte aligned: on completion *amax = max(*amax, max |x|). It is an atomic max on
 *         the float's bits, so *amax must hold a non-negative float on entry (0 for the tensor's own
 *         max-abs). The max-abs is exact (a bf16 value).
 *   rows == 0 or cols == 0: no-op. */
fg_status fg_amax_bf16(const void* x, int64_t rows, int64_t cols, int64_t ld_x, float* amax, hipStream_t stream);

typedef enum {
    FG_LAYOUT_ACT_1x128 = 0,   /* f32 [cols/128][rows], as fg_quantize_act_1x128 along the columns */
    FG_LAYOUT_W_128x128 = 1    /* f32 [ceil(rows/128)][cols/128], as fg_quantize_w_128x128         */
} fg_scale_layout;

/* One scale for the whole tensor, taken from a device-resident max-abs history:
 *   A = max over i < n_hist of |amax_hist[i]|, rounded up to a bf16 value and capped at the largest
 *       finite bf16 (A = 0 for n_hist == 0);
 *   s = the scale rule of the 1x128 quantizers applied to A (A == 0 gives s = 1; mode as there);
 *   q = E4M3 code of RN_f32(x / s); quotients beyond +-448 (values above A) saturate to +-448.
 * n_hist == 1 holding the tensor's own max-abs (from fg_amax_bf16) is current per-tensor scaling, two
 * reads of x. Earlier iterations' max-abs values are delayed scaling, one read.
 *   x        bf16 [rows][cols], row stride ld_x; cols % 128 == 0; any rows; rows * cols < 2^34.
 *   amax_hist DEVICE floats, finite; 0 <= n_hist <= 4096.
 *   q        u8 [rows][cols] (row stride cols).
 *   scales   every entry set to s, in `layout`, so the GEMMs of this header take q and scales unchanged.
 *   amax_out NULL, or a DEVICE float outside amax_hist[0, n_hist): *amax_out = max(*amax_out, max |x|),
 *            as fg_amax_bf16 (records this tensor's max-abs for the next iteration's history).
 *   Alignment: x, q 16-byte aligned; ld_x % 8 == 0; scales, amax_hist, amax_out 4-byte aligned.
 *   rows == 0: no-op. */
fg_status fg_quantize_per_tensor(const void* x, int64_t rows, int64_t cols, int64_t ld_x, const float* amax_hist,
                                 int64_t n_hist, fg_scale_mode mode, fg_scale_layout layout, uint8_t* q,
                                 float* scales, float* amax_out, hipStream_t stream);

/* Static description of a status code. */
const char* fg_status_string(fg_status s);

/* hipError_t (as int) of the most recent FG_ERR_HIP on the calling thread; 0 if none. */
int fg_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8FG_H */
