// C-ABI entry points of libfp8fg: host-side argument checks, then one kernel launch on the caller's
// stream. Declarations, layouts and error behaviour: include/fp8fg.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8fg.h"

hipError_t fg_launch_quant_act_cols(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, int pow2,
                                    uint8_t* q, float* scales, hipStream_t stream);
hipError_t fg_launch_quant_act_rows(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, int pow2,
                                    uint8_t* q, float* scales, hipStream_t stream);
hipError_t fg_launch_requant_rows(const uint8_t* q_in, const float* s_in, int64_t rows, int64_t cols, int pow2,
                                  uint8_t* q, float* scales, hipStream_t stream);
hipError_t fg_launch_quant_w(const uint16_t* w, int64_t n, int64_t k, int64_t ld, int pow2, uint8_t* q,
                             float* scales, hipStream_t stream);
hipError_t fg_launch_gemm_grouped_dgrad(const uint8_t* dyq, const float* sdy, const uint8_t* wq, const float* sw,
                                        const int32_t* offsets, int32_t G, int64_t T, int64_t N, int64_t K, void* dx,
                                        int out_bf16, int pow2, hipStream_t stream);
hipError_t fg_launch_gemm_grouped_wgrad(const uint8_t* dytq, const float* sdyt, const uint8_t* xtq, const float* sxt,
                                        const int32_t* offsets, int32_t G, int64_t T, int64_t N, int64_t K, float* dw,
                                        int accumulate, int pow2, hipStream_t stream);
hipError_t fg_launch_quant_act_both(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, int pow2,
                                    uint8_t* qc, float* sc, uint8_t* qr, float* sr, hipStream_t stream);
hipError_t fg_launch_quant_x_both_w(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, uint8_t* qc, float* sc,
                                    uint8_t* qr, float* sr, const uint16_t* w, int64_t n, int64_t ldw, uint8_t* qw,
                                    float* sw, int pow2, hipStream_t stream);
hipError_t fg_launch_gemm_fprop(const uint8_t* xq, const float* sx, const uint8_t* wq, const float* sw, int64_t M,
                                int64_t N, int64_t K, void* y, int out_bf16, int pow2, hipStream_t stream);
hipError_t fg_launch_gemm_fprop_quant(const uint8_t* xq, const float* sx, const uint8_t* wq, const float* sw,
                                      int64_t M, int64_t N, int64_t K, uint8_t* yq, float* sy, int pow2, int out_pow2,
                                      hipStream_t stream);
hipError_t fg_launch_gemm_dgrad(const uint8_t* dyq, const float* sdy, const uint8_t* wq, const float* sw, int64_t M,
                                int64_t N, int64_t K, void* dx, int out_bf16, int pow2, hipStream_t stream);
hipError_t fg_launch_gemm_wgrad(const uint8_t* dytq, const float* sdyt, const uint8_t* xtq, const float* sxt,
                                int64_t M, int64_t N, int64_t K, float* dw, int accumulate, int pow2, hipStream_t stream);
hipError_t fg_launch_gemm_grouped(const uint8_t* xq, const float* sx, const uint8_t* wq, const float* sw,
                                  const int32_t* offsets, int32_t G, int64_t T, int64_t N, int64_t K, void* y,
                                  int out_bf16, int pow2, hipStream_t stream);

hipError_t fg_launch_quant_e5m6(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, uint8_t* packed,
                                float* scales, hipStream_t stream);
hipError_t fg_launch_dequant_e5m6(const uint8_t* packed, const float* scales, int64_t rows, int64_t cols, uint16_t* y,
                                  int64_t ldy, hipStream_t stream);
hipError_t fg_launch_fprop_limited(const uint8_t* xq, const float* sx, const uint8_t* wq, const float* sw, int64_t M,
                                   int64_t N, int64_t K, int bits, float* y, hipStream_t stream);
hipError_t fg_launch_amax(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, float* amax, hipStream_t stream);
hipError_t fg_launch_quant_per_tensor(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, const float* hist,
                                      int64_t n_hist, int pow2, int64_t n_scales, uint8_t* q, float* scales,
                                      float* amax_out, hipStream_t stream);

namespace {

thread_local int g_last_hip_error = 0;

// Grid limits of the launchers: 2^31-1 workgroups in x, 65535 in y.
constexpr int64_t kMaxGridX = 2147483647LL;
constexpr int64_t kMaxGridY = 65535LL;
constexpr int64_t kMaxGemmTiles = 2147483647LL;
constexpr int32_t kMaxGroups = 65536;
// The grouped GEMMs' grid covers the worst-case row tiles (rows / 256 + G) rounded up to a multiple of 8;
// the host bounds that padded count times the column tiles.
constexpr int64_t kGroupedRowPad = 7;
constexpr int64_t kMaxFlatChunks = 1LL << 31;   // per-tensor kernels index 16 B chunks in 32 bits
// The GEMM kernels address a tile's operand rows with 32-bit offsets from the tile base: up to 255 rows of
// the contraction length (A, and B stored [N][K]), and up to 128 rows of the output width for the
// transposed B of Dgrad. These bounds keep every such offset below 2^32.
constexpr int64_t kMaxContraction = 1LL << 24;
constexpr int64_t kMaxTransposedWidth = 1LL << 25;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

fg_status from_hip(hipError_t e) {
    if (e == hipSuccess) return FG_OK;
    g_last_hip_error = (int)e;
    return FG_ERR_HIP;
}

bool valid_mode(int m) { return m == FG_SCALE_FP32 || m == FG_SCALE_POW2; }
bool valid_out(int o) { return o == FG_OUT_F32 || o == FG_OUT_BF16; }

// Size arithmetic on caller-supplied extents, free of signed overflow for any non-negative input.
int64_t cdiv(int64_t a, int64_t b) { return a / b + (a % b != 0); }        // ceil(a / b), a >= 0, b > 0
bool prod_over(int64_t a, int64_t b, int64_t limit) { return a != 0 && b > limit / a; }   // a * b > limit
// Output tiles of a GEMM counted at the finest tile any launch uses (256 x 128): more than the grid holds?
bool too_many_tiles(int64_t a, int64_t b) { return prod_over(cdiv(a, 256), cdiv(b, 128), kMaxGemmTiles); }

}  // namespace

extern "C" {

fg_status fg_quantize_e5m6_1x128(const void* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* packed,
                                 float* scales, hipStream_t stream) {
    if (rows < 0 || cols < 0 || ld_x < cols) return FG_ERR_INVALID_ARG;
    if (rows == 0 || cols == 0) return FG_OK;
    if (!x || !packed || !scales) return FG_ERR_INVALID_ARG;
    if (cols % 128 != 0) return FG_ERR_UNSUPPORTED_SHAPE;
    if (!aligned16(x) || (ld_x % 8) != 0 || !aligned4(packed) || !aligned4(scales)) return FG_ERR_MISALIGNED;
    if (prod_over(cols / 128, cdiv(rows, 32), kMaxGridX)) return FG_ERR_UNSUPPORTED_SHAPE;
    return from_hip(fg_launch_quant_e5m6((const uint16_t*)x, rows, cols, ld_x, packed, scales, stream));
}

fg_status fg_dequantize_e5m6_1x128(const uint8_t* packed, const float* scales, int64_t rows, int64_t cols, void* y,
                                   int64_t ld_y, hipStream_t stream) {
    if (rows < 0 || cols < 0 || ld_y < cols) return FG_ERR_INVALID_ARG;
    if (rows == 0 || cols == 0) return FG_OK;
    if (!packed || !scales || !y) return FG_ERR_INVALID_ARG;
    if (cols % 128 != 0) return FG_ERR_UNSUPPORTED_SHAPE;
    if (!aligned16(y) || (ld_y % 8) != 0 || !aligned4(packed) || !aligned4(scales)) return FG_ERR_MISALIGNED;
    if (prod_over(cols / 128, cdiv(rows, 32), kMaxGridX)) return FG_ERR_UNSUPPORTED_SHAPE;
    return from_hip(fg_launch_dequant_e5m6(packed, scales, rows, cols, (uint16_t*)y, ld_y, stream));
}

fg_status fg_fp8_gemm_fprop_limited_accum(const uint8_t* xq, const float* sx, const uint8_t* wq, const float* sw,
                                          int64_t M, int64_t N, int64_t K, int mantissa_bits, float* y,
                                          hipStream_t stream) {
    if (M < 0 || N < 0 || K < 0 || mantissa_bits < 1 || mantissa_bits > 23) return FG_ERR_INVALID_ARG;
    if (M == 0 || N == 0) return FG_OK;
    if (!y || (K > 0 && (!xq || !sx || !wq || !sw))) return FG_ERR_INVALID_ARG;
    if (K % 128 != 0 || prod_over(cdiv(M, 16), cdiv(N, 16), kMaxGridX)) return FG_ERR_UNSUPPORTED_SHAPE;
    if (((uintptr_t)xq & 7u) || ((uintptr_t)wq & 7u) || !aligned4(y) || !aligned4(sx) || !aligned4(sw))
        return FG_ERR_MISALIGNED;
    return from_hip(fg_launch_fprop_limited(xq, sx, wq, sw, M, N, K, mantissa_bits, y, stream));
}

fg_status fg_amax_bf16(const void* x, int64_t rows, int64_t cols, int64_t ld_x, float* amax, hipStream_t stream) {
    if (rows < 0 || cols < 0 || ld_x < cols) return FG_ERR_INVALID_ARG;
    if (rows == 0 || cols == 0) return FG_OK;
    if (!x || !amax) return FG_ERR_INVALID_ARG;
    if (cols % 8 != 0 || prod_over(rows, cols / 8, kMaxFlatChunks - 1)) return FG_ERR_UNSUPPORTED_SHAPE;
    if (!aligned16(x) || !aligned4(amax) || (ld_x % 8) != 0) return FG_ERR_MISALIGNED;
    return from_hip(fg_launch_amax((const uint16_t*)x, rows, cols, ld_x, amax, stream));
}

fg_status fg_quantize_per_tensor(const void* x, int64_t rows, int64_t cols, int64_t ld_x, const float* amax_hist,
                                 int64_t n_hist, fg_scale_mode mode, fg_scale_layout layout, uint8_t* q,
                                 float* scales, float* amax_out, hipStream_t stream) {
    if (rows < 0 || cols < 0 || ld_x < cols || n_hist < 0 || !valid_mode(mode) ||
        (layout != FG_LAYOUT_ACT_1x128 && layout != FG_LAYOUT_W_128x128))
        return FG_ERR_INVALID_ARG;
    if (rows == 0) return FG_OK;
    if (!x || !q || !scales || (n_hist > 0 && !amax_hist)) return FG_ERR_INVALID_ARG;
    if (amax_out && n_hist > 0 && amax_out >= amax_hist && amax_out < amax_hist + n_hist) return FG_ERR_INVALID_ARG;
    if (cols % 128 != 0 || n_hist > 4096 || prod_over(rows, cols / 8, kMaxFlatChunks - 1)) return FG_ERR_UNSUPPORTED_SHAPE;
    if (cols == 0) return FG_OK;
    if (!aligned16(x) || !aligned16(q) || (ld_x % 8) != 0 || !aligned4(scales) || (amax_hist && !aligned4(amax_hist)) ||
        (amax_out && !aligned4(amax_out)))
        return FG_ERR_MISALIGNED;
    const int64_t n_scales = layout == FG_LAYOUT_ACT_1x128 ? (cols / 128) * rows : ((rows + 127) / 128) * (cols / 128);
    return from_hip(fg_launch_quant_per_tensor((const uint16_t*)x, rows, cols, ld_x, amax_hist, n_hist,
                                               mode == FG_SCALE_POW2, n_scales, q, scales, amax_out, stream));
}

const char* fg_status_string(fg_status s) {
    switch (s) {
        case FG_OK: return "ok";
        case FG_ERR_INVALID_ARG: return "invalid argument";
        case FG_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
        case FG_ERR_MISALIGNED: return "misaligned pointer or leading dimension";
        case FG_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

int fg_last_hip_error(void) { return g_last_hip_error; }

fg_status fg_quantize_act_1x128(const void* x, int64_t rows, int64_t cols, int64_t ld_x, fg_tile_axis axis,
                                fg_scale_mode mode, uint8_t* q, float* scales, hipStream_t stream) {
    if (rows < 0 || cols < 0 || !valid_mode(mode) || (axis != FG_ALONG_COLS && axis != FG_ALONG_ROWS))
        return FG_ERR_INVALID_ARG;
    if (ld_x < cols) return FG_ERR_INVALID_ARG;
    if (rows == 0 || cols == 0) return FG_OK;
    if (!x || !q || !scales) return FG_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(q) || !aligned4(scales) || (ld_x % 8) != 0) return FG_ERR_MISALIGNED;
    const int pow2 = mode == FG_SCALE_POW2;
    if (axis == FG_ALONG_COLS) {
        if (cols % 128 != 0) return FG_ERR_UNSUPPORTED_SHAPE;
        if (prod_over(cols / 128, cdiv(rows, 32), kMaxGridX)) return FG_ERR_UNSUPPORTED_SHAPE;
        return from_hip(fg_launch_quant_act_cols((const uint16_t*)x, rows, cols, ld_x, pow2, q, scales, stream));
    }
    if (rows % 128 != 0 || cols % 8 != 0) return FG_ERR_UNSUPPORTED_SHAPE;
    if (cdiv(cols, 64) > kMaxGridY || rows / 128 > kMaxGridX) return FG_ERR_UNSUPPORTED_SHAPE;
    return from_hip(fg_launch_quant_act_rows((const uint16_t*)x, rows, cols, ld_x, pow2, q, scales, stream));
}

fg_status fg_quantize_act_1x128_both(const void* x, int64_t rows, int64_t cols, int64_t ld_x, fg_scale_mode mode,
                                     uint8_t* q_cols, float* scales_cols, uint8_t* q_rows, float* scales_rows,
                                     hipStream_t stream) {
    if (rows < 0 || cols < 0 || !valid_mode(mode) || ld_x < cols) return FG_ERR_INVALID_ARG;
    if (rows == 0 || cols == 0) return FG_OK;
    if (!x || !q_cols || !scales_cols || !q_rows || !scales_rows) return FG_ERR_INVALID_ARG;
    if (rows % 128 != 0 || cols % 128 != 0) return FG_ERR_UNSUPPORTED_SHAPE;
    if (!aligned16(x) || !aligned16(q_cols) || !aligned16(q_rows) || !aligned4(scales_cols) || !aligned4(scales_rows) ||
        (ld_x % 8) != 0)
        return FG_ERR_MISALIGNED;
    if (cols / 128 > kMaxGridY || rows / 128 > kMaxGridX) return FG_ERR_UNSUPPORTED_SHAPE;
    return from_hip(fg_launch_quant_act_both((const uint16_t*)x, rows, cols, ld_x, mode == FG_SCALE_POW2, q_cols,
                                             scales_cols, q_rows, scales_rows, stream));
}

fg_status fg_quantize_fprop_operands(const void* x, int64_t rows, int64_t ld_x, const void* w, int64_t n, int64_t ld_w,
                                     int64_t k, fg_scale_mode mode, uint8_t* q_cols, float* scales_cols,
                                     uint8_t* q_rows, float* scales_rows, uint8_t* qw, float* sw, hipStream_t stream) {
    if (rows < 0 || n < 0 || k < 0 || !valid_mode(mode)) return FG_ERR_INVALID_ARG;
    // a tensor with no rows is not read: its pointers and row stride are ignored
    if ((rows > 0 && ld_x < k) || (n > 0 && ld_w < k)) return FG_ERR_INVALID_ARG;
    const bool has_x = rows > 0 && k > 0, has_w = n > 0 && k > 0;
    if (!has_x && !has_w) return FG_OK;
    if (has_x && (!x || !q_cols || !scales_cols || !q_rows || !scales_rows)) return FG_ERR_INVALID_ARG;
    if (has_w && (!w || !qw || !sw)) return FG_ERR_INVALID_ARG;
    if (rows % 128 != 0 || k % 128 != 0) return FG_ERR_UNSUPPORTED_SHAPE;
    if (has_x && (!aligned16(x) || !aligned16(q_cols) || !aligned16(q_rows) || !aligned4(scales_cols) ||
                  !aligned4(scales_rows) || (ld_x % 8) != 0))
        return FG_ERR_MISALIGNED;
    if (has_w && (!aligned16(w) || !aligned16(qw) || !aligned4(sw) || (ld_w % 8) != 0)) return FG_ERR_MISALIGNED;
    // X blocks plus W blocks, one workgroup each, in a one-dimensional grid
    const int64_t kb = k / 128;
    const int64_t xb = rows / 128, wb = cdiv(n, 128);
    if (prod_over(xb + wb, kb, kMaxGridX)) return FG_ERR_UNSUPPORTED_SHAPE;
    return from_hip(fg_launch_quant_x_both_w((const uint16_t*)x, has_x ? rows : 0, k, ld_x, q_cols, scales_cols, q_rows,
                                             scales_rows, (const uint16_t*)w, has_w ? n : 0, ld_w, qw, sw,
                                             mode == FG_SCALE_POW2, stream));
}

fg_status fg_requantize_1x128_to_tokens(const uint8_t* q_in, const float* s_in, int64_t rows, int64_t cols,
                                        fg_scale_mode mode, uint8_t* q_out, float* s_out, hipStream_t stream) {
    if (rows < 0 || cols < 0 || !valid_mode(mode)) return FG_ERR_INVALID_ARG;
    if (rows == 0 || cols == 0) return FG_OK;
    if (!q_in || !s_in || !q_out || !s_out) return FG_ERR_INVALID_ARG;
    if (rows % 128 != 0 || cols % 128 != 0) return FG_ERR_UNSUPPORTED_SHAPE;
    if (!aligned16(q_in) || !aligned16(s_in) || !aligned16(q_out) || !aligned4(s_out)) return FG_ERR_MISALIGNED;
    if (cols / 64 > kMaxGridY || rows / 128 > kMaxGridX) return FG_ERR_UNSUPPORTED_SHAPE;
    return from_hip(fg_launch_requant_rows(q_in, s_in, rows, cols, mode == FG_SCALE_POW2, q_out, s_out, stream));
}

fg_status fg_quantize_w_128x128(const void* w, int64_t n, int64_t k, int64_t ld_w, fg_scale_mode mode, uint8_t* q,
                                float* scales, hipStream_t stream) {
    if (n < 0 || k < 0 || !valid_mode(mode) || ld_w < k) return FG_ERR_INVALID_ARG;
    if (n == 0 || k == 0) return FG_OK;
    if (!w || !q || !scales) return FG_ERR_INVALID_ARG;
    if (k % 128 != 0) return FG_ERR_UNSUPPORTED_SHAPE;
    if (!aligned16(w) || !aligned16(q) || !aligned4(scales) || (ld_w % 8) != 0) return FG_ERR_MISALIGNED;
    if (cdiv(n, 128) > kMaxGridY || k / 128 > kMaxGridX) return FG_ERR_UNSUPPORTED_SHAPE;
    return from_hip(fg_launch_quant_w((const uint16_t*)w, n, k, ld_w, mode == FG_SCALE_POW2, q, scales, stream));
}

fg_status fg_fp8_gemm_fprop(const uint8_t* xq, const float* sx, const uint8_t* wq, const float* sw, int64_t M,
                            int64_t N, int64_t K, void* y, fg_out_dtype out, fg_scale_mode scales, hipStream_t stream) {
    if (M < 0 || N < 0 || K < 0 || !valid_out(out) || !valid_mode(scales)) return FG_ERR_INVALID_ARG;
    if (M == 0 || N == 0) return FG_OK;
    if (!y || (K > 0 && (!xq || !sx || !wq || !sw))) return FG_ERR_INVALID_ARG;
    if (K % 128 != 0 || K > kMaxContraction || too_many_tiles(M, N)) return FG_ERR_UNSUPPORTED_SHAPE;
    if (!aligned16(xq) || !aligned16(wq) || !aligned16(y) || !aligned4(sx) || !aligned4(sw)) return FG_ERR_MISALIGNED;
    return from_hip(fg_launch_gemm_fprop(xq, sx, wq, sw, M, N, K, y, out == FG_OUT_BF16, scales == FG_SCALE_POW2, stream));
}

fg_status fg_fp8_gemm_fprop_quant(const uint8_t* xq, const float* sx, const uint8_t* wq, const float* sw, int64_t M,
                                  int64_t N, int64_t K, uint8_t* yq, float* sy, fg_scale_mode scales,
                                  fg_scale_mode out_scales, hipStream_t stream) {
    if (M < 0 || N < 0 || K < 0 || !valid_mode(scales) || !valid_mode(out_scales)) return FG_ERR_INVALID_ARG;
    if (M == 0 || N == 0) return FG_OK;
    if (!yq || !sy || (K > 0 && (!xq || !sx || !wq || !sw))) return FG_ERR_INVALID_ARG;
    if (N % 128 != 0 || K % 128 != 0 || K > kMaxContraction || too_many_tiles(M, N))
        return FG_ERR_UNSUPPORTED_SHAPE;
    if (!aligned16(xq) || !aligned16(wq) || !aligned16(yq) || !aligned4(sx) || !aligned4(sw) || !aligned4(sy))
        return FG_ERR_MISALIGNED;
    return from_hip(fg_launch_gemm_fprop_quant(xq, sx, wq, sw, M, N, K, yq, sy, scales == FG_SCALE_POW2,
                                               out_scales == FG_SCALE_POW2, stream));
}

fg_status fg_fp8_gemm_dgrad(const uint8_t* dyq, const float* sdy, const uint8_t* wq, const float* sw, int64_t M,
                            int64_t N, int64_t K, void* dx, fg_out_dtype out, fg_scale_mode scales, hipStream_t stream) {
    if (M < 0 || N < 0 || K < 0 || !valid_out(out) || !valid_mode(scales)) return FG_ERR_INVALID_ARG;
    if (M == 0 || K == 0) return FG_OK;
    if (!dx || (N > 0 && (!dyq || !sdy || !wq || !sw))) return FG_ERR_INVALID_ARG;
    if (N % 128 != 0 || K % 128 != 0 || N > kMaxContraction || K > kMaxTransposedWidth || too_many_tiles(M, K))
        return FG_ERR_UNSUPPORTED_SHAPE;
    if (!aligned16(dyq) || !aligned16(wq) || !aligned16(dx) || !aligned4(sdy) || !aligned4(sw)) return FG_ERR_MISALIGNED;
    return from_hip(fg_launch_gemm_dgrad(dyq, sdy, wq, sw, M, N, K, dx, out == FG_OUT_BF16, scales == FG_SCALE_POW2, stream));
}

fg_status fg_fp8_gemm_wgrad(const uint8_t* dytq, const float* sdyt, const uint8_t* xtq, const float* sxt, int64_t M,
                            int64_t N, int64_t K, float* dw, int accumulate, fg_scale_mode scales, hipStream_t stream) {
    if (M < 0 || N < 0 || K < 0 || !valid_mode(scales)) return FG_ERR_INVALID_ARG;
    if (N == 0 || K == 0) return FG_OK;
    if (!dw || (M > 0 && (!dytq || !sdyt || !xtq || !sxt))) return FG_ERR_INVALID_ARG;
    if (M % 128 != 0 || K % 4 != 0 || M > kMaxContraction || too_many_tiles(N, K)) return FG_ERR_UNSUPPORTED_SHAPE;
    if (!aligned16(dytq) || !aligned16(xtq) || !aligned16(dw) || !aligned16(sxt) || !aligned4(sdyt))
        return FG_ERR_MISALIGNED;
    return from_hip(fg_launch_gemm_wgrad(dytq, sdyt, xtq, sxt, M, N, K, dw, accumulate != 0, scales == FG_SCALE_POW2, stream));
}

fg_status fg_fp8_grouped_gemm(const uint8_t* xq, const float* sx, const uint8_t* wq, const float* sw,
                              const int32_t* d_offsets, int32_t G, int64_t total_rows, int64_t N, int64_t K, void* y,
                              fg_out_dtype out, fg_scale_mode scales, hipStream_t stream) {
    if (G < 1 || G > kMaxGroups || total_rows < 0 || N < 0 || K < 0 || !valid_out(out) || !valid_mode(scales))
        return FG_ERR_INVALID_ARG;
    if (total_rows == 0 || N == 0) return FG_OK;
    if (!y || !d_offsets || (K > 0 && (!xq || !sx || !wq || !sw))) return FG_ERR_INVALID_ARG;
    if (K % 128 != 0 || K > kMaxContraction) return FG_ERR_UNSUPPORTED_SHAPE;
    if (prod_over(cdiv(total_rows, 256) + G + kGroupedRowPad, cdiv(N, 128), kMaxGemmTiles)) return FG_ERR_UNSUPPORTED_SHAPE;
    if (!aligned16(xq) || !aligned16(wq) || !aligned16(y) || !aligned4(sx) || !aligned4(sw) || !aligned4(d_offsets))
        return FG_ERR_MISALIGNED;
    return from_hip(fg_launch_gemm_grouped(xq, sx, wq, sw, d_offsets, G, total_rows, N, K, y, out == FG_OUT_BF16,
                                           scales == FG_SCALE_POW2, stream));
}

fg_status fg_fp8_grouped_gemm_dgrad(const uint8_t* dyq, const float* sdy, const uint8_t* wq, const float* sw,
                                    const int32_t* d_offsets, int32_t G, int64_t total_rows, int64_t N, int64_t K,
                                    void* dx, fg_out_dtype out, fg_scale_mode scales, hipStream_t stream) {
    if (G < 1 || G > kMaxGroups || total_rows < 0 || N < 0 || K < 0 || !valid_out(out) || !valid_mode(scales))
        return FG_ERR_INVALID_ARG;
    if (total_rows == 0 || K == 0) return FG_OK;
    if (!dx || !d_offsets || (N > 0 && (!dyq || !sdy || !wq || !sw))) return FG_ERR_INVALID_ARG;
    if (N % 128 != 0 || K % 128 != 0 || N > kMaxContraction || K > kMaxTransposedWidth) return FG_ERR_UNSUPPORTED_SHAPE;
    if (prod_over(cdiv(total_rows, 256) + G + kGroupedRowPad, cdiv(K, 128), kMaxGemmTiles)) return FG_ERR_UNSUPPORTED_SHAPE;
    if (!aligned16(dyq) || !aligned16(wq) || !aligned16(dx) || !aligned4(sdy) || !aligned4(sw) || !aligned4(d_offsets))
        return FG_ERR_MISALIGNED;
    return from_hip(fg_launch_gemm_grouped_dgrad(dyq, sdy, wq, sw, d_offsets, G, total_rows, N, K, dx, out == FG_OUT_BF16,
                                                 scales == FG_SCALE_POW2, stream));
}

fg_status fg_fp8_grouped_gemm_wgrad(const uint8_t* dytq, const float* sdyt, const uint8_t* xtq, const float* sxt,
                                    const int32_t* d_offsets, int32_t G, int64_t total_rows, int64_t N, int64_t K,
                                    float* dw, int accumulate, fg_scale_mode scales, hipStream_t stream) {
    if (G < 1 || G > kMaxGroups || total_rows < 0 || N < 0 || K < 0 || !valid_mode(scales)) return FG_ERR_INVALID_ARG;
    if (N == 0 || K == 0) return FG_OK;
    if (!dw || !d_offsets || (total_rows > 0 && (!dytq || !sdyt || !xtq || !sxt))) return FG_ERR_INVALID_ARG;
    if (total_rows % 128 != 0 || K % 4 != 0 || total_rows > kMaxContraction) return FG_ERR_UNSUPPORTED_SHAPE;
    if (too_many_tiles(N, K) || prod_over(cdiv(N, 256) * cdiv(K, 128), G, kMaxGemmTiles))
        return FG_ERR_UNSUPPORTED_SHAPE;
    if (!aligned16(dytq) || !aligned16(xtq) || !aligned16(dw) || !aligned16(sxt) || !aligned4(sdyt) ||
        !aligned4(d_offsets))
        return FG_ERR_MISALIGNED;
    return from_hip(fg_launch_gemm_grouped_wgrad(dytq, sdyt, xtq, sxt, d_offsets, G, total_rows, N, K, dw,
                                                 accumulate != 0, scales == FG_SCALE_POW2, stream));
}

}  // extern "C"
