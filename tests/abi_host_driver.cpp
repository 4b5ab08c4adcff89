// Host-side checks of the C ABI (fp8_fine_grained_amax_amd/csrc/api.hip) with every kernel launcher
// replaced by a recording stub, for a build with AddressSanitizer and UndefinedBehaviorSanitizer
// (tests/test_abi_sanitized.py). Each entry point is driven through its rejection paths (a status, and
// no launcher reached) and its accept paths (FG_OK, exactly one launcher call with the translated
// arguments), and a launcher error must come back as FG_ERR_HIP with the HIP code kept per thread.
// Exit status 0 and no sanitizer report: the argument checks read nothing out of bounds and overflow no
// integer on any path driven here.
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "fp8fg.h"

namespace {
struct Call {
    const char* name = nullptr;
    int64_t v[6] = {0, 0, 0, 0, 0, 0};
    int flags[3] = {0, 0, 0};
};
Call g_last;
int g_calls = 0;
hipError_t g_ret = hipSuccess;
int g_failures = 0;

hipError_t rec(const char* name, int64_t a, int64_t b, int64_t c, int64_t d = 0, int f0 = 0, int f1 = 0, int f2 = 0) {
    g_last = Call{};
    g_last.name = name;
    g_last.v[0] = a; g_last.v[1] = b; g_last.v[2] = c; g_last.v[3] = d;
    g_last.flags[0] = f0; g_last.flags[1] = f1; g_last.flags[2] = f2;
    g_calls++;
    return g_ret;
}
}  // namespace

// ---- recording launchers (same signatures as the library's) ----
hipError_t fg_launch_quant_act_cols(const uint16_t*, int64_t rows, int64_t cols, int64_t ld, int pow2, uint8_t*, float*,
                                    hipStream_t) { return rec("quant_act_cols", rows, cols, ld, 0, pow2); }
hipError_t fg_launch_quant_act_rows(const uint16_t*, int64_t rows, int64_t cols, int64_t ld, int pow2, uint8_t*, float*,
                                    hipStream_t) { return rec("quant_act_rows", rows, cols, ld, 0, pow2); }
hipError_t fg_launch_requant_rows(const uint8_t*, const float*, int64_t rows, int64_t cols, int pow2, uint8_t*, float*,
                                  hipStream_t) { return rec("requant_rows", rows, cols, 0, 0, pow2); }
hipError_t fg_launch_quant_w(const uint16_t*, int64_t n, int64_t k, int64_t ld, int pow2, uint8_t*, float*, hipStream_t) {
    return rec("quant_w", n, k, ld, 0, pow2);
}
hipError_t fg_launch_quant_act_both(const uint16_t*, int64_t rows, int64_t cols, int64_t ld, int pow2, uint8_t*, float*,
                                    uint8_t*, float*, hipStream_t) { return rec("quant_act_both", rows, cols, ld, 0, pow2); }
hipError_t fg_launch_quant_x_both_w(const uint16_t*, int64_t rows, int64_t cols, int64_t ldx, uint8_t*, float*, uint8_t*,
                                    float*, const uint16_t*, int64_t n, int64_t ldw, uint8_t*, float*, int pow2,
                                    hipStream_t) { return rec("quant_x_both_w", rows, cols, ldx, n, pow2, (int)ldw); }
hipError_t fg_launch_gemm_fprop(const uint8_t*, const float*, const uint8_t*, const float*, int64_t M, int64_t N,
                                int64_t K, void*, int out_bf16, int pow2, hipStream_t) {
    return rec("gemm_fprop", M, N, K, 0, out_bf16, pow2);
}
hipError_t fg_launch_gemm_fprop_quant(const uint8_t*, const float*, const uint8_t*, const float*, int64_t M, int64_t N,
                                      int64_t K, uint8_t*, float*, int pow2, int out_pow2, hipStream_t) {
    return rec("gemm_fprop_quant", M, N, K, 0, pow2, out_pow2);
}
hipError_t fg_launch_gemm_dgrad(const uint8_t*, const float*, const uint8_t*, const float*, int64_t M, int64_t N,
                                int64_t K, void*, int out_bf16, int pow2, hipStream_t) {
    return rec("gemm_dgrad", M, N, K, 0, out_bf16, pow2);
}
hipError_t fg_launch_gemm_wgrad(const uint8_t*, const float*, const uint8_t*, const float*, int64_t M, int64_t N,
                                int64_t K, float*, int accumulate, int pow2, hipStream_t) {
    return rec("gemm_wgrad", M, N, K, 0, accumulate, pow2);
}
hipError_t fg_launch_gemm_grouped(const uint8_t*, const float*, const uint8_t*, const float*, const int32_t*, int32_t G,
                                  int64_t T, int64_t N, int64_t K, void*, int out_bf16, int pow2, hipStream_t) {
    return rec("gemm_grouped", T, N, K, G, out_bf16, pow2);
}
hipError_t fg_launch_gemm_grouped_dgrad(const uint8_t*, const float*, const uint8_t*, const float*, const int32_t*,
                                        int32_t G, int64_t T, int64_t N, int64_t K, void*, int out_bf16, int pow2,
                                        hipStream_t) {
    return rec("gemm_grouped_dgrad", T, N, K, G, out_bf16, pow2);
}
hipError_t fg_launch_gemm_grouped_wgrad(const uint8_t*, const float*, const uint8_t*, const float*, const int32_t*,
                                        int32_t G, int64_t T, int64_t N, int64_t K, float*, int accumulate, int pow2,
                                        hipStream_t) {
    return rec("gemm_grouped_wgrad", T, N, K, G, accumulate, pow2);
}
hipError_t fg_launch_quant_e5m6(const uint16_t*, int64_t rows, int64_t cols, int64_t ld, uint8_t*, float*, hipStream_t) {
    return rec("quant_e5m6", rows, cols, ld);
}
hipError_t fg_launch_dequant_e5m6(const uint8_t*, const float*, int64_t rows, int64_t cols, uint16_t*, int64_t ldy,
                                  hipStream_t) { return rec("dequant_e5m6", rows, cols, ldy); }
hipError_t fg_launch_fprop_limited(const uint8_t*, const float*, const uint8_t*, const float*, int64_t M, int64_t N,
                                   int64_t K, int bits, float*, hipStream_t) { return rec("fprop_limited", M, N, K, bits); }
hipError_t fg_launch_amax(const uint16_t*, int64_t rows, int64_t cols, int64_t ld, float*, hipStream_t) {
    return rec("amax", rows, cols, ld);
}
hipError_t fg_launch_quant_per_tensor(const uint16_t*, int64_t rows, int64_t cols, int64_t ld, const float*,
                                      int64_t n_hist, int pow2, int64_t n_scales, uint8_t*, float*, float*, hipStream_t) {
    return rec("quant_per_tensor", rows, cols, ld, n_scales, pow2, (int)n_hist);
}

// ---- checks ----
#define P16 ((void*)(uintptr_t)0x100000)
#define P16B ((void*)(uintptr_t)0x200000)
#define PODD ((void*)(uintptr_t)0x100004)
#define U8(p) ((uint8_t*)(p))
#define F32(p) ((float*)(p))
#define I32(p) ((int32_t*)(p))

static void expect(fg_status got, fg_status want, const char* launcher, int line) {
    // launcher == nullptr: nothing may be launched
    const bool launched = g_calls > 0;
    bool ok = got == want && (launcher ? (launched && g_calls == 1 && strcmp(g_last.name, launcher) == 0) : !launched);
    if (!ok) {
        printf("line %d: status %d (want %d), launcher %s (want %s), calls %d\n", line, (int)got, (int)want,
               launched ? g_last.name : "none", launcher ? launcher : "none", g_calls);
        g_failures++;
    }
    g_calls = 0;
}
#define REJECT(call, st) do { g_calls = 0; expect((call), (st), nullptr, __LINE__); } while (0)
#define ACCEPT(call, launcher) do { g_calls = 0; fg_status s_ = (call); const Call c_ = g_last; \
    expect(s_, FG_OK, (launcher), __LINE__); g_last = c_; } while (0)
#define NOOP(call) do { g_calls = 0; expect((call), FG_OK, nullptr, __LINE__); } while (0)
#define CHECK(cond) do { if (!(cond)) { printf("line %d: %s\n", __LINE__, #cond); g_failures++; } } while (0)

int main() {
    const fg_status INV = FG_ERR_INVALID_ARG, SHP = FG_ERR_UNSUPPORTED_SHAPE, MIS = FG_ERR_MISALIGNED;
    // 1x128 activations
    REJECT(fg_quantize_act_1x128(P16, -1, 128, 128, FG_ALONG_COLS, FG_SCALE_FP32, U8(P16), F32(P16), 0), INV);
    REJECT(fg_quantize_act_1x128(P16, 4, 128, 128, (fg_tile_axis)2, FG_SCALE_FP32, U8(P16), F32(P16), 0), INV);
    REJECT(fg_quantize_act_1x128(P16, 4, 128, 128, FG_ALONG_COLS, (fg_scale_mode)7, U8(P16), F32(P16), 0), INV);
    REJECT(fg_quantize_act_1x128(P16, 4, 128, 100, FG_ALONG_COLS, FG_SCALE_FP32, U8(P16), F32(P16), 0), INV);
    REJECT(fg_quantize_act_1x128(nullptr, 4, 128, 128, FG_ALONG_COLS, FG_SCALE_FP32, U8(P16), F32(P16), 0), INV);
    REJECT(fg_quantize_act_1x128(P16, 4, 100, 104, FG_ALONG_COLS, FG_SCALE_FP32, U8(P16), F32(P16), 0), SHP);
    REJECT(fg_quantize_act_1x128(P16, 100, 64, 64, FG_ALONG_ROWS, FG_SCALE_FP32, U8(P16), F32(P16), 0), SHP);
    REJECT(fg_quantize_act_1x128(P16, 128, 60, 64, FG_ALONG_ROWS, FG_SCALE_FP32, U8(P16), F32(P16), 0), SHP);
    REJECT(fg_quantize_act_1x128(PODD, 4, 128, 128, FG_ALONG_COLS, FG_SCALE_FP32, U8(P16), F32(P16), 0), MIS);
    REJECT(fg_quantize_act_1x128(P16, 4, 128, 132, FG_ALONG_COLS, FG_SCALE_FP32, U8(P16), F32(P16), 0), MIS);
    const int64_t huge = (INT64_MAX / 128) * 128;     // extents whose products and roundings overflow int64
    REJECT(fg_quantize_act_1x128(P16, 4, huge, huge, FG_ALONG_COLS, FG_SCALE_FP32, U8(P16), F32(P16), 0), SHP);
    REJECT(fg_quantize_act_1x128(P16, huge, 128, 128, FG_ALONG_COLS, FG_SCALE_FP32, U8(P16), F32(P16), 0), SHP);
    REJECT(fg_quantize_act_1x128(P16, huge, 128, 128, FG_ALONG_ROWS, FG_SCALE_FP32, U8(P16), F32(P16), 0), SHP);
    REJECT(fg_quantize_w_128x128(P16, INT64_MAX, 128, 128, FG_SCALE_FP32, U8(P16), F32(P16), 0), SHP);
    REJECT(fg_amax_bf16(P16, INT64_MAX, 128, 128, F32(P16B), 0), SHP);
    REJECT(fg_quantize_e5m6_1x128(P16, INT64_MAX, 128, 128, U8(P16), F32(P16), 0), SHP);
    REJECT(fg_fp8_gemm_fprop_limited_accum(U8(P16), F32(P16), U8(P16), F32(P16), INT64_MAX, INT64_MAX, 128, 10, F32(P16),
                                           0), SHP);
    NOOP(fg_quantize_act_1x128(nullptr, 0, 128, 128, FG_ALONG_COLS, FG_SCALE_FP32, nullptr, nullptr, 0));
    ACCEPT(fg_quantize_act_1x128(P16, 37, 384, 392, FG_ALONG_COLS, FG_SCALE_POW2, U8(P16), F32(P16), 0), "quant_act_cols");
    CHECK(g_last.v[0] == 37 && g_last.v[1] == 384 && g_last.v[2] == 392 && g_last.flags[0] == 1);
    ACCEPT(fg_quantize_act_1x128(P16, 256, 72, 72, FG_ALONG_ROWS, FG_SCALE_FP32, U8(P16), F32(P16), 0), "quant_act_rows");
    CHECK(g_last.v[0] == 256 && g_last.v[1] == 72 && g_last.flags[0] == 0);
    // both tilings
    REJECT(fg_quantize_act_1x128_both(P16, 100, 128, 128, FG_SCALE_FP32, U8(P16), F32(P16), U8(P16), F32(P16), 0), SHP);
    REJECT(fg_quantize_act_1x128_both(P16, 128, 128, 128, FG_SCALE_FP32, U8(P16), F32(P16), U8(PODD), F32(P16), 0), MIS);
    REJECT(fg_quantize_act_1x128_both(P16, 128, 128, 128, FG_SCALE_FP32, U8(P16), F32(P16), nullptr, F32(P16), 0), INV);
    ACCEPT(fg_quantize_act_1x128_both(P16, 256, 384, 384, FG_SCALE_POW2, U8(P16), F32(P16), U8(P16), F32(P16), 0),
           "quant_act_both");
    CHECK(g_last.v[0] == 256 && g_last.v[1] == 384 && g_last.flags[0] == 1);
    // X both tilings + W blocks in one launch
    REJECT(fg_quantize_fprop_operands(P16, 100, 128, P16, 256, 128, 128, FG_SCALE_FP32, U8(P16), F32(P16), U8(P16),
                                      F32(P16), U8(P16), F32(P16), 0), SHP);
    REJECT(fg_quantize_fprop_operands(P16, 128, 128, P16, 256, 128, 128, FG_SCALE_FP32, U8(P16), F32(P16), U8(P16),
                                      F32(P16), U8(PODD), F32(P16), 0), MIS);
    REJECT(fg_quantize_fprop_operands(P16, 128, 128, nullptr, 256, 128, 128, FG_SCALE_FP32, U8(P16), F32(P16), U8(P16),
                                      F32(P16), U8(P16), F32(P16), 0), INV);
    REJECT(fg_quantize_fprop_operands(P16, 128, 128, P16, 256, 120, 128, FG_SCALE_FP32, U8(P16), F32(P16), U8(P16),
                                      F32(P16), U8(P16), F32(P16), 0), INV);
    REJECT(fg_quantize_fprop_operands(P16, INT64_MAX - 127, INT64_MAX - 7, P16, INT64_MAX, INT64_MAX - 7, 128, FG_SCALE_FP32,
                                      U8(P16), F32(P16), U8(P16), F32(P16), U8(P16), F32(P16), 0), SHP);
    NOOP(fg_quantize_fprop_operands(nullptr, 0, 128, nullptr, 0, 128, 128, FG_SCALE_FP32, nullptr, nullptr, nullptr,
                                    nullptr, nullptr, nullptr, 0));
    ACCEPT(fg_quantize_fprop_operands(P16, 256, 392, P16, 300, 400, 384, FG_SCALE_POW2, U8(P16), F32(P16), U8(P16),
                                      F32(P16), U8(P16), F32(P16), 0), "quant_x_both_w");
    CHECK(g_last.v[0] == 256 && g_last.v[1] == 384 && g_last.v[2] == 392 && g_last.v[3] == 300 &&
          g_last.flags[0] == 1 && g_last.flags[1] == 400);
    ACCEPT(fg_quantize_fprop_operands(nullptr, 0, 128, P16, 300, 384, 384, FG_SCALE_FP32, nullptr, nullptr, nullptr,
                                      nullptr, U8(P16), F32(P16), 0), "quant_x_both_w");
    CHECK(g_last.v[0] == 0 && g_last.v[3] == 300);
    ACCEPT(fg_quantize_fprop_operands(P16, 128, 384, nullptr, 0, 384, 384, FG_SCALE_FP32, U8(P16), F32(P16), U8(P16),
                                      F32(P16), nullptr, nullptr, 0), "quant_x_both_w");
    CHECK(g_last.v[0] == 128 && g_last.v[3] == 0);
    // requantize
    REJECT(fg_requantize_1x128_to_tokens(U8(P16), F32(P16), 100, 128, FG_SCALE_FP32, U8(P16), F32(P16), 0), SHP);
    REJECT(fg_requantize_1x128_to_tokens(U8(P16), F32(PODD), 128, 128, FG_SCALE_FP32, U8(P16), F32(P16), 0), MIS);
    ACCEPT(fg_requantize_1x128_to_tokens(U8(P16), F32(P16), 256, 128, FG_SCALE_POW2, U8(P16), F32(P16), 0), "requant_rows");
    // weights
    REJECT(fg_quantize_w_128x128(P16, 128, 100, 100, FG_SCALE_FP32, U8(P16), F32(P16), 0), SHP);
    REJECT(fg_quantize_w_128x128(P16, 128, 128, 128, (fg_scale_mode)3, U8(P16), F32(P16), 0), INV);
    REJECT(fg_quantize_w_128x128(P16, 128, 128, 128, FG_SCALE_FP32, U8(PODD), F32(P16), 0), MIS);
    ACCEPT(fg_quantize_w_128x128(P16, 300, 256, 264, FG_SCALE_FP32, U8(P16), F32(P16), 0), "quant_w");
    CHECK(g_last.v[0] == 300 && g_last.v[1] == 256 && g_last.v[2] == 264);
    // Fprop
    REJECT(fg_fp8_gemm_fprop(U8(P16), F32(P16), U8(P16), F32(P16), 128, 128, 100, P16, FG_OUT_F32, FG_SCALE_FP32, 0), SHP);
    REJECT(fg_fp8_gemm_fprop(U8(P16), F32(P16), U8(P16), F32(P16), 128, 128, 128, P16, (fg_out_dtype)7, FG_SCALE_FP32, 0), INV);
    REJECT(fg_fp8_gemm_fprop(U8(P16), F32(P16), nullptr, F32(P16), 128, 128, 128, P16, FG_OUT_F32, FG_SCALE_FP32, 0), INV);
    REJECT(fg_fp8_gemm_fprop(U8(P16), F32(P16), U8(P16), F32(P16), 128, 128, 128, PODD, FG_OUT_F32, FG_SCALE_FP32, 0), MIS);
    REJECT(fg_fp8_gemm_fprop(U8(P16), F32(P16), U8(P16), F32(P16), 128, 128, (1LL << 24) + 128, P16, FG_OUT_F32,
                             FG_SCALE_FP32, 0), SHP);
    REJECT(fg_fp8_gemm_fprop(U8(P16), F32(P16), U8(P16), F32(P16), INT64_MAX, INT64_MAX, 128, P16, FG_OUT_F32,
                             FG_SCALE_FP32, 0), SHP);
    REJECT(fg_fp8_gemm_dgrad(U8(P16), F32(P16), U8(P16), F32(P16), INT64_MAX, 128, 128, P16, FG_OUT_F32, FG_SCALE_FP32,
                             0), SHP);
    REJECT(fg_fp8_gemm_wgrad(U8(P16), F32(P16), U8(P16), F32(P16), 128, INT64_MAX, 128, F32(P16), 0, FG_SCALE_FP32, 0), SHP);
    REJECT(fg_fp8_grouped_gemm(U8(P16), F32(P16), U8(P16), F32(P16), I32(P16B), 8, INT64_MAX, 128, 128, P16, FG_OUT_BF16,
                               FG_SCALE_FP32, 0), SHP);
    REJECT(fg_fp8_grouped_gemm_dgrad(U8(P16), F32(P16), U8(P16), F32(P16), I32(P16B), 8, INT64_MAX, 128, 128, P16,
                                     FG_OUT_F32, FG_SCALE_FP32, 0), SHP);
    // the grouped grid pads the worst-case row tiles (rows / 256 + G) by up to 7: bounded with the padding
    // ((2 + 7) x 2^28 > 2^31 - 1 although 2 x 2^28 is not)
    REJECT(fg_fp8_grouped_gemm(U8(P16), F32(P16), U8(P16), F32(P16), I32(P16B), 1, 256, 1LL << 35, 128, P16, FG_OUT_BF16,
                               FG_SCALE_FP32, 0), SHP);
    ACCEPT(fg_fp8_grouped_gemm(U8(P16), F32(P16), U8(P16), F32(P16), I32(P16B), 1, 256, 1LL << 34, 128, P16, FG_OUT_BF16,
                               FG_SCALE_FP32, 0), "gemm_grouped");
    REJECT(fg_fp8_grouped_gemm_dgrad(U8(P16), F32(P16), U8(P16), F32(P16), I32(P16B), 1, 256, 128, 1LL << 34, P16,
                                     FG_OUT_F32, FG_SCALE_FP32, 0), SHP);
    REJECT(fg_fp8_grouped_gemm_wgrad(U8(P16), F32(P16), U8(P16), F32(P16), I32(P16B), 65536, 128, 1LL << 20, 1LL << 20,
                                     F32(P16), 0, FG_SCALE_FP32, 0), SHP);
    NOOP(fg_fp8_gemm_fprop(nullptr, nullptr, nullptr, nullptr, 0, 128, 128, nullptr, FG_OUT_F32, FG_SCALE_FP32, 0));
    ACCEPT(fg_fp8_gemm_fprop(U8(P16), F32(P16), U8(P16), F32(P16), 300, 520, 1LL << 24, P16, FG_OUT_BF16, FG_SCALE_POW2, 0),
           "gemm_fprop");
    CHECK(g_last.v[0] == 300 && g_last.v[1] == 520 && g_last.v[2] == (1LL << 24) && g_last.flags[0] == 1 &&
          g_last.flags[1] == 1);
    ACCEPT(fg_fp8_gemm_fprop(nullptr, nullptr, nullptr, nullptr, 5, 7, 0, P16, FG_OUT_F32, FG_SCALE_FP32, 0), "gemm_fprop");
    // quantizing Fprop
    REJECT(fg_fp8_gemm_fprop_quant(U8(P16), F32(P16), U8(P16), F32(P16), 128, 200, 128, U8(P16), F32(P16), FG_SCALE_FP32,
                                   FG_SCALE_FP32, 0), SHP);
    REJECT(fg_fp8_gemm_fprop_quant(U8(P16), F32(P16), U8(P16), F32(P16), 128, 128, 128, U8(P16), nullptr, FG_SCALE_FP32,
                                   FG_SCALE_FP32, 0), INV);
    ACCEPT(fg_fp8_gemm_fprop_quant(U8(P16), F32(P16), U8(P16), F32(P16), 64, 256, 512, U8(P16), F32(P16), FG_SCALE_FP32,
                                   FG_SCALE_POW2, 0), "gemm_fprop_quant");
    CHECK(g_last.flags[0] == 0 && g_last.flags[1] == 1);
    // Dgrad
    REJECT(fg_fp8_gemm_dgrad(U8(P16), F32(P16), U8(P16), F32(P16), 128, 200, 128, P16, FG_OUT_F32, FG_SCALE_FP32, 0), SHP);
    REJECT(fg_fp8_gemm_dgrad(U8(P16), F32(P16), U8(P16), F32(P16), 128, 256, (1LL << 25) + 128, P16, FG_OUT_F32,
                             FG_SCALE_FP32, 0), SHP);
    ACCEPT(fg_fp8_gemm_dgrad(U8(P16), F32(P16), U8(P16), F32(P16), 100, 512, 1LL << 25, P16, FG_OUT_F32, FG_SCALE_FP32, 0),
           "gemm_dgrad");
    CHECK(g_last.v[0] == 100 && g_last.v[1] == 512 && g_last.v[2] == (1LL << 25));
    // Wgrad
    REJECT(fg_fp8_gemm_wgrad(U8(P16), F32(P16), U8(P16), F32(P16), 100, 128, 128, F32(P16), 0, FG_SCALE_FP32, 0), SHP);
    REJECT(fg_fp8_gemm_wgrad(U8(P16), F32(P16), U8(P16), F32(PODD), 128, 128, 128, F32(P16), 0, FG_SCALE_FP32, 0), MIS);
    REJECT(fg_fp8_gemm_wgrad(U8(P16), F32(P16), U8(P16), F32(P16), (1LL << 24) + 128, 128, 128, F32(P16), 0,
                             FG_SCALE_FP32, 0), SHP);
    ACCEPT(fg_fp8_gemm_wgrad(U8(P16), F32(P16), U8(P16), F32(P16), 4096, 200, 136, F32(P16), 5, FG_SCALE_POW2, 0),
           "gemm_wgrad");
    CHECK(g_last.v[0] == 4096 && g_last.v[1] == 200 && g_last.v[2] == 136 && g_last.flags[0] == 1 && g_last.flags[1] == 1);
    // grouped
    REJECT(fg_fp8_grouped_gemm(U8(P16), F32(P16), U8(P16), F32(P16), I32(P16B), 0, 128, 128, 128, P16, FG_OUT_BF16,
                               FG_SCALE_FP32, 0), INV);
    REJECT(fg_fp8_grouped_gemm(U8(P16), F32(P16), U8(P16), F32(P16), nullptr, 2, 128, 128, 128, P16, FG_OUT_BF16,
                               FG_SCALE_FP32, 0), INV);
    REJECT(fg_fp8_grouped_gemm(U8(P16), F32(P16), U8(P16), F32(P16), I32(P16B), 70000, 128, 128, 128, P16, FG_OUT_BF16,
                               FG_SCALE_FP32, 0), INV);
    ACCEPT(fg_fp8_grouped_gemm(U8(P16), F32(P16), U8(P16), F32(P16), I32(P16B), 8, 65536, 2048, 7168, P16, FG_OUT_BF16,
                               FG_SCALE_FP32, 0), "gemm_grouped");
    CHECK(g_last.v[0] == 65536 && g_last.v[1] == 2048 && g_last.v[2] == 7168 && g_last.v[3] == 8);
    REJECT(fg_fp8_grouped_gemm_dgrad(U8(P16), F32(P16), U8(P16), F32(P16), I32(P16B), 2, 128, 100, 128, P16, FG_OUT_F32,
                                     FG_SCALE_FP32, 0), SHP);
    ACCEPT(fg_fp8_grouped_gemm_dgrad(U8(P16), F32(P16), U8(P16), F32(P16), I32(P16B), 8, 66176, 2048, 7168, P16,
                                     FG_OUT_F32, FG_SCALE_FP32, 0), "gemm_grouped_dgrad");
    REJECT(fg_fp8_grouped_gemm_wgrad(U8(P16), F32(P16), U8(P16), F32(P16), I32(P16B), 2, 200, 128, 128, F32(P16), 0,
                                     FG_SCALE_FP32, 0), SHP);
    REJECT(fg_fp8_grouped_gemm_wgrad(U8(P16), F32(P16), U8(P16), F32(P16), I32(P16B), 2, (1LL << 24) + 128, 128, 128,
                                     F32(P16), 0, FG_SCALE_FP32, 0), SHP);
    ACCEPT(fg_fp8_grouped_gemm_wgrad(U8(P16), F32(P16), U8(P16), F32(P16), I32(P16B), 8, 66176, 2048, 7168, F32(P16), 1,
                                     FG_SCALE_POW2, 0), "gemm_grouped_wgrad");
    CHECK(g_last.flags[0] == 1 && g_last.flags[1] == 1 && g_last.v[3] == 8);
    // E5M6, limited accumulation, per-tensor
    REJECT(fg_quantize_e5m6_1x128(P16, 4, 200, 200, U8(P16), F32(P16), 0), SHP);
    ACCEPT(fg_quantize_e5m6_1x128(P16, 4, 256, 256, U8(P16), F32(P16), 0), "quant_e5m6");
    REJECT(fg_dequantize_e5m6_1x128(U8(P16), nullptr, 4, 128, P16, 128, 0), INV);
    ACCEPT(fg_dequantize_e5m6_1x128(U8(P16), F32(P16), 4, 128, P16, 136, 0), "dequant_e5m6");
    CHECK(g_last.v[2] == 136);
    REJECT(fg_fp8_gemm_fprop_limited_accum(U8(P16), F32(P16), U8(P16), F32(P16), 16, 16, 128, 24, F32(P16), 0), INV);
    ACCEPT(fg_fp8_gemm_fprop_limited_accum(U8(P16), F32(P16), U8(P16), F32(P16), 16, 16, 128, 10, F32(P16), 0),
           "fprop_limited");
    CHECK(g_last.v[3] == 10);
    REJECT(fg_amax_bf16(P16, 4, 124, 128, F32(P16B), 0), SHP);
    ACCEPT(fg_amax_bf16(P16, 4, 128, 128, F32(P16B), 0), "amax");
    REJECT(fg_quantize_per_tensor(P16, 4, 128, 128, F32(P16B), 4, FG_SCALE_FP32, FG_LAYOUT_ACT_1x128, U8(P16), F32(P16),
                                  F32((char*)P16B + 8), 0), INV);
    ACCEPT(fg_quantize_per_tensor(P16, 300, 256, 256, F32(P16B), 3, FG_SCALE_POW2, FG_LAYOUT_W_128x128, U8(P16), F32(P16),
                                  nullptr, 0), "quant_per_tensor");
    CHECK(g_last.v[3] == 3 * 2 && g_last.flags[0] == 1 && g_last.flags[1] == 3);
    ACCEPT(fg_quantize_per_tensor(P16, 300, 256, 256, F32(P16B), 0, FG_SCALE_FP32, FG_LAYOUT_ACT_1x128, U8(P16), F32(P16),
                                  nullptr, 0), "quant_per_tensor");
    CHECK(g_last.v[3] == 2 * 300);
    // a launcher error comes back as FG_ERR_HIP, with the HIP code kept for fg_last_hip_error
    CHECK(fg_last_hip_error() == 0);
    g_ret = hipErrorInvalidValue;
    g_calls = 0;
    CHECK(fg_fp8_gemm_fprop(U8(P16), F32(P16), U8(P16), F32(P16), 128, 128, 128, P16, FG_OUT_F32, FG_SCALE_FP32, 0) ==
          FG_ERR_HIP);
    CHECK(fg_last_hip_error() == (int)hipErrorInvalidValue);
    g_ret = hipSuccess;
    for (int s = 0; s <= 5; s++) CHECK(fg_status_string((fg_status)s) != nullptr);
    if (g_failures) {
        printf("%d ABI check(s) failed\n", g_failures);
        return 1;
    }
    printf("abi host driver done\n");
    return 0;
}
