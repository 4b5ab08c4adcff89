/* Drives every function of oracle/oracle.c on small, ragged shapes with buffers of exactly the documented
 * sizes, for a build with AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_oracle_sanitized.py).
 * Exit status 0 and no sanitizer report means no out-of-bounds access, leak or undefined behaviour. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

double oracle_e4m3_decode(uint8_t code);
uint8_t oracle_e4m3_encode(float v);
void oracle_e4m3_encode_many(const float* v, int64_t n, uint8_t* out);
uint16_t oracle_f32_to_bf16(float f);
float oracle_scale_from_amax(float amax, int pow2);
void oracle_quantize_act_1x128(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, int axis, int pow2,
                               uint8_t* q, float* scales);
void oracle_quantize_w_128x128(const uint16_t* w, int64_t n, int64_t k, int64_t ld, int pow2, uint8_t* q,
                               float* scales);
void oracle_requantize_1x128_to_tokens(const uint8_t* q, const float* s, int64_t rows, int64_t cols, int pow2,
                                       uint8_t* q_out, float* s_out);
double oracle_e5m6_decode(uint16_t code);
uint16_t oracle_e5m6_encode(float v);
void oracle_quantize_e5m6_1x128(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, uint8_t* packed,
                                float* scales);
void oracle_dequantize_e5m6_1x128(const uint8_t* packed, const float* scales, int64_t rows, int64_t cols,
                                  uint16_t* y);
float oracle_amax_bf16(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld);
void oracle_quantize_per_tensor(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, const float* hist,
                                int64_t n_hist, int pow2, int layout, uint8_t* q, float* scales);
void oracle_gemm_fprop(const uint8_t* xq, const float* sx, const uint8_t* wq, const float* sw, int64_t M, int64_t N,
                       int64_t K, const int64_t* pts, int64_t npts, int out_bf16, void* out, double* exact);
void oracle_gemm_dgrad(const uint8_t* dyq, const float* sdy, const uint8_t* wq, const float* sw, int64_t M,
                       int64_t N, int64_t K, const int64_t* pts, int64_t npts, int out_bf16, void* out,
                       double* exact);
void oracle_gemm_wgrad(const uint8_t* dytq, const float* sdyt, const uint8_t* xtq, const float* sxt, int64_t M,
                       int64_t N, int64_t K, int accumulate, const int64_t* pts, int64_t npts, float* out,
                       double* exact);
void oracle_gemm_grouped(const uint8_t* xq, const float* sx, const uint8_t* wq, const float* sw, const int32_t* off,
                         int32_t G, int64_t T, int64_t N, int64_t K, const int64_t* pts, int64_t npts, int out_bf16,
                         void* out, double* exact);
void oracle_gemm_fprop_limited(const uint8_t* xq, const float* sx, const uint8_t* wq, const float* sw, int64_t M,
                               int64_t N, int64_t K, int64_t chunk, int bits, const int64_t* pts, int64_t npts,
                               double* out);

static uint32_t rng_state = 12345u;
static uint32_t next_u32(void) {            /* xorshift32: input patterns only */
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 17;
    rng_state ^= rng_state << 5;
    return rng_state;
}
static uint16_t* bf16_buf(int64_t n) {       /* finite bf16 values of mixed magnitude */
    uint16_t* b = malloc((size_t)n * sizeof(uint16_t));
    for (int64_t i = 0; i < n; i++) {
        uint16_t v = (uint16_t)next_u32();
        if (((v >> 7) & 0xFF) == 0xFF) v &= 0xBFFF;   /* no Inf/NaN */
        b[i] = v;
    }
    return b;
}
static uint8_t* code_buf(int64_t n) {
    uint8_t* b = malloc((size_t)n);
    for (int64_t i = 0; i < n; i++) b[i] = (uint8_t)(next_u32() % 0x7F) | (uint8_t)((next_u32() & 1) << 7);
    return b;
}
static float* scale_buf(int64_t n) {
    float* b = malloc((size_t)n * sizeof(float));
    for (int64_t i = 0; i < n; i++) b[i] = 1e-3f * (float)(1 + next_u32() % 1000);
    return b;
}

int main(void) {
    double acc = 0.0;
    for (int c = 0; c < 256; c++) acc += oracle_e4m3_decode((uint8_t)c) == oracle_e4m3_decode((uint8_t)c);
    for (int c = 0; c < 4096; c++) acc += oracle_e5m6_decode((uint16_t)c) == oracle_e5m6_decode((uint16_t)c);
    float vals[7] = {0.0f, -0.0f, 1e-30f, 447.9f, 448.0f, 1e30f, -3.25f};
    uint8_t enc[7];
    oracle_e4m3_encode_many(vals, 7, enc);
    for (int i = 0; i < 7; i++) acc += enc[i] + oracle_e4m3_encode(vals[i]) + oracle_e5m6_encode(vals[i]) +
                                      oracle_f32_to_bf16(vals[i]) + oracle_scale_from_amax(vals[i], i & 1);

    /* activation tiles, ragged, both axes, row stride wider than the row */
    const int64_t R = 131, C = 300, LD = 304;
    uint16_t* x = bf16_buf(R * LD);
    uint8_t* q = malloc((size_t)(R * C));
    float* s = malloc((size_t)(((C + 127) / 128) * R) * sizeof(float));
    oracle_quantize_act_1x128(x, R, C, LD, 0, 0, q, s);
    free(s);
    s = malloc((size_t)(((R + 127) / 128) * C) * sizeof(float));
    oracle_quantize_act_1x128(x, R, C, LD, 1, 1, q, s);
    free(s);
    /* weight blocks, ragged */
    s = malloc((size_t)(((R + 127) / 128) * ((C + 127) / 128)) * sizeof(float));
    oracle_quantize_w_128x128(x, R, C, LD, 1, q, s);
    free(s);
    /* per-tensor, both layouts */
    float hist[3] = {2.0f, -5.0f, 1.0f + 1.0f / 1024};
    acc += oracle_amax_bf16(x, R, C, LD);
    s = malloc((size_t)(((C + 127) / 128) * R) * sizeof(float));
    oracle_quantize_per_tensor(x, R, C, LD, hist, 3, 0, 0, q, s);
    free(s);
    s = malloc((size_t)(((R + 127) / 128) * ((C + 127) / 128)) * sizeof(float));
    oracle_quantize_per_tensor(x, R, C, LD, hist, 0, 1, 1, q, s);
    free(s);
    free(q);
    free(x);

    /* E5M6 and re-quantization (whole tiles) */
    const int64_t R2 = 256, C2 = 384;
    x = bf16_buf(R2 * C2);
    uint8_t* packed = malloc((size_t)(R2 * C2 * 3 / 2));
    s = malloc((size_t)((C2 / 128) * R2) * sizeof(float));
    oracle_quantize_e5m6_1x128(x, R2, C2, C2, packed, s);
    uint16_t* y16 = malloc((size_t)(R2 * C2) * sizeof(uint16_t));
    oracle_dequantize_e5m6_1x128(packed, s, R2, C2, y16);
    uint8_t* qc = malloc((size_t)(R2 * C2));
    oracle_quantize_act_1x128(x, R2, C2, C2, 0, 0, qc, s);
    uint8_t* qt = malloc((size_t)(R2 * C2));
    float* st = malloc((size_t)((R2 / 128) * C2) * sizeof(float));
    oracle_requantize_1x128_to_tokens(qc, s, R2, C2, 0, qt, st);
    free(st); free(qt); free(qc); free(y16); free(s); free(packed); free(x);

    /* GEMMs: ragged M and N, every point and sampled points, both output types */
    const int64_t M = 37, N = 130, K = 256, KB = K / 128, NB = (N + 127) / 128;
    uint8_t* xq = code_buf(M * K);
    uint8_t* wq = code_buf(N * K);
    float* sx = scale_buf(KB * M);
    float* sw = scale_buf(NB * KB);
    float* out = malloc((size_t)(M * N) * sizeof(float));
    double* ex = malloc((size_t)(M * N) * sizeof(double));
    int64_t pts[3] = {0, M * N - 1, 77};
    oracle_gemm_fprop(xq, sx, wq, sw, M, N, K, NULL, 0, 0, out, ex);
    oracle_gemm_fprop(xq, sx, wq, sw, M, N, K, pts, 3, 1, out, NULL);
    oracle_gemm_fprop_limited(xq, sx, wq, sw, M, N, K, 32, 10, pts, 3, ex);
    free(out); free(ex);
    /* Dgrad: dY [M][N2] with N2 % 128 == 0, W [N2][K2] with ragged K2 */
    const int64_t N2 = 256, K2 = 200;
    uint8_t* dyq = code_buf(M * N2);
    float* sdy = scale_buf((N2 / 128) * M);
    uint8_t* w2 = code_buf(N2 * K2);
    float* sw2 = scale_buf((N2 / 128) * ((K2 + 127) / 128));
    out = malloc((size_t)(M * K2) * sizeof(float));
    ex = malloc((size_t)(M * K2) * sizeof(double));
    oracle_gemm_dgrad(dyq, sdy, w2, sw2, M, N2, K2, NULL, 0, 0, out, ex);
    free(out); free(ex); free(w2); free(sw2); free(sdy); free(dyq);
    /* Wgrad: tokens T (multiple of 128), dW [N3][K3] ragged, accumulate */
    const int64_t T = 256, N3 = 40, K3 = 72;
    uint8_t* dytq = code_buf(N3 * T);
    uint8_t* xtq = code_buf(K3 * T);
    float* sdyt = scale_buf((T / 128) * N3);
    float* sxt = scale_buf((T / 128) * K3);
    out = calloc((size_t)(N3 * K3), sizeof(float));
    ex = malloc((size_t)(N3 * K3) * sizeof(double));
    oracle_gemm_wgrad(dytq, sdyt, xtq, sxt, T, N3, K3, 1, NULL, 0, out, ex);
    free(out); free(ex); free(dytq); free(xtq); free(sdyt); free(sxt);
    /* grouped: 3 groups, one empty */
    const int32_t G = 3, off[4] = {0, 10, 10, (int32_t)M};
    uint8_t* wg = code_buf(G * N * K);
    float* swg = scale_buf(G * NB * KB);
    out = malloc((size_t)(M * N) * sizeof(float));
    oracle_gemm_grouped(xq, sx, wg, swg, off, G, M, N, K, NULL, 0, 0, out, NULL);
    free(out); free(wg); free(swg);
    free(xq); free(wq); free(sx); free(sw);

    printf("oracle driver done %.1f\n", acc);
    return 0;
}
