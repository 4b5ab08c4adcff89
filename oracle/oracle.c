/*
 * Fine-grained FP8 oracle — TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously-correct CPU statement of what the fine-grained FP8 quantize and GEMM path
 * computes. Only the test suite, the package's smoke check and the benchmark's CPU-baseline leg may load
 * this library. The GPU library never links, includes or calls it, and this file shares no code, table
 * or constant generator with the GPU kernels.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fopenmp -shared -fPIC (see oracle/build.py).
 * All float arithmetic below is IEEE-754 binary32/binary64 with round-to-nearest-even, no contraction.
 *
 * Sources (web pages quoting the FP8 training section of the DeepSeek-V3 report):
 *   [W1] "5 Ways You can get More Deepseek While Spending Less"
 *   [W2] untitled page, why-be.why-be.co.kr board "as_center", post 65967
 *   [W3] untitled page, cameseeing.com board "community", post 22576
 *   [W4] "Three Fast Methods To Study Deepseek"
 *   [W5] untitled page, gnrental.net board "free", post 15227
 *
 * Readings where the pages are silent (each one is listed with its reason in the design notes):
 *   R1  E4M3 is the OCP "E4M3FN" encoding: bias 7, no infinities, S.1111.111 is NaN, max 448.
 *   R2  Encoding rounds to nearest, ties to the even code; magnitudes above 448 saturate to 448;
 *       the sign is kept, also when the magnitude rounds to zero.
 *   R3  Scale s = RN_f32(amax / 448); amax == 0 gives s = 1; s below FLT_MIN becomes FLT_MIN.
 *   R4  Power-of-2 mode: t as in R3, then s = the smallest power of two >= t.
 *   R5  Codes are enc(RN_f32(x / s)).
 *   R6  Scales are fp32, stored MN-major for activations: scale[group][row].
 *   R7  GEMM promotion: per 128-element K block, P = exact block sum of decoded products,
 *       acc = fmaf(RN_f32(P), RN_f32(sa*sb), acc), blocks in ascending K order, acc starts at 0
 *       (or at the old output when accumulating).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <float.h>
#include <omp.h>

#define GROUP 128

/* ------------------------------------------------------------------------------------------------ */
/* Number formats                                                                                   */
/* ------------------------------------------------------------------------------------------------ */

/* E4M3 decode, byte "s eeee mmm" ([W4]/[W5] contrast of E4M3 with E5M2: "4-bit exponent and 3-bit
 * mantissa", adopted on all tensors; R1 fixes the bias and the special codes). */
double oracle_e4m3_decode(uint8_t code) {
    int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
    if (e == 15 && m == 7) return NAN;
    double mag = (e == 0) ? ldexp((double)m, -9)              /* subnormal: m * 2^-9        */
                          : ldexp(1.0 + m / 8.0, e - 7);      /* normal: (1 + m/8) * 2^(e-7) */
    return s ? -mag : mag;
}

/* E4M3 encode of a binary32 value (R2). Written from the rounding definition: the representable
 * values near |v| are spaced by q = 2^-9 below 2^-6 and by 2^(floor(log2|v|) - 3) above; |v|/q is
 * rounded to the nearest integer with ties to even (the even integer is the even mantissa). */
uint8_t oracle_e4m3_encode(float v) {
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    if (a >= 448.0) return sign | 0x7E;                        /* 448 and all larger: saturate */
    double q;
    if (a < ldexp(1.0, -6)) {
        q = ldexp(1.0, -9);
    } else {
        int e;
        frexp(a, &e);                                           /* a = f * 2^e, f in [0.5, 1)  */
        q = ldexp(1.0, (e - 1) - 3);
    }
    double r = nearbyint(a / q);                                /* a/q is exact: q = 2^j       */
    double val = r * q;                                         /* the rounded magnitude       */
    if (val == 0.0) return sign;
    if (val < ldexp(1.0, -6)) return sign | (uint8_t)r;         /* subnormal code = r (1..7)   */
    int e2;
    double f2 = frexp(val, &e2);                                /* val = f2 * 2^e2             */
    int exp_field = (e2 - 1) + 7;
    int mant = (int)((2.0 * f2 - 1.0) * 8.0);                   /* exact: val has 3 frac bits  */
    return sign | (uint8_t)(exp_field << 3) | (uint8_t)mant;
}

/* oracle_e4m3_encode over an array (for the exhaustive checks of the tests). */
void oracle_e4m3_encode_many(const float* v, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) out[i] = oracle_e4m3_encode(v[i]);
}

float oracle_bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* binary32 -> bfloat16, round to nearest even (finite inputs). Written as "nearest of the two
 * neighbouring bf16 values", computed in double where both neighbours and the midpoint are exact. */
uint16_t oracle_f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t lo = u & 0xFFFF0000u;                              /* truncation toward zero      */
    uint32_t hi = lo + 0x00010000u;                             /* next bf16 away from zero    */
    float flo, fhi;
    memcpy(&flo, &lo, 4);
    memcpy(&fhi, &hi, 4);
    double d = fabs((double)f), dlo = fabs((double)flo), dhi = fabs((double)fhi);
    uint32_t pick;
    if (d - dlo < dhi - d) pick = lo;
    else if (d - dlo > dhi - d) pick = hi;
    else pick = ((lo >> 16) & 1) ? hi : lo;                     /* tie: even bf16 mantissa     */
    return (uint16_t)(pick >> 16);
}

/* ------------------------------------------------------------------------------------------------ */
/* Scale from the online max-abs                                                                    */
/* ------------------------------------------------------------------------------------------------ */

/* The group's max-abs is aligned to the largest E4M3 value ([W1], the passage on scaling the maximum
 * absolute value of the input to the maximum representable FP8 value), R3; mode 1 rounds the scale up
 * to an integral power of two ([W1], opening paragraph on the inputs of the Linear after attention), R4. */
float oracle_scale_from_amax(float amax, int pow2) {
    if (amax == 0.0f) return 1.0f;
    float s = amax / 448.0f;
    if (s < FLT_MIN) s = FLT_MIN;
    if (pow2) {
        int e;
        float f = frexpf(s, &e);                               /* s = f * 2^e, f in [0.5,1) */
        if (f != 0.5f) s = ldexpf(1.0f, e);                    /* next power of two above   */
    }
    return s;
}

static float amax_of(const uint16_t* base, int64_t n_rows, int64_t n_cols, int64_t ld) {
    float m = 0.0f;
    for (int64_t r = 0; r < n_rows; r++)
        for (int64_t c = 0; c < n_cols; c++) {
            float a = fabsf(oracle_bf16_to_f32(base[r * ld + c]));
            if (a > m) m = a;
        }
    return m;
}

/* ------------------------------------------------------------------------------------------------ */
/* Quantizers                                                                                       */
/* ------------------------------------------------------------------------------------------------ */

/* 1x128 activation tiles ([W2]/[W3]/[W4], Figure 7 (a): one scale per token per 128 channels; the max
 * abs is computed online per tile, [W3] passage next to Figure 7 (a)).
 *   axis 0 (along columns): x [rows][cols] (row stride ld) -> q [rows][cols], scales [cols/128][rows]
 *   axis 1 (along rows, the token dimension, for the weight-gradient GEMM that contracts over tokens):
 *          tile = 128 consecutive rows of one column; q written transposed [cols][rows],
 *          scales [rows/128][cols]
 * The tile count along the tiled axis is ceil(len/128); a short last tile takes the max over what it has. */
void oracle_quantize_act_1x128(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, int axis,
                               int pow2, uint8_t* q, float* scales) {
    if (axis == 0) {
        int64_t ngroups = (cols + GROUP - 1) / GROUP;
        for (int64_t r = 0; r < rows; r++)
            for (int64_t g = 0; g < ngroups; g++) {
                int64_t c0 = g * GROUP, c1 = c0 + GROUP < cols ? c0 + GROUP : cols;
                float s = oracle_scale_from_amax(amax_of(x + r * ld + c0, 1, c1 - c0, ld), pow2);
                scales[g * rows + r] = s;
                for (int64_t c = c0; c < c1; c++)
                    q[r * cols + c] = oracle_e4m3_encode(oracle_bf16_to_f32(x[r * ld + c]) / s);
            }
    } else {
        int64_t ngroups = (rows + GROUP - 1) / GROUP;
        for (int64_t g = 0; g < ngroups; g++)
            for (int64_t c = 0; c < cols; c++) {
                int64_t r0 = g * GROUP, r1 = r0 + GROUP < rows ? r0 + GROUP : rows;
                float s = oracle_scale_from_amax(amax_of(x + r0 * ld + c, r1 - r0, 1, ld), pow2);
                scales[g * cols + c] = s;
                for (int64_t r = r0; r < r1; r++)
                    q[c * rows + r] = oracle_e4m3_encode(oracle_bf16_to_f32(x[r * ld + c]) / s);
            }
    }
}

/* 128x128 weight blocks ([W2]/[W3]/[W4], Figure 7 (a): per 128 input channels per 128 output channels).
 * w [n][k] (row stride ld) -> q [n][k], scales [ceil(n/128)][ceil(k/128)] row-major. */
void oracle_quantize_w_128x128(const uint16_t* w, int64_t n, int64_t k, int64_t ld, int pow2,
                               uint8_t* q, float* scales) {
    int64_t nb = (n + GROUP - 1) / GROUP, kb = (k + GROUP - 1) / GROUP;
    for (int64_t bi = 0; bi < nb; bi++)
        for (int64_t bj = 0; bj < kb; bj++) {
            int64_t r0 = bi * GROUP, r1 = r0 + GROUP < n ? r0 + GROUP : n;
            int64_t c0 = bj * GROUP, c1 = c0 + GROUP < k ? c0 + GROUP : k;
            float s = oracle_scale_from_amax(amax_of(w + r0 * ld + c0, r1 - r0, c1 - c0, ld), pow2);
            scales[bi * kb + bj] = s;
            for (int64_t r = r0; r < r1; r++)
                for (int64_t c = c0; c < c1; c++)
                    q[r * k + c] = oracle_e4m3_encode(oracle_bf16_to_f32(w[r * ld + c]) / s);
        }
}

/* Token tiles from cached FP8 activations: codes q [rows][cols] with their 1x128 row-tile scales
 * s [cols/128][rows] stand for the bf16 activations bf16(RN_f32(dec(q) * s)) (activations kept in FP8 for
 * the backward pass, [W4]/[W5] Figure 6 passage; dequantized in fp32 and stored back as the activation's
 * bf16, the reading taken here), which are then quantized along the tokens as above (axis 1). */
void oracle_requantize_1x128_to_tokens(const uint8_t* q, const float* s, int64_t rows, int64_t cols, int pow2,
                                       uint8_t* q_out, float* s_out) {
    uint16_t* x = (uint16_t*)malloc((size_t)(rows * cols) * sizeof(uint16_t));
    if (!x) return;
    for (int64_t r = 0; r < rows; r++)
        for (int64_t c = 0; c < cols; c++) {
            float v = (float)oracle_e4m3_decode(q[r * cols + c]) * s[(c / GROUP) * rows + r];
            x[r * cols + c] = oracle_f32_to_bf16(v);
        }
    oracle_quantize_act_1x128(x, rows, cols, cols, 1, pow2, q_out, s_out);
    free(x);
}

/* ------------------------------------------------------------------------------------------------ */
/* E5M6 storage of cached activations                                                               */
/* ------------------------------------------------------------------------------------------------ */

/* [W1] names a customized E5M6 format for some cached activations, with power-of-2 scaling factors.
 * Reading R16: 12-bit code s eeeee mmmmmm, exponent bias 15, exponent 31 holds infinities (fraction 0) and
 * NaN as in the other E5 formats, subnormals m * 2^-20; largest finite (2 - 2^-6) * 2^15 = 65024. */
double oracle_e5m6_decode(uint16_t code) {
    int s = (code >> 11) & 1, e = (code >> 6) & 31, m = code & 63;
    double mag;
    if (e == 31) mag = m ? NAN : INFINITY;
    else if (e == 0) mag = ldexp((double)m, -20);
    else mag = ldexp(1.0 + m / 64.0, e - 15);
    return s ? -mag : mag;
}

/* Nearest E5M6 value, ties to the even fraction, magnitudes above 65024 saturate, sign kept (R16).
 * Written like the E4M3 encoder: the spacing near |v| is 2^-20 below 2^-14 and 2^(floor(log2|v|) - 6)
 * above; |v| / spacing is rounded to the nearest integer with ties to even. */
uint16_t oracle_e5m6_encode(float v) {
    uint16_t sign = signbit(v) ? 0x800 : 0;
    double a = fabs((double)v);
    if (a >= 65024.0) return sign | 0x7BF;
    double q;
    if (a < ldexp(1.0, -14)) {
        q = ldexp(1.0, -20);
    } else {
        int e;
        frexp(a, &e);
        q = ldexp(1.0, (e - 1) - 6);
    }
    double r = nearbyint(a / q), val = r * q;
    if (val == 0.0) return sign;
    if (val < ldexp(1.0, -14)) return sign | (uint16_t)r;       /* subnormal: fraction = r (1..63)    */
    if (val >= 65024.0) return sign | 0x7BF;
    int e2;
    double f2 = frexp(val, &e2);
    int exp_field = (e2 - 1) + 15;
    int mant = (int)((2.0 * f2 - 1.0) * 64.0);
    return sign | (uint16_t)(exp_field << 6) | (uint16_t)mant;
}

/* 1x128 tiles along the columns with power-of-2 scales ([W1], opening paragraph): s = the smallest power
 * of two >= RN_f32(amax / 65024) (R3/R4 with the E5M6 maximum); codes enc(x / s), packed two per three
 * bytes, little-endian (byte 0: c0 bits 0-7; byte 1: c0 bits 8-11, c1 bits 0-3; byte 2: c1 bits 4-11).
 * x [rows][cols] -> packed [rows][cols * 3 / 2], scales [cols/128][rows]; cols a multiple of 128. */
void oracle_quantize_e5m6_1x128(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, uint8_t* packed,
                                float* scales) {
    int64_t ngroups = cols / GROUP, ldp = cols * 3 / 2;
    for (int64_t r = 0; r < rows; r++)
        for (int64_t g = 0; g < ngroups; g++) {
            float amax = amax_of(x + r * ld + g * GROUP, 1, GROUP, ld);
            float s = 1.0f;
            if (amax != 0.0f) {
                s = amax / 65024.0f;
                if (s < FLT_MIN) s = FLT_MIN;
                int e;
                float f = frexpf(s, &e);
                if (f != 0.5f) s = ldexpf(1.0f, e);
            }
            scales[g * rows + r] = s;
            for (int64_t c = g * GROUP; c < (g + 1) * GROUP; c += 2) {
                uint16_t c0 = oracle_e5m6_encode(oracle_bf16_to_f32(x[r * ld + c]) / s);
                uint16_t c1 = oracle_e5m6_encode(oracle_bf16_to_f32(x[r * ld + c + 1]) / s);
                uint8_t* p = packed + r * ldp + (c / 2) * 3;
                p[0] = (uint8_t)(c0 & 0xFF);
                p[1] = (uint8_t)((c0 >> 8) | ((c1 & 0xF) << 4));
                p[2] = (uint8_t)(c1 >> 4);
            }
        }
}

/* The bf16 values E5M6 storage stands for: bf16(RN_f32(dec(code) * s)). */
void oracle_dequantize_e5m6_1x128(const uint8_t* packed, const float* scales, int64_t rows, int64_t cols,
                                  uint16_t* y) {
    int64_t ldp = cols * 3 / 2;
    for (int64_t r = 0; r < rows; r++)
        for (int64_t c = 0; c < cols; c += 2) {
            const uint8_t* p = packed + r * ldp + (c / 2) * 3;
            uint16_t c0 = (uint16_t)(p[0] | ((p[1] & 0xF) << 8));
            uint16_t c1 = (uint16_t)((p[1] >> 4) | (p[2] << 4));
            float s = scales[(c / GROUP) * rows + r];
            y[r * cols + c] = oracle_f32_to_bf16((float)oracle_e5m6_decode(c0) * s);
            y[r * cols + c + 1] = oracle_f32_to_bf16((float)oracle_e5m6_decode(c1) * s);
        }
}

/* ------------------------------------------------------------------------------------------------ */
/* Per-tensor scaling: the prior practice the tiles are contrasted with                             */
/* ------------------------------------------------------------------------------------------------ */

/* Max-abs of a whole bf16 tensor ([W1], the passage on aligning the input tensor's max-abs to the
 * largest FP8 value, the common practice it calls sensitive to activation outliers). */
float oracle_amax_bf16(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld) {
    return amax_of(x, rows, cols, ld);
}

/* The max-abs a per-tensor scale is taken from: the largest |h[i]| of a history ([W4], the passage on
 * delayed quantization, which infers the current max-abs from those of prior iterations; one entry
 * holding the tensor's own max-abs is current scaling). Readings: a value between two bf16 numbers is
 * taken as the next bf16 number up, and values beyond the largest finite bf16 as that number. */
static float hist_amax(const float* h, int64_t n) {
    double m = 0.0;
    for (int64_t i = 0; i < n; i++)
        if (fabs((double)h[i]) > m) m = fabs((double)h[i]);
    const double bf16_max = ldexp(255.0 / 128.0, 127);           /* (2 - 2^-7) * 2^127          */
    if (m >= bf16_max) return (float)bf16_max;
    if (m == 0.0) return 0.0f;
    int e;
    frexp(m, &e);                                                  /* m in [2^(e-1), 2^e)          */
    double ulp = ldexp(1.0, (e - 1) - 7);                          /* bf16 spacing: 7 fraction bits */
    if (e - 1 < -126) ulp = ldexp(1.0, -133);                      /* subnormal bf16 spacing        */
    return (float)(ceil(m / ulp) * ulp);
}

/* Per-tensor quantization: s from the history's max-abs by the same rule as the tiles (R3, R4), codes
 * enc(RN_f32(x / s)) with saturation above 448 (R2) for values beyond that max-abs. Every scale entry of
 * the layout (0: the 1x128 activation layout [cols/128][rows]; 1: the 128x128 weight layout
 * [ceil(rows/128)][cols/128]) holds s. */
void oracle_quantize_per_tensor(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, const float* hist,
                                int64_t n_hist, int pow2, int layout, uint8_t* q, float* scales) {
    float s = oracle_scale_from_amax(hist_amax(hist, n_hist), pow2);
    int64_t n_scales = layout == 0 ? ((cols + GROUP - 1) / GROUP) * rows
                                   : ((rows + GROUP - 1) / GROUP) * ((cols + GROUP - 1) / GROUP);
    for (int64_t i = 0; i < n_scales; i++) scales[i] = s;
    for (int64_t r = 0; r < rows; r++)
        for (int64_t c = 0; c < cols; c++)
            q[r * cols + c] = oracle_e4m3_encode(oracle_bf16_to_f32(x[r * ld + c]) / s);
}

/* ------------------------------------------------------------------------------------------------ */
/* Block-scaled GEMM                                                                                */
/* ------------------------------------------------------------------------------------------------ */

/* One output element of a GEMM whose operands are E4M3 codes with one fp32 scale per 128-element
 * group along the contraction dimension ([W1], per-group scaling along the inner dimension).
 *   a(k) = code at a_base + k*a_step,  b(k) = code at b_base + k*b_step,  k in [0, kdim)
 *   sa(g) = sa_base[g*sa_step],        sb(g) = sb_base[g*sb_step],         g = k / 128
 * Returns the promoted result R7 (what the method computes: per-128 FP32 promotion, [W1] passage on the
 * 128-element accumulation interval) and, through *exact, the real value sum_g sa*sb*P_g in fp64.
 * Every E4M3 value is an integer multiple of 2^-9 below 2^9, so each decoded product is a multiple of
 * 2^-18 below 2^18 and a block sum of 128 of them is exact in binary64: P_g below is exact. */
static float dot_promoted(const uint8_t* a_base, int64_t a_step, const uint8_t* b_base, int64_t b_step,
                          const float* sa_base, int64_t sa_step, const float* sb_base, int64_t sb_step,
                          int64_t kdim, float acc0, double* exact) {
    float acc = acc0;
    double ex = (double)acc0;
    for (int64_t g = 0; g * GROUP < kdim; g++) {
        double p = 0.0;
        for (int64_t k = g * GROUP; k < (g + 1) * GROUP && k < kdim; k++)
            p += oracle_e4m3_decode(a_base[k * a_step]) * oracle_e4m3_decode(b_base[k * b_step]);
        float sa = sa_base[g * sa_step], sb = sb_base[g * sb_step];
        float s = sa * sb;
        acc = fmaf((float)p, s, acc);
        ex += (double)sa * (double)sb * p;
    }
    if (exact) *exact = ex;
    return acc;
}

static void store_out(void* out, int out_bf16, int64_t idx, float v) {
    if (out_bf16) ((uint16_t*)out)[idx] = oracle_f32_to_bf16(v);
    else ((float*)out)[idx] = v;
}

/* Points: if pts == NULL every output (row-major) is computed; otherwise pts[i] is a flat row-major
 * output index and results go to position i of the outputs. `out` and `exact` may be NULL. */

/* Fprop (Figure 6, forward pass): Y[m][n] = sum_k X[m][k] W[n][k].
 * xq [M][K] codes, sx [K/128][M]; wq [N][K] codes, sw [ceil(N/128)][K/128]. */
void oracle_gemm_fprop(const uint8_t* xq, const float* sx, const uint8_t* wq, const float* sw,
                       int64_t M, int64_t N, int64_t K, const int64_t* pts, int64_t npts,
                       int out_bf16, void* out, double* exact) {
    int64_t kb = K / GROUP, total = pts ? npts : M * N;
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < total; i++) {
        int64_t flat = pts ? pts[i] : i, m = flat / N, n = flat % N;
        double ex;
        float v = dot_promoted(xq + m * K, 1, wq + n * K, 1, sx + m, M, sw + (n / GROUP) * kb, 1, K, 0.0f, &ex);
        if (out) store_out(out, out_bf16, i, v);
        if (exact) exact[i] = ex;
    }
}

/* Dgrad (Figure 6, activation backward pass): dX[m][k] = sum_n dY[m][n] W[n][k].
 * dyq [M][N] codes, sdy [N/128][M]; wq [N][K] codes, sw [N/128][ceil(K/128)] (the same 128x128
 * blocks as Fprop, read along the other axis). */
void oracle_gemm_dgrad(const uint8_t* dyq, const float* sdy, const uint8_t* wq, const float* sw,
                       int64_t M, int64_t N, int64_t K, const int64_t* pts, int64_t npts,
                       int out_bf16, void* out, double* exact) {
    int64_t kbk = (K + GROUP - 1) / GROUP, total = pts ? npts : M * K;
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < total; i++) {
        int64_t flat = pts ? pts[i] : i, m = flat / K, k = flat % K;
        double ex;
        float v = dot_promoted(dyq + m * N, 1, wq + k, K, sdy + m, M, sw + k / GROUP, kbk, N, 0.0f, &ex);
        if (out) store_out(out, out_bf16, i, v);
        if (exact) exact[i] = ex;
    }
}

/* Wgrad (Figure 6, weight backward pass): dW[n][k] (+)= sum_m dY[m][n] X[m][k], contracting over tokens.
 * dytq [N][M] codes (dY quantized in 1x128 tiles along tokens, transposed), sdyt [M/128][N];
 * xtq [K][M] codes, sxt [M/128][K]. Output fp32 (gradients stay fp32, [W5] passage on master weights and
 * gradients). With accumulate != 0 the sum starts from the existing dW value (`out` holds it on entry). */
void oracle_gemm_wgrad(const uint8_t* dytq, const float* sdyt, const uint8_t* xtq, const float* sxt,
                       int64_t M, int64_t N, int64_t K, int accumulate, const int64_t* pts, int64_t npts,
                       float* out, double* exact) {
    int64_t total = pts ? npts : N * K;
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < total; i++) {
        int64_t flat = pts ? pts[i] : i, n = flat / K, k = flat % K;
        float acc0 = accumulate ? out[i] : 0.0f;
        double ex;
        float v = dot_promoted(dytq + n * M, 1, xtq + k * M, 1, sdyt + n, N, sxt + k, K, M, acc0, &ex);
        out[i] = v;
        if (exact) exact[i] = ex;
    }
}

/* Grouped Fprop for a set of experts with contiguous row segments [off[g], off[g+1]) of X.
 * xq [T][K] codes, sx [K/128][T]; wq [G][N][K], sw [G][ceil(N/128)][K/128]; Y [T][N]. */
void oracle_gemm_grouped(const uint8_t* xq, const float* sx, const uint8_t* wq, const float* sw,
                         const int32_t* off, int32_t G, int64_t T, int64_t N, int64_t K,
                         const int64_t* pts, int64_t npts, int out_bf16, void* out, double* exact) {
    int64_t kb = K / GROUP, nb = (N + GROUP - 1) / GROUP, total = pts ? npts : T * N;
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < total; i++) {
        int64_t flat = pts ? pts[i] : i, m = flat / N, n = flat % N;
        int32_t g = 0;
        while (g < G && !(off[g] <= m && m < off[g + 1])) g++;
        if (g == G) {                                           /* row outside every segment    */
            if (out) store_out(out, out_bf16, i, 0.0f);
            if (exact) exact[i] = 0.0;
            continue;
        }
        double ex;
        float v = dot_promoted(xq + m * K, 1, wq + ((int64_t)g * N + n) * K, 1, sx + m, T,
                               sw + ((int64_t)g * nb + n / GROUP) * kb, 1, K, 0.0f, &ex);
        if (out) store_out(out, out_bf16, i, v);
        if (exact) exact[i] = ex;
    }
}

/* ------------------------------------------------------------------------------------------------ */
/* Limited-precision accumulation (the contrast the pages draw, [W1] first paragraph: about 2% max     */
/* relative error at K = 4096 from the Tensor Cores' limited accumulation precision).                */
/* ------------------------------------------------------------------------------------------------ */

/* Keep `bits` explicit mantissa bits of x, truncating toward zero. */
static double truncate_mantissa(double x, int bits) {
    if (x == 0.0) return 0.0;
    int e;
    double f = frexp(x, &e);                                    /* |f| in [0.5, 1)              */
    double scaled = ldexp(f, bits + 1);                         /* bits+1 significant bits      */
    return ldexp(trunc(scaled), e - (bits + 1));
}

/* Fprop-shaped result without promotion: the dequantized products (code value times its scale) are
 * summed exactly in chunks of `chunk` elements, and each chunk is added to a single accumulator that
 * keeps only `bits` mantissa bits after every addition. No per-128 FP32 promotion. */
void oracle_gemm_fprop_limited(const uint8_t* xq, const float* sx, const uint8_t* wq, const float* sw,
                               int64_t M, int64_t N, int64_t K, int64_t chunk, int bits,
                               const int64_t* pts, int64_t npts, double* out) {
    int64_t kb = K / GROUP, total = pts ? npts : M * N;
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < total; i++) {
        int64_t flat = pts ? pts[i] : i, m = flat / N, n = flat % N;
        double acc = 0.0;
        for (int64_t c0 = 0; c0 < K; c0 += chunk) {
            double part = 0.0;
            for (int64_t k = c0; k < c0 + chunk && k < K; k++) {
                double a = oracle_e4m3_decode(xq[m * K + k]) * (double)sx[(k / GROUP) * M + m];
                double b = oracle_e4m3_decode(wq[n * K + k]) * (double)sw[(n / GROUP) * kb + k / GROUP];
                part += a * b;
            }
            acc = truncate_mantissa(acc + part, bits);
        }
        out[i] = acc;
    }
}

/* Thread count OpenMP will use (reported next to CPU timings). */
int oracle_num_threads(void) {
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
    return n;
}
