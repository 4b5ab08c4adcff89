// E5M6 storage for cached activations.
//
// "5 Ways You can get More Deepseek While Spending Less" keeps some cached activations (those entering
// the Linear after the attention operator) in a customized E5M6 format, with scaling factors that are
// integral powers of 2, and stores forward activations as 1x128 tiles. The format is not spelled out;
// it is read here as the E5 family's layout with a 6-bit fraction: sign, 5 exponent bits with bias 15,
// 6 fraction bits, exponent 31 for infinities and NaN as in E5M2 and binary16, largest finite value
// (2 - 2^-6) * 2^15 = 65024, subnormals down to 2^-20. Encoding rounds to nearest even and saturates.
//
// A 1x128 tile's scale is the smallest power of two >= RN_f32(max-abs / 65024) (max-abs 0 gives 1,
// scales below FLT_MIN become FLT_MIN), so dividing by it is exact and no tile value exceeds 65024.
// Two 12-bit codes pack into 3 bytes, little-endian: a 128-element tile row is 192 bytes, 12 bytes per
// lane of the 16 lanes that read its 256 bf16 bytes.
#include "common.h"

namespace {

constexpr float kE5M6Max = 65024.0f;

__device__ __forceinline__ float e5m6_scale(uint32_t amax_bits) {
    const float amax = __uint_as_float(amax_bits << 16);
    float s = amax / kE5M6Max;                          // IEEE division (correctly rounded)
    s = s < 1.17549435e-38f ? 1.17549435e-38f : s;
    uint32_t u = __float_as_uint(s);
    if (u & 0x007FFFFFu) u = (u & 0x7F800000u) + 0x00800000u;
    return amax_bits == 0 ? 1.0f : __uint_as_float(u);
}

// fp32 -> 12-bit E5M6 code, round to nearest even, saturating at 65024, sign kept.
__device__ __forceinline__ uint32_t e5m6_encode(float q) {
    const uint32_t u = __float_as_uint(q);
    const uint32_t sign = (u >> 20) & 0x800u;
    const uint32_t a = u & 0x7FFFFFFFu;
    uint32_t code;
    if (a >= 0x38800000u) {                             // |q| >= 2^-14: normal
        uint32_t r = (a + 0xFFFFu + ((a >> 17) & 1u)) >> 17;   // 6 fraction bits, ties to even
        r -= 112u << 6;                                 // exponent bias 127 -> 15
        code = r > 0x7BFu ? 0x7BFu : r;                 // saturate at (30, 63) = 65024
    } else {                                            // subnormal: multiples of 2^-20, 64 = 2^-14
        code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 0x1p20f);
    }
    return sign | code;
}

__device__ __forceinline__ float e5m6_decode(uint32_t c) {
    const uint32_t sign = (c & 0x800u) << 20;
    const uint32_t e = (c >> 6) & 31u, m = c & 63u;
    uint32_t mag;
    if (e == 0)
        mag = __float_as_uint((float)m * 0x1p-20f);
    else if (e == 31)
        mag = m == 0 ? 0x7F800000u : 0x7FC00000u;
    else
        mag = ((e + 112u) << 23) | (m << 17);
    return __uint_as_float(mag | sign);
}

__device__ __forceinline__ uint3 pack8(const uint32_t (&c)[8]) {
    return make_uint3(c[0] | (c[1] << 12) | (c[2] << 24),
                      (c[2] >> 8) | (c[3] << 4) | (c[4] << 16) | (c[5] << 28),
                      (c[5] >> 4) | (c[6] << 8) | (c[7] << 20));
}

__device__ __forceinline__ void unpack8(uint3 p, uint32_t (&c)[8]) {
    c[0] = p.x & 0xFFFu;
    c[1] = (p.x >> 12) & 0xFFFu;
    c[2] = (p.x >> 24) | ((p.y & 0xFu) << 8);
    c[3] = (p.y >> 4) & 0xFFFu;
    c[4] = (p.y >> 16) & 0xFFFu;
    c[5] = (p.y >> 28) | ((p.z & 0xFFu) << 4);
    c[6] = (p.z >> 8) & 0xFFFu;
    c[7] = p.z >> 20;
}

// One 256-thread workgroup covers 16 rows x UNROLL of one 128-column group (16 lanes per tile row, as
// the FP8 1x128 quantizer); tile max-abs by DPP, one scale per tile row.
template <int UNROLL>
__global__ __launch_bounds__(256) void fg_quant_e5m6_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t ld,
                                                            int64_t groups, uint8_t* __restrict__ packed,
                                                            int64_t ldp, float* __restrict__ scales) {
    const int lane16 = threadIdx.x & 15;
    const int slot = threadIdx.x >> 4;
    const uint32_t bid = blockIdx.x, ng = (uint32_t)groups;
    const int64_t g = bid % ng;
    const int64_t r_base = (int64_t)(bid / ng) * (16 * UNROLL) + slot;
    uint4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; u++) {
        const int64_t r = r_base + 16 * u;
        v[u] = r < rows ? *reinterpret_cast<const uint4*>(x + r * ld + g * FG_GROUP + lane16 * 8) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < UNROLL; u++) {
        const int64_t r = r_base + 16 * u;
        uint32_t m = fg_pk_max_u16(fg_pk_max_u16(v[u].x & 0x7FFF7FFFu, v[u].y & 0x7FFF7FFFu),
                                   fg_pk_max_u16(v[u].z & 0x7FFF7FFFu, v[u].w & 0x7FFF7FFFu));
        m = fg_max_halves(fg_row16_max_pk(m));
        const float s = e5m6_scale(m);
        const float rcp = __uint_as_float((254u - (__float_as_uint(s) >> 23)) << 23);   // 1/s, exact
        uint32_t c[8];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint32_t w = (&v[u].x)[i];
            c[2 * i] = e5m6_encode(fg_bf16_lo(w) * rcp);
            c[2 * i + 1] = e5m6_encode(fg_bf16_hi(w) * rcp);
        }
        if (r < rows) {
            *reinterpret_cast<uint3*>(packed + r * ldp + g * 192 + lane16 * 12) = pack8(c);
            if (lane16 == 0) scales[g * rows + r] = s;
        }
    }
}

__global__ __launch_bounds__(256) void fg_dequant_e5m6_kernel(const uint8_t* __restrict__ packed, int64_t ldp,
                                                              const float* __restrict__ scales, int64_t rows,
                                                              int64_t groups, uint16_t* __restrict__ y, int64_t ldy) {
    const int lane16 = threadIdx.x & 15;
    const int slot = threadIdx.x >> 4;
    const uint32_t bid = blockIdx.x, ng = (uint32_t)groups;
    const int64_t g = bid % ng;
    const int64_t r_base = (int64_t)(bid / ng) * 32 + slot;
    uint3 p[2];
    float s[2];
#pragma unroll
    for (int u = 0; u < 2; u++) {
        const int64_t r = r_base + 16 * u;
        p[u] = r < rows ? *reinterpret_cast<const uint3*>(packed + r * ldp + g * 192 + lane16 * 12) : make_uint3(0, 0, 0);
        s[u] = r < rows ? scales[g * rows + r] : 1.0f;
    }
#pragma unroll
    for (int u = 0; u < 2; u++) {
        const int64_t r = r_base + 16 * u;
        uint32_t c[8];
        unpack8(p[u], c);
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint32_t lo = __builtin_bit_cast(unsigned short, (__bf16)(e5m6_decode(c[2 * i]) * s[u]));
            const uint32_t hi = __builtin_bit_cast(unsigned short, (__bf16)(e5m6_decode(c[2 * i + 1]) * s[u]));
            w[i] = lo | (hi << 16);
        }
        if (r < rows) *reinterpret_cast<uint4*>(y + r * ldy + g * FG_GROUP + lane16 * 8) = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

}  // namespace

hipError_t fg_launch_quant_e5m6(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, uint8_t* packed,
                                float* scales, hipStream_t stream) {
    const int64_t groups = cols / FG_GROUP;
    const int64_t row_blocks = (rows + 31) / 32;
    hipLaunchKernelGGL(fg_quant_e5m6_kernel<2>, dim3((unsigned)(groups * row_blocks)), dim3(256), 0, stream, x, rows,
                       ld, groups, packed, cols * 3 / 2, scales);
    return hipGetLastError();
}

hipError_t fg_launch_dequant_e5m6(const uint8_t* packed, const float* scales, int64_t rows, int64_t cols, uint16_t* y,
                                  int64_t ldy, hipStream_t stream) {
    const int64_t groups = cols / FG_GROUP;
    const int64_t row_blocks = (rows + 31) / 32;
    hipLaunchKernelGGL(fg_dequant_e5m6_kernel, dim3((unsigned)(groups * row_blocks)), dim3(256), 0, stream, packed,
                       cols * 3 / 2, scales, rows, groups, y, ldy);
    return hipGetLastError();
}
