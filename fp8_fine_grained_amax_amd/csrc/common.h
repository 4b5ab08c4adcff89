// Device helpers shared by the fp8fg HIP kernels (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define FG_GROUP 128

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

#define FG_GLOBAL(p) ((const __attribute__((address_space(1))) void*)(p))
#define FG_LDS(p) ((__attribute__((address_space(3))) void*)(p))

__device__ __forceinline__ float fg_bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float fg_bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Larger of two packed |bf16| magnitudes (sign bits already cleared): the non-negative bf16 bit
// patterns order like the values, so the max-abs is an unsigned 16-bit max on the bits.
__device__ __forceinline__ uint32_t fg_pk_max_u16(uint32_t a, uint32_t b) {
    u16x2 x = __builtin_bit_cast(u16x2, a), y = __builtin_bit_cast(u16x2, b);
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(x, y));
}

// Scale from the group's max-abs (given as the bf16 bit pattern of |x|max):
//   s = amax / 448 (IEEE division); amax == 0 -> 1; s < FLT_MIN -> FLT_MIN; pow2 -> next power of two up.
__device__ __forceinline__ float fg_scale_from_amax_bits(uint32_t amax_bits, int pow2) {
    float amax = __uint_as_float(amax_bits << 16);
    float s = amax / 448.0f;
    s = s < 1.17549435e-38f ? 1.17549435e-38f : s;
    if (pow2) {
        uint32_t u = __float_as_uint(s);
        if (u & 0x007FFFFFu) u = (u & 0x7F800000u) + 0x00800000u;
        s = __uint_as_float(u);
    }
    return amax_bits == 0 ? 1.0f : s;
}

// Per-group division setup. Quotients x / s are formed as q0 = RN(x r) with r = RN(1/s), the exact
// remainder x - q0 s (one FMA) and one correction q0 + rem r (Markstein's correction step). The remainder
// is exact only while it stays a binary32 normal number, so tiny scales (s < 2^-100, i.e. max-abs below
// 448 * 2^-100) are moved up by 2^64 together with x, which changes no quotient. Checked exhaustively for
// every bf16 max-abs and every bf16 |x| <= max-abs in both scale modes: the quotient is the correctly
// rounded x / s whenever |x / s| >= 2^-12, and below that both encode to the same signed E4M3 zero.
struct fg_divisor {
    float s, r, pre;
};
__device__ __forceinline__ fg_divisor fg_make_divisor(float s) {
    fg_divisor d;
    d.pre = s < 0x1p-100f ? 0x1p64f : 1.0f;
    d.s = s * d.pre;
    d.r = 1.0f / d.s;
    return d;
}
// The quotient always has the sign of x (s > 0); copying that sign back keeps x = -0 at -0 (code 0x80),
// which the FMA sum of two opposite zeros would otherwise turn into +0.
__device__ __forceinline__ float fg_div(float x, const fg_divisor& d) {
    float xs = x * d.pre;
    float q0 = xs * d.r;
    float rem = __builtin_fmaf(-q0, d.s, xs);
    return __builtin_copysignf(__builtin_fmaf(rem, d.r, q0), xs);
}

// Two E4M3 codes (round to nearest even, OCP encoding on gfx950) into the low or high 16 bits of `old`.
template <bool HI>
__device__ __forceinline__ uint32_t fg_cvt2(float a, float b, uint32_t old) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
}

// Max across the 16 lanes of a DPP row (row_ror 8, row_ror 4, quad_perm [2,3,0,1], quad_perm [1,0,3,2]).
__device__ __forceinline__ uint32_t fg_row16_max_pk(uint32_t v) {
    v = fg_pk_max_u16(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false));
    v = fg_pk_max_u16(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false));
    v = fg_pk_max_u16(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
    v = fg_pk_max_u16(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
    return v;
}

__device__ __forceinline__ uint32_t fg_max_halves(uint32_t v) {
    uint32_t lo = v & 0xFFFFu, hi = v >> 16;
    return lo > hi ? lo : hi;
}
