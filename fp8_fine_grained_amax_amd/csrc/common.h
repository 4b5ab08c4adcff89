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
//   s = amax / 448 (correctly rounded); amax == 0 -> 1; s < FLT_MIN -> FLT_MIN; pow2 -> next power of two up.
// The quotient is formed without a division: q0 = RN(amax * RN(1/448)), the exact remainder
// amax - 448 q0 and one correction (Markstein). Checked against IEEE division for every bf16 max-abs.
__device__ __forceinline__ float fg_scale_from_amax_bits(uint32_t amax_bits, int pow2) {
    const float amax = __uint_as_float(amax_bits << 16);
    const float c = 0x1.24924ap-9f;                     // RN(1/448)
    const float q0 = amax * c;
    const float rem = __builtin_fmaf(-q0, 448.0f, amax);
    float s = __builtin_fmaf(rem, c, q0);
    s = s < 1.17549435e-38f ? 1.17549435e-38f : s;
    if (pow2) {
        uint32_t u = __float_as_uint(s);
        if (u & 0x007FFFFFu) u = (u & 0x7F800000u) + 0x00800000u;
        s = __uint_as_float(u);
    }
    return amax_bits == 0 ? 1.0f : s;
}

// Per-group quotient setup. Every element's x / s is handed to the E4M3 conversion as one of:
//   FG_Q_POW2: x * r with r = 2^-k (s = 2^k, from the exponent field): the exact quotient;
//   FG_Q_FAST: fma(-t, r, q0) with q0 = RN(x r), t = fma(q0, s, -x) (the exact remainder, negated) and
//              r = RN(1/s): the correction step of Markstein; the negations are free FMA operand modifiers,
//              and carrying the remainder negated keeps x = -0 at -0 (code 0x80);
//   FG_Q_TINY: the same after moving s and x up by 2^64 (s < 2^-100, where the remainder of the unscaled
//              form is no longer exact).
// Checked exhaustively for every bf16 max-abs and every bf16 |x| <= max-abs of either sign, in both scale
// modes: the quotient is the correctly rounded x / s whenever |x / s| >= 2^-12, and below that both encode
// to the same signed E4M3 zero. A wave picks FAST or TINY for all its groups at once (TINY only arises
// for groups whose max-abs is below 448 * 2^-100).
enum { FG_Q_POW2 = 0, FG_Q_FAST = 1, FG_Q_TINY = 2 };
struct fg_divisor {
    float s, r;
};
__device__ __forceinline__ fg_divisor fg_make_divisor(float s, int pow2) {
    fg_divisor d;
    d.s = s;
    d.r = pow2 ? __uint_as_float((254u - (__float_as_uint(s) >> 23)) << 23) : 1.0f / s;
    return d;
}
__device__ __forceinline__ bool fg_divisor_tiny(const fg_divisor& d) { return d.s < 0x1p-100f; }
// The divisor of the TINY form: s and r moved by 2^64 and 2^-64 (both exact).
__device__ __forceinline__ fg_divisor fg_divisor_shifted(const fg_divisor& d) {
    return fg_divisor{d.s * 0x1p64f, d.r * 0x1p-64f};
}

template <int MODE>
__device__ __forceinline__ float fg_quot_arg(float x, const fg_divisor& d) {
    if constexpr (MODE == FG_Q_POW2) return x * d.r;
    const float xs = MODE == FG_Q_TINY ? x * 0x1p64f : x;
    const float q0 = xs * d.r;
    const float t = __builtin_fmaf(q0, d.s, -xs);
    return __builtin_fmaf(-t, d.r, q0);
}

// Two E4M3 codes of x0 / s and x1 / s (round to nearest even, OCP encoding on gfx950) into the low or
// high 16 bits of `old`.
template <int MODE, bool HI>
__device__ __forceinline__ uint32_t fg_cvt2q(float x0, float x1, const fg_divisor& d, uint32_t old) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fg_quot_arg<MODE>(x0, d), fg_quot_arg<MODE>(x1, d), (int)old, HI);
}

// Eight bf16 values (one 16 B load) -> eight E4M3 codes (8 B).
template <int MODE>
__device__ __forceinline__ uint2 fg_quant8(uint4 v, const fg_divisor& d) {
    uint32_t lo = fg_cvt2q<MODE, false>(fg_bf16_lo(v.x), fg_bf16_hi(v.x), d, 0);
    lo = fg_cvt2q<MODE, true>(fg_bf16_lo(v.y), fg_bf16_hi(v.y), d, lo);
    uint32_t hi = fg_cvt2q<MODE, false>(fg_bf16_lo(v.z), fg_bf16_hi(v.z), d, 0);
    hi = fg_cvt2q<MODE, true>(fg_bf16_lo(v.w), fg_bf16_hi(v.w), d, hi);
    return make_uint2(lo, hi);
}
// Same, picking the form at run time: pow2 is uniform; FAST unless some lane of the wave has a tiny scale,
// and then each lane takes the form of its own group. Call with the whole wave active.
__device__ __forceinline__ uint2 fg_quant8_any(uint4 v, const fg_divisor& d, int pow2) {
    if (pow2) return fg_quant8<FG_Q_POW2>(v, d);
    if (__builtin_amdgcn_ballot_w64(fg_divisor_tiny(d)) == 0) return fg_quant8<FG_Q_FAST>(v, d);
    return fg_divisor_tiny(d) ? fg_quant8<FG_Q_TINY>(v, fg_divisor_shifted(d)) : fg_quant8<FG_Q_FAST>(v, d);
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
