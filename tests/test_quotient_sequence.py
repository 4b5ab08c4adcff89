"""Exhaustive host-side proof of the quantizers' scale and division sequences.

The GPU kernels never call an IEEE division per element. For a group with max-abs a (a bf16 value) they form
  s  = RN(a / 448) as q0 = RN(a * RN(1/448)), rem = fma(-q0, 448, a), s = fma(rem, RN(1/448), q0)
       (then the clamp to FLT_MIN and, in power-of-2 mode, the round-up to 2^k), and r = RN(1/s);
and the quotient handed to the E4M3 conversion for each element x is
  power-of-2 scales:  x * r                              (r = 2^-k, taken from the exponent field of s,
                                                          so the product is the exact quotient);
  other scales:       fma(-t, r, q0), q0 = RN(x * r), t = fma(q0, s, -x)
                      (Markstein's correction step with the remainder carried negated: the negations
                      are free FMA operand modifiers on the GPU, and they keep x = -0 at -0);
                      a group with s < 2^-100 first moves s and x up by 2^64 (exact, changes no quotient).
This test runs exactly these sequences in C on the host, for every positive bf16 max-abs in both modes and
every bf16 |x| <= max-abs of either sign, and checks that s equals the IEEE quotient, and that the
element quotient equals IEEE division whenever |x/s| >= 2^-12 and encodes to the same E4M3 code (nearest,
ties to even, signed zero) in every case. It shares no code with the oracle or the kernels; it only
justifies replacing divisions by multiplies and FMAs.
"""
import os
import subprocess
import tempfile

SRC = r"""
#include <stdio.h>
#include <stdint.h>
#include <string.h>
#include <math.h>
static float f_of(uint32_t u){float f; memcpy(&f,&u,4); return f;}
static uint32_t u_of(float f){uint32_t u; memcpy(&u,&f,4); return u;}
static float pow2_up(float s){ uint32_t u = u_of(s); if (u & 0x7FFFFF) u = (u & 0x7F800000u) + 0x800000u; return f_of(u); }
/* reference: IEEE division, clamp, round-up */
static float scale_ieee(uint32_t ab, int pow2){
  float s = f_of(ab << 16) / 448.0f; if (s < 1.17549435e-38f) s = 1.17549435e-38f;
  return pow2 ? pow2_up(s) : s; }
/* the kernels' sequence */
static float scale_seq(uint32_t ab, int pow2){
  const float a = f_of(ab << 16), c = 0x1.24924ap-9f;
  float q0 = a * c, rem = fmaf(-q0, 448.0f, a), s = fmaf(rem, c, q0);
  if (s < 1.17549435e-38f) s = 1.17549435e-38f;
  return pow2 ? pow2_up(s) : s; }
static int code(float v){ double a = fabs(v); int sg = signbit(v) ? 0x80 : 0; double best = 1e300; int bc = 0;
  for (int c = 0; c < 127; c++) { int e = c >> 3, m = c & 7; double val = e ? ldexp(1.0 + m / 8.0, e - 7) : ldexp(m, -9);
    double d = fabs(a - val); if (d < best || (d == best && (c & 1) == 0)) { best = d; bc = c; } }
  return sg | bc; }
int main(){
  long long bad_s = 0, bad_q = 0, bad_code = 0, total = 0, tiny = 0;
  for (int pow2 = 0; pow2 < 2; pow2++)
    for (uint32_t ab = 1; ab < 0x7F80; ab++)
      if (u_of(scale_seq(ab, pow2)) != u_of(scale_ieee(ab, pow2))) bad_s++;
  for (int pow2 = 0; pow2 < 2; pow2++) {
    #pragma omp parallel for reduction(+:bad_q,bad_code,total,tiny) schedule(dynamic,64)
    for (uint32_t ab = 1; ab < 0x7F80; ab++) {
      const float s0 = scale_ieee(ab, pow2), r0 = 1.0f / s0;
      const int is_tiny = !pow2 && s0 < 0x1p-100f;
      const float pre = is_tiny ? 0x1p64f : 1.0f, s = s0 * pre, r = r0 * (is_tiny ? 0x1p-64f : 1.0f);
      if (is_tiny && u_of(r) != u_of(1.0f / s)) bad_q += 1000000;   /* r must be RN(1/s) after the shift */
      /* power-of-2 mode: r = 2^-k from the exponent field alone */
      if (pow2 && u_of(r0) != ((254u - (u_of(s0) >> 23)) << 23)) bad_q += 1000000;
      tiny += is_tiny;
      for (uint32_t xb = 0; xb <= ab; xb++) {
        for (int sign = 0; sign < 2; sign++) {
          const float x0 = f_of((xb << 16) | (sign ? 0x80000000u : 0)), e = x0 / s0;
          float q;
          if (pow2) {
            q = x0 * r0;
          } else {
            /* every FMA result and negated operand goes through a volatile: gcc otherwise folds a
               negation into a neighbouring FMA (-(a*b+c) as -(a*b)-c), which loses the sign of a zero
               result; the GPU executes the two FMAs exactly as written, with negated operands */
            const float x = x0 * pre, q0 = x * r;
            volatile float nx = -x;
            volatile float t = fmaf(q0, s, nx);
            volatile float nt = -t;
            q = fmaf(nt, r, q0);
          }
          total++;
          if (u_of(q) != u_of(e)) {
            if (fabsf(e) >= 0x1p-12f) bad_q++;
            if (fabsf(q) >= 0x1p-11f || fabsf(e) >= 0x1p-11f) { if (code(q) != code(e)) bad_code++; }
            else if (signbit(q) != signbit(e)) bad_code++;
          }
        }
      }
    }
  }
  printf("%lld %lld %lld %lld %lld\n", total, bad_s, bad_q, bad_code, tiny);
  return 0;
}
"""


def test_scale_and_division_sequences_exhaustive():
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "q.c"), os.path.join(d, "q")
        open(src, "w").write(SRC)
        subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-mfma", src, "-o", exe, "-lm"], check=True)
        out = subprocess.run([exe], check=True, capture_output=True, text=True, timeout=900).stdout.split()
    total, bad_s, bad_q, bad_code, tiny = map(int, out)
    assert total > 2_000_000_000
    assert tiny > 0                      # the prescaled path was exercised
    assert bad_s == 0
    assert bad_q == 0
    assert bad_code == 0
