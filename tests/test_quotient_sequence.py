"""Exhaustive host-side proof of the quantizers' division sequence.

The GPU kernels form x / s as q0 = RN(x * RN(1/s)), rem = fma(-q0, s, x), q = copysign(fma(rem, RN(1/s), q0), x),
after moving tiny scales (s < 2^-100) and x up by 2^64. This test runs the same sequence in C on the
host for every positive bf16 max-abs (both scale modes) and every bf16 |x| <= max-abs and checks that it
equals IEEE division whenever |x/s| >= 2^-12 and that the E4M3 code (nearest, ties to even, signed zero)
is the same in all cases. It shares no code with the oracle or the kernels; it only justifies replacing
a division by a multiply and two FMAs.
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
static float scale_of(uint32_t ab, int pow2){
  float s = f_of(ab << 16) / 448.0f; if (s < 1.17549435e-38f) s = 1.17549435e-38f;
  if (pow2) { uint32_t u = u_of(s); if (u & 0x7FFFFF) u = (u & 0x7F800000u) + 0x800000u; s = f_of(u); }
  return s; }
static int code(float v){ double a = fabs(v); int sg = signbit(v) ? 0x80 : 0; double best = 1e300; int bc = 0;
  for (int c = 0; c < 127; c++) { int e = c >> 3, m = c & 7; double val = e ? ldexp(1.0 + m / 8.0, e - 7) : ldexp(m, -9);
    double d = fabs(a - val); if (d < best || (d == best && (c & 1) == 0)) { best = d; bc = c; } }
  return sg | bc; }
int main(){
  long long bad_q = 0, bad_code = 0, total = 0;
  for (int pow2 = 0; pow2 < 2; pow2++) {
    #pragma omp parallel for reduction(+:bad_q,bad_code,total) schedule(dynamic,64)
    for (uint32_t ab = 1; ab < 0x7F80; ab++) {
      float s0 = scale_of(ab, pow2), pre = s0 < 0x1p-100f ? 0x1p64f : 1.0f, s = s0 * pre, r = 1.0f / s;
      for (uint32_t xb = 0; xb <= ab; xb++) {
        for (int sign = 0; sign < 2; sign++) {
          float x0 = f_of((xb << 16) | (sign ? 0x80000000u : 0)), x = x0 * pre;
          float q0 = x * r, rem = fmaf(-q0, s, x), q = copysignf(fmaf(rem, r, q0), x), e = x0 / s0;
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
  printf("%lld %lld %lld\n", total, bad_q, bad_code);
  return 0;
}
"""


def test_division_sequence_exhaustive():
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "q.c"), os.path.join(d, "q")
        open(src, "w").write(SRC)
        subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-mfma", src, "-o", exe, "-lm"], check=True)
        out = subprocess.run([exe], check=True, capture_output=True, text=True, timeout=600).stdout.split()
    total, bad_q, bad_code = map(int, out)
    assert total > 2_000_000_000
    assert bad_q == 0
    assert bad_code == 0
