/* Exhaustive check of the FP8 row quantizer's fast division (CPU, test only).
 *
 * The quantizer's code is RNE_E4M3(fl32(x / s)) with s = fl32(amax / 448) the row
 * scale.  For rows whose largest magnitude amax is at least AMAX_MIN_BITS (a bf16
 * bit pattern) the kernel forms the quotient as
 *     r  = fl32(1 / s)                      (IEEE division, once per row)
 *     q0 = fl32(|x| * r)
 *     q  = copysign(fma(fma(-q0, s, |x|), r, q0), x)
 * This program checks, for every positive finite bf16 amax >= AMAX_MIN_BITS and every
 * bf16 x with |x| <= amax, that q equals fl32(x / s) bit for bit whenever
 * |x / s| >= 2^-10, and that otherwise |q| <= 2^-10 with the sign of x: below 2^-10
 * (the rounding midpoint under E4M3's smallest subnormal, 2^-9) both round to the same
 * signed zero.  Exit status 0 when every pair passes.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#ifndef AMAX_MIN_BITS
#define AMAX_MIN_BITS 0x2180u   /* 2^-60 */
#endif

static float bf16(uint32_t b) { uint32_t u = b << 16; float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

int main(void) {
  const float tiny = ldexpf(1.0f, -10);
  long long pairs = 0, bad = 0;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : pairs, bad)
  for (uint32_t a = AMAX_MIN_BITS; a <= 0x7F7Fu; ++a) {
    const float s = bf16(a) / 448.0f;
    const float r = 1.0f / s;
    for (uint32_t m = 0; m <= a; ++m)
      for (uint32_t sg = 0; sg < 2; ++sg) {
        const float x = bf16(m | (sg << 15));
        const float ref = x / s;
        const float ax = fabsf(x);
        const float q0 = ax * r;
        const float q = copysignf(fmaf(fmaf(-q0, s, ax), r, q0), x);
        ++pairs;
        const int ok = fabsf(ref) >= tiny ? bits(q) == bits(ref)
                                          : fabsf(q) <= tiny && signbit(q) == signbit(ref);
        if (!ok) {
          ++bad;
#pragma omp critical
          if (bad < 5) printf("mismatch: amax %04x x %04x: x/s %a, fast %a\n", a, m | (sg << 15), ref, q);
        }
      }
  }
  printf("pairs %lld, mismatches %lld\n", pairs, bad);
  return bad != 0;
}
