/* Exhaustive check of the reciprocal-and-residual quotient the per-row int8
 * quantiser kernel uses in place of a full IEEE division.
 *
 * The quantiser's scale is s = RN(a / 127) with a the absmax of a row of
 * fp16 values, so s takes one of 31743 values (a positive and finite).  For
 * each such s, with r = RN(1 / s), and for every finite fp16 x, this program
 * evaluates q0 = RN(x r), e = fma(-q0, s, x), q = RN(e r + q0) in binary32
 * and counts the pairs where q differs from RN(x / s), and the pairs where
 * the int8 code (nearest-even integer, clamped to [-127, 127]) differs.
 * Prints "pairs P quotient_mismatches Q code_mismatches C".
 *
 * Built with -ffp-contract=off: every product and sum above is one IEEE
 * operation, fmaf a fused one. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>

static float half_value(uint16_t h) {
  const int e = (h >> 10) & 31, m = h & 1023;
  const float v = e == 0 ? ldexpf((float)m, -24) : ldexpf((float)(m | 1024), e - 25);
  return (h & 0x8000) ? -v : v;
}

static int code_of(float q) {
  float c = rintf(q);
  if (c > 127.f) c = 127.f;
  if (c < -127.f) c = -127.f;
  return (int)c;
}

int main(void) {
  long long pairs = 0, bad_q = 0, bad_code = 0;
#pragma omp parallel for reduction(+ : pairs, bad_q, bad_code) schedule(dynamic, 64)
  for (int a = 1; a < 0x7C00; ++a) {
    volatile float amax = half_value((uint16_t)a);
    volatile float s = amax / 127.0f;
    volatile float r = 1.0f / s;
    for (int xb = 0; xb < 0xFC00; ++xb) {
      if (xb >= 0x7C00 && xb < 0x8000) continue; /* inf and NaN */
      const float x = half_value((uint16_t)xb);
      volatile float exact = x / s;
      volatile float q0 = x * r;
      const float q = fmaf(fmaf(-q0, s, x), r, q0);
      ++pairs;
      bad_q += q != exact;
      bad_code += code_of(q) != code_of(exact);
    }
  }
  printf("pairs %lld quotient_mismatches %lld code_mismatches %lld\n", pairs, bad_q, bad_code);
  return 0;
}
