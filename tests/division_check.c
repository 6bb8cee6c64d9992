/* Exhaustive check of the quantizer's quotient: for every bf16 divisor significand
 * b in [1, 2) and every fp32 dividend significand a in [1, 2),
 *   y = 1 / b (IEEE), q0 = a y, r = fma(-b, q0, a), q = fma(r, y, q0)
 * equals the IEEE quotient a / b (Markstein's one-step correction from a correctly
 * rounded reciprocal).  Powers of two scale every step exactly, so this covers every
 * normal dividend and bf16 divisor.  Prints the counts; exit status 1 on any mismatch. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float from_bits(uint32_t u) {
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

int main(void) {
  long long bad = 0, total = 0;
#pragma omp parallel for reduction(+ : bad, total) schedule(dynamic)
  for (int bs = 0x3F80; bs <= 0x3FFF; ++bs) {
    const float b = from_bits((uint32_t)bs << 16);
    const float y = 1.0f / b;
    for (uint32_t m = 0; m < (1u << 23); ++m) {
      const float a = from_bits(0x3F800000u | m);
      const float q0 = a * y;
      const float q = fmaf(fmaf(-b, q0, a), y, q0);
      total++;
      if (q != a / b) bad++;
    }
  }
  printf("checked %lld pairs, mismatches %lld\n", total, bad);
  return bad != 0;
}
