/* divby_exhaustive.c -- CPU check of the correctly rounded division by the
 * constants 6 and 7 that the quantizers use for the block maximum: with
 * q0 = a * fp32(1/d), r = fma(-q0, d, a) and q = fma(r, fp32(1/d), q0), q is
 * the IEEE quotient a / d for every finite fp32 a >= 2^-119 (below that the
 * kernels divide).  Built and run by tests/test_divby_cpu.py; prints the
 * number of mismatches for d = 6 and d = 7 and the first one. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float from_bits(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }

static unsigned long long check(float d, uint32_t *first) {
  const float inv = 1.0f / d;
  const uint32_t lo = 0x04000000u;                   /* 2^-119 */
  unsigned long long bad = 0;
  uint32_t f = 0;
#pragma omp parallel for reduction(+ : bad) schedule(dynamic, 1 << 20)
  for (int64_t i = lo; i < 0x7F800000; i++) {
    const float a = from_bits((uint32_t)i);
    const float q0 = a * inv;
    const float r = fmaf(-q0, d, a);
    const float q = fmaf(r, inv, q0);
    const float want = a / d;
    if (memcmp(&q, &want, 4) != 0) {
      bad++;
#pragma omp critical
      if (!f) f = (uint32_t)i;
    }
  }
  *first = f;
  return bad;
}

int main(void) {
  uint32_t f6, f7;
  unsigned long long b6 = check(6.0f, &f6), b7 = check(7.0f, &f7);
  printf("%llu %u %llu %u\n", b6, f6, b7, f7);
  return 0;
}
