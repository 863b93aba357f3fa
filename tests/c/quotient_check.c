/* Division-free correctly rounded quotient, checked against IEEE division.
 *
 * The quantizers form RN(a / s) for a = RN(x - mn) (0, or at least 2^-24, since x and
 * mn are float16 values) and a float16 scale s > 0 as
 *     inv = RN(1 / s);  q0 = RN(a * inv);  q = RN(q0 + RN(a - q0 * s) * inv)
 * with both inner steps single FMAs (Markstein's theorem).  This program compares
 * q with a / s for every positive finite float16 s and, for each, every float32 a
 * within 300 ulps of k*s and (k + 1/2)*s for k = 0 .. 24 (every code boundary and
 * tie, including codes past 2^b - 1 that a subnormal s can produce) plus 2000
 * pseudo-random a in [2^-24, 24 s].  Exit status 0 when all agree.
 * Build: gcc -O2 -ffp-contract=off quotient_check.c -lm */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float half_to_float(uint16_t h) {
  const int e = (h >> 10) & 31, m = h & 1023;
  return e == 0 ? ldexpf((float)m, -24) : ldexpf((float)(m | 1024), e - 25);
}

static float step_ulps(float x, int k) {
  uint32_t u;
  memcpy(&u, &x, 4);
  u += (uint32_t)k;
  memcpy(&x, &u, 4);
  return x;
}

static long n_tests, n_bad;

static void check(float a, float s, float inv) {
  if (!(a >= 0x1p-24f)) return;
  volatile float q0 = a * inv;
  const float q = fmaf(fmaf(-q0, s, a), inv, q0);
  volatile float ref = a / s;
  ++n_tests;
  if (q != ref) {
    if (n_bad < 10) printf("mismatch: s=%a a=%a q=%a a/s=%a\n", s, a, q, ref);
    ++n_bad;
  }
}

int main(void) {
  uint64_t state = 12345;
  for (uint32_t hs = 1; hs < 0x7c00; ++hs) {
    const float s = half_to_float((uint16_t)hs);
    volatile float one = 1.0f;
    const float inv = one / s;
    for (int k = 0; k <= 24; ++k)
      for (int half = 0; half < 2; ++half) {
        const float c = (k + 0.5f * half) * s;
        for (int p = -300; p <= 300; ++p) check(step_ulps(c, p), s, inv);
      }
    for (int i = 0; i < 2000; ++i) {
      state = state * 6364136223846793005ULL + 1442695040888963407ULL;
      check((float)((state >> 40) * (1.0 / 16777216.0)) * 24.f * s, s, inv);
    }
  }
  printf("checked %ld quotients, %ld mismatches\n", n_tests, n_bad);
  return n_bad != 0;
}
