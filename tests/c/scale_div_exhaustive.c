/* Exhaustive check of the INT8 kernels' block-scale formula: for every
 * non-negative finite binary32 m,
 *   q0 = RN(m * RN(1/127)),  s = RN(fma(RN(fma(-q0, 127, m)), RN(1/127), q0))
 * equals the correctly rounded quotient RN(m / 127).  Prints the number of
 * mismatches (0 expected). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

int main(void) {
  const float inv = 1.0f / 127.0f;
  unsigned long long bad = 0;
#pragma omp parallel for reduction(+ : bad) schedule(static)
  for (long long u = 0; u < 0x7f800000ll; ++u) {
    const uint32_t b = (uint32_t)u;
    float m, want, s;
    memcpy(&m, &b, 4);
    want = m / 127.0f;
    const float q0 = m * inv;
    s = fmaf(fmaf(-q0, 127.0f, m), inv, q0);
    uint32_t ws, gs;
    memcpy(&ws, &want, 4);
    memcpy(&gs, &s, 4);
    bad += ws != gs;
  }
  printf("%llu\n", bad);
  return 0;
}
