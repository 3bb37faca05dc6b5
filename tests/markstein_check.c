/* Exhaustive check, on the host, that the quotient fl32(x / s) is obtained from the
 * correctly rounded reciprocal r = fl32(1 / s) by one residual step
 *     q = fl32(x r),  e = fma(-q, s, x) (exact),  t = fl32(fma(e, r, q))
 * (Markstein's division) for every float x of one binade and every positive E4M3
 * value s.  Scaling x by a power of two scales q, e and t exactly while no value
 * leaves the normal range, so one binade of x stands for every binade whose
 * quotients stay normal.  Prints the number of mismatches; exits 1 if any. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float e4m3_value(int c) { /* positive E4M3 (OCP FN): codes 1..126 */
  int e = (c >> 3) & 15, m = c & 7;
  return e == 0 ? ldexpf((float)m, -9) : ldexpf((float)(8 + m), e - 10);
}

int main(int argc, char** argv) {
  int lo = argc > 1 ? atoi(argv[1]) : 1, hi = argc > 2 ? atoi(argv[2]) : 126;
  long long bad = 0, n = 0;
  for (int c = lo; c <= hi; c++) {
    const volatile float s = e4m3_value(c);
    const float r = 1.0f / s;
    for (uint32_t m = 0; m < (1u << 23); m++) {
      uint32_t u = (127u << 23) | m; /* x in [1, 2) */
      float x;
      memcpy(&x, &u, 4);
      const float q = x * r;
      const float t = fmaf(fmaf(-q, s, x), r, q);
      const volatile float ref = x / s;
      n++;
      if (t != ref) bad++;
    }
  }
  printf("%lld of %lld quotients differ\n", bad, n);
  return bad != 0;
}
