/* Host check of the two division sequences of the device quantizer
 * (div_by_levels and recip_of_half_value in the library's device header),
 * written with the same IEEE operations (binary32 multiply and fused
 * multiply-add, round to nearest even, no flush of subnormals):
 *
 *   1. q = fma(fma(-L, q0, a), y, q0), q0 = a * y, y = RN(1/L), equals the
 *      correctly rounded a / L for every non-negative finite binary32 a,
 *      L = 3 and 15 (Markstein's residual correction);
 *   2. r = fma(fma(-b, y0, 1), y0, y0) equals the correctly rounded 1 / b for
 *      every positive finite binary16 value b and every start y0 within two
 *      ulps of 1 / b (the hardware reciprocal is within one ulp).
 *
 * Usage: quantizer_division_check PART NPARTS  (checks its share of the
 * binary32 range; part 0 also runs the reciprocal check).  Prints the
 * mismatch counts and exits non-zero on any mismatch. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float as_float(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }
static uint32_t as_bits(float x) { uint32_t u; memcpy(&u, &x, 4); return u; }

int main(int argc, char **argv) {
  const int64_t part = argc > 2 ? atoll(argv[1]) : 0, nparts = argc > 2 ? atoll(argv[2]) : 1;
  const int64_t top = 0x7F7FFFFFLL, chunk = (top + nparts) / nparts;
  const int64_t lo = part * chunk, hi = lo + chunk - 1 < top ? lo + chunk - 1 : top;
  long bad = 0;
  const float levels[2] = {3.0f, 15.0f};
  for (int li = 0; li < 2; ++li) {
    const float L = levels[li];
    volatile float one = 1.0f;
    const float y = one / L;
    for (int64_t a = lo; a <= hi; ++a) {
      const float x = as_float((uint32_t)a);
      const float q0 = x * y;
      const float r = fmaf(-L, q0, x);
      const float q = fmaf(r, y, q0);
      if (as_bits(q) != as_bits(x / L)) ++bad;
    }
  }
  long badr = 0, tried = 0;
  if (part == 0) {
    for (uint32_t h = 1; h < 0x7C00; ++h) {
      const uint32_t e = (h >> 10) & 31, m = h & 1023;
      const float b = e ? ldexpf((float)(1024 + m), (int)e - 25) : ldexpf((float)m, -24);
      const float ref = 1.0f / b;
      const float ulp = nextafterf(ref, INFINITY) - ref;
      float y0 = nextafterf(nextafterf(ref, 0.0f), 0.0f);
      for (int k = 0; k < 5; ++k, y0 = nextafterf(y0, INFINITY)) {
        if (fabsf(y0 - ref) > 2.0f * ulp) continue;
        const float ee = fmaf(-b, y0, 1.0f);
        const float r1 = fmaf(ee, y0, y0);
        ++tried;
        if (as_bits(r1) != as_bits(ref)) ++badr;
      }
    }
  }
  printf("part %lld/%lld: division mismatches %ld, reciprocal mismatches %ld of %ld\n",
         (long long)part, (long long)nparts, bad, badr, tried);
  return (bad || badr || (part == 0 && tried < 60000)) ? 1 : 0;
}
