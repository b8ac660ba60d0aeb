/* The quotient the library's FP8 encoders use, checked against true division.
 *
 * The encoders turn a value v of a block with scale s = amax/448 into the
 * E4M3 code of v/s. Instead of dividing, they take r = 1/s (correctly
 * rounded), y = v*r, and correct y once with its residual:
 *     q = copysign(fma(fma(-s, y, v), r, y), v).
 * This program compares the E4M3 code (round to nearest even, saturating at
 * 448) of q with that of the correctly rounded fp32 quotient v/s, for every
 * fp32 v of both signs whose magnitude lies in [amax * 2^-lo_binades, amax],
 * for the scales given on the command line as amax values (hex floats).
 * Prints the number of code mismatches per scale; exit status 1 if any.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static double val[127]; /* the non-negative finite E4M3 values, by code */

static void init(void) {
  for (int c = 0; c < 127; ++c) {
    const int e = c >> 3, m = c & 7;
    val[c] = e == 0 ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
  }
}

static int e4m3(float v) {
  if (isnan(v)) return 0x7f;
  const int sg = signbit(v) ? 0x80 : 0;
  const double a = fabs((double)v);
  if (a >= 448.0) return sg | 0x7e;
  int lo = 0, hi = 126;
  while (hi - lo > 1) {
    const int mid = (lo + hi) / 2;
    if (val[mid] <= a) lo = mid; else hi = mid;
  }
  const double m = (val[lo] + val[hi]) / 2;
  return sg | (a < m ? lo : a > m ? hi : ((lo & 1) ? hi : lo));
}

int main(int argc, char** argv) {
  init();
  if (argc < 3) { fprintf(stderr, "usage: %s lo_binades amax...\n", argv[0]); return 2; }
  const int lo_binades = atoi(argv[1]);
  long long all_bad = 0;
  for (int t = 2; t < argc; ++t) {
    const float amax = strtof(argv[t], NULL);
    const float s = amax / 448.0f, r = 1.0f / s;
    const uint32_t top = u_of(amax);
    const float lo_v = ldexpf(amax, -lo_binades);
    const uint32_t bottom = u_of(lo_v);
    long long bad = 0, n = 0;
#pragma omp parallel for reduction(+ : bad, n) schedule(static)
    for (int64_t i = bottom; i <= (int64_t)top; ++i) {
      for (int sg = 0; sg < 2; ++sg) {
        const float v = f_of((uint32_t)i | (sg ? 0x80000000u : 0u));
        const float y = v * r;
        const float q = copysignf(fmaf(fmaf(-s, y, v), r, y), v);
        n++;
        if (e4m3(q) != e4m3(v / s)) bad++;
      }
    }
    printf("amax %a: %lld values, %lld code mismatches\n", amax, n, bad);
    all_bad += bad;
  }
  return all_bad != 0;
}
