/* Host check of the quantize kernels' quotient: for a divisor D with at most 4
 * significant bits, the quotient computed as
 *     q0 = RN(x r),  rem = x - q0 D (one fma, exact),  q = RN(q0 + rem r)
 * with r = RN(1/D) must take the same nearest-even decision as the exact real
 * x / D, both for the E2M1 element codes (D = M 2^E, M = 1..15: every E4M3
 * value) and for the E4M3 block scale (D = 6, times the global scale's power of
 * two). Powers of two scale x, D and q exactly, so one binade range of D per
 * mantissa covers all of them. Every binary32 x in the binades where the
 * decision can change is tried; the exact decision is taken from comparisons of
 * x with exact products (double), independently of the quotient.
 *
 * Exit status 0 when every decision agrees; prints the first mismatches. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static float quotient(float x, float D, float r) {
  float q0 = x * r;
  float rem = fmaf(-q0, D, x);
  return -fmaf(-rem, r, -q0);
}

/* E2M1 magnitude code of the real y = a / D: the number of midpoints
 * 0.25 0.75 1.25 1.75 2.5 3.5 5 (times D) that a passes, where a tie passes
 * only a midpoint whose lower code is odd. */
static int e2m1_decision(double a, double D) {
  static const double mid[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
  int k = 0;
  for (int i = 0; i < 7; ++i) k += (a > mid[i] * D) || (a == mid[i] * D && (i & 1));
  return k;
}

static double e4m3_value(int k) { return k < 8 ? k / 512.0 : ldexp(8 + (k & 7), (k >> 3) - 10); }

/* E4M3 byte of the real a / den: binary search over the midpoints of the 127
 * finite non-negative values, ties to the even byte, saturating at 126. */
static int e4m3_decision(double a, double den) {
  int lo = 0, hi = 126;
  while (lo < hi) {
    int k = (lo + hi) / 2;
    double t = den * 0.5 * (e4m3_value(k) + e4m3_value(k + 1));
    if (a > t || (a == t && (k & 1))) lo = k + 1; else hi = k;
  }
  return lo;
}

int main(void) {
  long bad = 0;
  /* element codes: x / M over [1/16, 8) (codes are 0 below and saturate above;
   * the kernel never forms the quotient of a block whose amax exceeds 6 * 448 g) */
  for (int M = 1; M <= 15; ++M) {
    const float D = (float)M, r = 1.0f / D;
    const uint32_t lo = to_bits(D / 16), hi = to_bits(8 * D);
    long b = 0;
#pragma omp parallel for reduction(+ : b) schedule(static)
    for (int64_t u = lo; u < (int64_t)hi; ++u) {
      const float x = from_bits((uint32_t)u);
      const float q = quotient(x, D, r);
      if (e2m1_decision((double)q, 1.0) != e2m1_decision((double)x, (double)D)) ++b;
      /* the sign of x is kept, also for a zero quotient */
      if (signbit(quotient(-x, D, r)) == 0) ++b;
    }
    if (b) printf("E2M1 divisor %d: %ld mismatches\n", M, b);
    bad += b;
  }
  if (!signbit(quotient(-0.0f, 3.0f, 1.0f / 3.0f)) || signbit(quotient(0.0f, 3.0f, 1.0f / 3.0f))) {
    printf("zero quotient loses its sign\n");
    ++bad;
  }
  /* block scale: amax / 6 over [2^-11, 2^10) (zero below, saturated above) */
  {
    const float D = 6.0f, r = 1.0f / D;
    const uint32_t lo = to_bits(6 * 0x1p-11f), hi = to_bits(6 * 1024.0f);
    long b = 0;
#pragma omp parallel for reduction(+ : b) schedule(static)
    for (int64_t u = lo; u < (int64_t)hi; ++u) {
      const float a = from_bits((uint32_t)u);
      if (e4m3_decision((double)quotient(a, D, r), 1.0) != e4m3_decision((double)a, 6.0)) ++b;
    }
    if (b) printf("E4M3 scale: %ld mismatches\n", b);
    bad += b;
  }
  printf("%s\n", bad ? "FAIL" : "all decisions agree");
  return bad ? 1 : 0;
}
