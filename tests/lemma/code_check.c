/* Exhaustive check of the division-free form the quantizer kernels use for fp32 scales: for
 * every pair of bf16 values (x, amax) with |x| <= amax, amax > 0, and a normal
 * s = fl32(amax / 448) (amax >= 448 * 2^-126), with
 *     h = 1/s rounded toward zero,  l = fl32(fl32(1 - h s) * h),  q = fl32(x h + fl32(x l))
 * (fma for the residual and for q), the E4M3 value of q, sign of zero included, equals the
 * E4M3 value of fl32(x / s). E4M3 rounding here: nearest, ties to even, on the grid with
 * 3 fraction bits, exponents -6 .. 8, subnormal step 2^-9, largest value 448.
 * Prints "pairs P mismatches Q maxabs A" (A: the largest |q|). Built with gcc -O2 -fopenmp
 * -ffp-contract=off; no fast-math. -DDROP_LOW_PART builds the control q = fl32(x h), which must
 * show mismatches (x / s exactly on an E4M3 rounding tie). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float bf16(uint32_t h) { uint32_t u = h << 16; float f; memcpy(&f, &u, 4); return f; }

static double e4m3(float v) {              /* |v| < 464 */
  const double a = fabs((double)v);
  int e = -6;
  if (a >= 0x1p-6) { frexp(a, &e); e -= 1; }   /* a in [2^e, 2^(e+1)) */
  const double step = ldexp(1.0, e - 3);
  double q = rint(a / step) * step;          /* exact: a / step has at most 24 bits */
  if (q > 448.0) q = 448.0;
  return copysign(q, (double)v);
}

static float round_down_reciprocal(float s) {
  float h = 1.0f / s;
  if (fmaf(-h, s, 1.0f) < 0.0f) { uint32_t u; memcpy(&u, &h, 4); --u; memcpy(&h, &u, 4); }
  return h;
}

int main(void) {
  long long pairs = 0, bad = 0;
  float maxabs = 0.0f;
#pragma omp parallel for reduction(+ : pairs, bad) reduction(max : maxabs) schedule(dynamic, 64)
  for (uint32_t ha = 1; ha < 0x7F80u; ++ha) {       /* every finite positive bf16 amax */
    const float amax = bf16(ha);
    const float s = amax / 448.0f;
    if (!(s >= 0x1p-126f)) continue;                 /* subnormal s: the fp64 form */
    const float h = round_down_reciprocal(s);
    const float l = fmaf(-h, s, 1.0f) * h;
    for (uint32_t hx = 0; hx <= ha; ++hx) {          /* every bf16 magnitude up to amax */
      for (uint32_t sg = 0; sg < 2; ++sg) {
        const float x = bf16(hx | (sg << 15));
#ifdef DROP_LOW_PART                                  /* control: the one-multiply form */
        const float q = x * h + 0.0f * l;
#else
        const float q = fmaf(x, h, x * l);
#endif
        const double want = e4m3(x / s), got = e4m3(q);
        ++pairs;
        if (memcmp(&want, &got, sizeof want) != 0) ++bad;
        if (fabsf(q) > maxabs) maxabs = fabsf(q);
      }
    }
  }
  printf("pairs %lld mismatches %lld maxabs %.9g\n", pairs, bad, maxabs);
  return bad != 0;
}
