/* Exhaustive check of the identity the quantizer kernels rely on: for every pair of bf16
 * values (x, amax) with |x| <= amax, amax > 0, and s = fl32(amax / 448),
 *     fl32(x * fl64(1 / s)) == fl32(x / s)         (both IEEE, round to nearest even)
 * and |x / s| < 464 (the range where the E4M3 converter saturates to 448 by rounding).
 * Prints "pairs P mismatches Q maxabs A". Built with gcc -O2 -fopenmp; no fast-math. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float bf16(uint32_t h) { uint32_t u = h << 16; float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

int main(void) {
  long long pairs = 0, bad = 0;
  float maxabs = 0.0f;
#pragma omp parallel for reduction(+ : pairs, bad) reduction(max : maxabs) schedule(dynamic, 64)
  for (uint32_t ha = 1; ha < 0x7F80u; ++ha) {       /* every finite positive bf16 amax */
    const float amax = bf16(ha);
    const float s = amax / 448.0f;
    const double r = 1.0 / (double)s;
    for (uint32_t hx = 0; hx <= ha; ++hx) {          /* every bf16 magnitude up to amax */
      for (uint32_t sg = 0; sg < 2; ++sg) {
        const float x = bf16(hx | (sg << 15));
        const float exact = x / s;
        const float fast = (float)((double)x * r);
        ++pairs;
        if (bits(exact) != bits(fast)) ++bad;
        if (fabsf(exact) > maxabs) maxabs = fabsf(exact);
      }
    }
  }
  printf("pairs %lld mismatches %lld maxabs %.9g\n", pairs, bad, maxabs);
  return bad != 0;
}
