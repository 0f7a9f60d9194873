/* Exhaustive check of the two division shortcuts in the INT4 group quantizer of the activation
 * kernel (w4a4_device.hip: int4_scale, int4_recip), against IEEE division as the method's oracle
 * computes it:
 *   1. s = bf16(fp32(amax / 7)), flushed to 0 below 2^-126, for every finite fp32 amax >= 0:
 *      the kernel forms q0 = amax * fp32(1/7), corrects it once with its exact fma residual,
 *      q = fma(fma(-7, q0, amax), fp32(1/7), q0), and rounds q to bf16. (With fp32 denormals
 *      flushed the residual of tiny maxima would be lost; the check also reports that case.)
 *   2. 1/s for every bf16 scale s >= 2^-126 that can occur (s <= FLT_MAX / 7): one Newton step
 *      y = fma(fma(-s, y0, 1), y0, y0) from any y0 within one ulp of 1/s (the hardware reciprocal
 *      is such an approximation) gives the correctly rounded quotient 1.0f / s.
 * Prints the mismatch counts; exit status 0 when both exact checks have none. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static uint32_t bf16_bits(float f) { uint32_t u = u_of(f); return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16; }
static float scale_of(float q) { float s = f_of(bf16_bits(q) << 16); return s >= 0x1p-126f ? s : 0.0f; }

int main(void) {
  const float c = 1.0f / 7.0f;
  unsigned long long bad = 0, bad_flushed = 0, bad_rcp = 0, n_rcp = 0;
#pragma omp parallel for reduction(+ : bad, bad_flushed) schedule(static)
  for (long long i = 0; i < 0x7F800000LL; ++i) {
    const float a = f_of((uint32_t)i);
    const float want = scale_of(a / 7.0f);
    const float q0 = a * c;
    const float r = fmaf(-7.0f, q0, a);
    if (u_of(scale_of(fmaf(r, c, q0))) != u_of(want)) ++bad;
    const float rf = fabsf(r) < 0x1p-126f ? 0.0f : r;
    if (u_of(scale_of(fmaf(rf, c, q0))) != u_of(want)) ++bad_flushed;
  }
  for (uint32_t h = 0x0080; h < 0x7F80; ++h) {
    const float s = f_of(h << 16);
    if (s > 0x1.fffffep127f / 7.0f) break;
    const float want = 1.0f / s;
    for (int d = -1; d <= 1; ++d) {
      const float y0 = f_of(u_of(want) + d);
      const float y = fmaf(fmaf(-s, y0, 1.0f), y0, y0);
      ++n_rcp;
      if (u_of(y) != u_of(want)) ++bad_rcp;
    }
  }
  printf("scale: %llu mismatches (%llu with fp32 denormals flushed); reciprocal: %llu of %llu\n", bad, bad_flushed,
         bad_rcp, n_rcp);
  return (bad == 0 && bad_rcp == 0) ? 0 : 1;
}
