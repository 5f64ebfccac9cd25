/*
 * Exhaustive check of the FP8 activation quantiser's quotient (the quantise + gate kernel of
 * the projections): for every bf16 token maximum m with s = m / 448 >= 2^-80 (fp32 division)
 * and every bf16 x with |x| <= m, the kernel's
 *     y = 1 / s,  q0 = x * y,  q = copysign(fma(fma(-s, q0, x), y, q0), x)   (IEEE fp32, nearest)
 * must equal the IEEE quotient x / s wherever |x / s| >= 2^-10, and where the quotient is
 * below that, must not exceed 2^-10 in magnitude and must have the quotient's sign (both then
 * give the zero code of that sign: E4M3FN's smallest subnormal is 2^-9, and 2^-10 rounds to
 * even, i.e. to zero).
 * Prints: pairs checked, differing pairs at or above 2^-10, and pairs crossing 2^-10.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float bf16(uint32_t b) {
  const uint32_t u = b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static uint32_t bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

int main(void) {
  long long pairs = 0, wrong = 0, crossing = 0;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : pairs, wrong, crossing)
  for (int a = 1; a < 0x7F80; ++a) {              /* positive finite bf16 maxima */
    const float m = bf16((uint32_t)a);
    volatile float vs = m / 448.0f;
    const float s = vs;
    if (!(s >= 0x1p-80f)) continue;
    volatile float vy = 1.0f / s;
    const float y = vy;
    for (int xb = 0; xb <= a; ++xb) {
      for (int sg = 0; sg < 2; ++sg) {
        const float x = sg ? -bf16((uint32_t)xb) : bf16((uint32_t)xb);
        volatile float vref = x / s;
        const float ref = vref;
        volatile float vq0 = x * y;
        const float q0 = vq0;
        const float q = copysignf(fmaf(fmaf(-s, q0, x), y, q0), x);
        ++pairs;
        if (fabsf(ref) >= 0x1p-10f) {
          if (bits(q) != bits(ref)) ++wrong;
        } else if (fabsf(q) > 0x1p-10f || signbit(q) != signbit(ref)) {
          ++crossing;
        }
      }
    }
  }
  printf("%lld %lld %lld\n", pairs, wrong, crossing);
  return 0;
}
