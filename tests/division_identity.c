/*
 * Exhaustive checks of the two division shortcuts the activation quantizer
 * uses in place of IEEE fp32 division (host C, no GPU):
 *
 *  1. quotient: for r = fl32(1/s), q0 = x*r, e = fma(q0, s, -x),
 *     q = fma(-e, r, q0) equals fl32(x/s) for every bf16 significand of x and
 *     every fp32 significand of s (2^7 * 2^23 pairs, both in [1, 2); the
 *     identity is invariant under scaling x and s by powers of two while no
 *     intermediate leaves the normal range);
 *  2. scale: with R = fl32(1/448), q0 = a*R, e = fma(q0, 448, -a),
 *     s = fma(-e, R, q0) equals fl32(a/448) for every fp32 a from fl32(1e-4)
 *     to the largest finite value.
 *
 * Exit status 0 when both hold.  Built with -ffp-contract=off so the only
 * fused operations are the explicit fmaf calls (correctly rounded, as the
 * GPU's v_fma_f32).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static inline float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static inline uint32_t to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

int main(void) {
  long long bad_q = 0, bad_s = 0, n_s = 0;
  volatile float one = 1.0f, c448 = 448.0f;

#pragma omp parallel for reduction(+ : bad_q) schedule(static)
  for (uint32_t sm = 0; sm < (1u << 23); ++sm) {
    const float s = from_bits(0x3F800000u | sm);
    const float r = one / s;
    for (uint32_t xm = 0; xm < 128; ++xm) {
      const float x = from_bits(0x3F800000u | (xm << 16));
      const float q0 = x * r;
      const float e = fmaf(q0, s, -x);
      const float q = fmaf(-e, r, q0);
      bad_q += to_bits(q) != to_bits(x / s);
    }
  }

  const float R = one / c448;
  const uint32_t lo = to_bits(1e-4f), hi = 0x7F7FFFFFu;
#pragma omp parallel for reduction(+ : bad_s, n_s) schedule(static)
  for (uint32_t u = lo; u <= hi; ++u) {
    const float a = from_bits(u);
    const float q0 = a * R;
    const float e = fmaf(q0, 448.0f, -a);
    const float s = fmaf(-e, R, q0);
    bad_s += to_bits(s) != to_bits(a / c448);
    n_s++;
  }
  printf("quotient identity: %lld mismatches of %lld; scale identity: %lld mismatches of %lld\n",
         bad_q, (long long)128 << 23, bad_s, n_s);
  return (bad_q || bad_s) ? 1 : 0;
}
