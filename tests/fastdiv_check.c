/* fastdiv_check.c -- host check of the division shortcuts the gfx950 kernel
 * takes on its fast paths (the kernel is written against the results below;
 * nothing here is shared with it or with the oracle).
 *
 *  1. x / r for a bf16 numerator x and any fp32 divisor r, from y = RN(1/r):
 *       q0 = x*y;  e = fma(-q0, r, x);  q = fma(e, y, q0)
 *     must equal the IEEE quotient when the quotient is normal.  Checked for
 *     every bf16 significand against every fp32 significand (exponents are a
 *     pure scaling), quotient in [1/2, 2).
 *  2. v / s for bf16 v and bf16 s, from a reciprocal rounded downwards
 *     (rs = RN(1/s), or its predecessor when s*rs > 1, so that the residual
 *     e = fma(-s, rs, 1) is >= 0) and rl = RN(e * rs):
 *       q = fma(v, rs, v*rl)
 *     must equal the IEEE quotient whenever that is at least 2^-100 (below
 *     it v*rl can underflow); below it both must stay under 2^-10, where
 *     every E4M3 code is +-0, so the codes still agree.  Checked for every
 *     pair of bf16 significands and every exponent difference in [-140, 12],
 *     at five absolute scale exponents of s (2^-98, 2^-80, 2^0, 2^92, 2^97).  With
 *     rl >= 0, v*rl has the sign of v, so q keeps the sign of a zero v; the
 *     check covers +-0 too.
 *  3. m / 448 for bf16 m, from the constants H = RN(1/448), Lo = RN(1/448 - H):
 *       q = fma(m, H, m*Lo)
 *     must equal the IEEE quotient for every bf16 m in [2^-71, 2^100].
 *  4. the same for every positive finite fp16 m (fp16 rows of the indexer's
 *     fp8 mode; all of them lie in [2^-24, 65504], inside that range).
 *  5. m / 6 for bf16 m (the FP4 nope mode's scale), from H6 = RN(1/6),
 *     L6 = RN(1/6 - H6): q = fma(m, H6, m*L6) must equal the IEEE quotient
 *     for every bf16 m in [2^-90, 2^100].
 * Prints the number of mismatches of each part and exits non-zero if any.
 * Build: gcc -O2 -std=c99 -ffp-contract=off -fno-fast-math fastdiv_check.c -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

int main(void) {
  long long bad1 = 0, bad2 = 0, bad3 = 0, n1 = 0, n2 = 0, n3 = 0;
  /* 1: bf16 significand a in [1,2), fp32 significand b in [1,2) */
  for (uint32_t mb = 0; mb < (1u << 23); ++mb) {
    const float b = f_of(0x3F800000u | mb);
    const float y = 1.0f / b;
    for (uint32_t ma = 0; ma < 128; ++ma) {
      const float a = f_of(0x3F800000u | (ma << 16));
      const float q0 = a * y;
      const float e = fmaf(-q0, b, a);
      const float q = fmaf(e, y, q0);
      ++n1;
      if (q != a / b) ++bad1;
    }
  }
  /* 2: bf16 / bf16 */
  const int sexp[5] = {-98, -80, 0, 92, 97};
  for (int k = 0; k < 5; ++k) {
    for (uint32_t ms = 0; ms < 128; ++ms) {
      const float s = ldexpf(f_of(0x3F800000u | (ms << 16)), sexp[k]);
      float rs = 1.0f / s;
      if (fmaf(-s, rs, 1.0f) < 0.0f) rs = nextafterf(rs, 0.0f);
      const float e = fmaf(-s, rs, 1.0f);
      const float rl = e * rs;
      if (e < 0.0f) ++bad2;
      for (int z = 0; z < 2; ++z) {
        const float v = z ? -0.0f : 0.0f;
        const float q = fmaf(v, rs, v * rl);
        ++n2;
        if (q != 0.0f || signbit(q) != signbit(v)) ++bad2;
      }
      for (int de = -140; de <= 12; ++de) {
        for (uint32_t mv = 0; mv < 128; ++mv) {
          const float v = ldexpf(f_of(0x3F800000u | (mv << 16)), sexp[k] + de);
          if (v == 0.0f || !isfinite(v)) continue;
          const float q = fmaf(v, rs, v * rl), ieee = v / s;
          ++n2;
          if (fabsf(ieee) >= 0x1p-100f ? q != ieee : !(fabsf(q) < 0x1p-10f && fabsf(ieee) < 0x1p-10f))
            ++bad2;
        }
      }
    }
  }
  /* 3: bf16 m / 448 */
  const float H = 1.0f / 448.0f;
  const float Lo = (float)(1.0 / 448.0 - (double)H);
  for (int em = -71; em < 100; ++em) {
    for (uint32_t mm = 0; mm < 128; ++mm) {
      const float m = ldexpf(f_of(0x3F800000u | (mm << 16)), em);
      const float q = fmaf(m, H, m * Lo);
      ++n3;
      if (q != m / 448.0f) ++bad3;
    }
  }
  /* 4: fp16 m / 448, m decoded from its fields (exponent 0: f * 2^-24) */
  long long bad4 = 0, n4 = 0;
  for (uint32_t h = 1; h < 0x7C00u; ++h) {
    const uint32_t e = h >> 10, f = h & 0x3FFu;
    const float m = e == 0 ? ldexpf((float)f, -24) : ldexpf((float)(1024 + f), (int)e - 25);
    const float q = fmaf(m, H, m * Lo);
    ++n4;
    if (q != m / 448.0f) ++bad4;
  }
  /* 5: bf16 m / 6 */
  long long bad5 = 0, n5 = 0;
  const float H6 = 1.0f / 6.0f;
  const float L6 = (float)(1.0 / 6.0 - (double)H6);
  for (int em = -90; em < 100; ++em) {
    for (uint32_t mm = 0; mm < 128; ++mm) {
      const float m = ldexpf(f_of(0x3F800000u | (mm << 16)), em);
      const float q = fmaf(m, H6, m * L6);
      ++n5;
      if (q != m / 6.0f) ++bad5;
    }
  }
  printf("markstein x/r: %lld of %lld differ\n", bad1, n1);
  printf("bf16/bf16 double reciprocal: %lld of %lld differ\n", bad2, n2);
  printf("m/448 double constant: %lld of %lld differ\n", bad3, n3);
  printf("fp16 m/448 double constant: %lld of %lld differ\n", bad4, n4);
  printf("m/6 double constant: %lld of %lld differ\n", bad5, n5);
  return (bad1 || bad2 || bad3 || bad4 || bad5) ? 1 : 0;
}
