// kvepi_arith.h -- gfx950 device arithmetic of the epilog's fast paths:
// correctly rounded division and square root from the hardware reciprocal
// and square root, the software E4M3 / E2M1 encoders of the slow paths and
// the e8m0 exponent.  Shared by the kernels (kvepi_kernels.hip) and the GPU
// check of the hardware instructions they rely on (tests/hw_check.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvepi {

// Correctly rounded a / b from rcp = RN(1 / b) with one FMA correction.
// Exact for a bf16 numerator whenever the quotient is a normal fp32 number
// and |a| >= 2^-100 (tests/fastdiv_check.c checks every bf16 significand
// against every fp32 divisor significand).  The last step is evaluated negated so that a zero
// quotient keeps the sign of a: -(-r*rcp - q0).
__device__ __forceinline__ float div_fast(float a, float b, float rcp) {
  const float q0 = a * rcp;
  const float r = __builtin_fmaf(-q0, b, a);
  return -__builtin_fmaf(-r, rcp, -q0);
}

// 1 / b correctly rounded, from the hardware reciprocal and one Newton step
// (tests/hw_check.hip compares it with IEEE division for every fp32
// significand, exponents in [-100, 100]; callers keep b in that range).
__device__ __forceinline__ float rcp_rn(float b) {
  const float y0 = __builtin_amdgcn_rcpf(b);
  const float e = __builtin_fmaf(-b, y0, 1.0f);
  return __builtin_fmaf(e, y0, y0);
}

// sqrt(x) correctly rounded for x in [2^-96, 2^127]: the hardware square
// root, within one ulp there, corrected by the signs of the residuals of its
// two neighbours (tests/hw_check.hip compares it with the library square
// root for every fp32 value of that range).
__device__ __forceinline__ float sqrt_rn(float x) {
  const float s = __builtin_amdgcn_sqrtf(x);
  const float sm = __uint_as_float(__float_as_uint(s) - 1u);
  const float sp = __uint_as_float(__float_as_uint(s) + 1u);
  const float rm = __builtin_fmaf(-sm, s, x);
  const float rp = __builtin_fmaf(-sp, s, x);
  const float r = rm <= 0.0f ? sm : s;
  return rp > 0.0f ? sp : r;
}

// The fp16 halves of a 32-bit word as fp32 (exact; v_cvt_f32_f16, which
// keeps fp16 subnormals: tests/hw_check.hip compares it with a bit-level
// decode of every pattern).
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(w & 0xFFFFu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(w >> 16));
}

// Two fp32 -> packed bf16, round to nearest even (v_cvt_pk_bf16_f32), a in
// the low half (tests/hw_check.hip compares it with a software rounding for
// every fp32 value).
__device__ __forceinline__ uint32_t pack_bf16_rn(float a, float b) {
  typedef __bf16 rn_bf16x2 __attribute__((ext_vector_type(2)));
  typedef float rn_f32x2 __attribute__((ext_vector_type(2)));
  rn_f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, rn_bf16x2));
}

// max(|a|, |b|, |c|) in one instruction (the compiler's fmaxf chain adds
// canonicalisations for inputs it cannot prove to be canonical).  With the
// IEEE mode of compute kernels, v_max3_f32 returns the larger number when an
// operand is a quiet NaN.
__device__ __forceinline__ float max3_abs(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, |%1|, |%2|, |%3|" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
// max(|a|, |b|, 0)
__device__ __forceinline__ float max2_abs0(float a, float b) {
  float r;
  asm("v_max3_f32 %0, |%1|, |%2|, 0" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
// The largest magnitude of eight values, NaN values left out (0 when all
// eight are NaN): the last step takes 0 as its third operand.  (A NaN only
// arises from 0 / 0 in RMSNorm, a zero row with eps = 0, where every value of
// the row is NaN and the scale becomes 0.)
__device__ __forceinline__ float amax8(const float (&v)[8]) {
  float m = max3_abs(v[0], v[1], v[2]);
  m = max3_abs(m, v[3], v[4]);
  m = max3_abs(m, v[5], v[6]);
  return max2_abs0(m, v[7]);
}

// E4M3FN code of q: round to nearest even, |q| > 448 saturates to 448,
// sign kept (also for zero); a NaN gives 0x7F.
__device__ __forceinline__ uint32_t enc_e4m3_sw(float q) {
  const uint32_t u = __float_as_uint(q);
  const uint32_t s = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a > 0x7F800000u) {
    return 0x7Fu;
  } else if (a > 0x43E00000u) {  // > 448
    code = 0x7Eu;
  } else if (a >= 0x3C800000u) {  // >= 2^-6: keep 3 mantissa bits, RNE
    const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
    code = (r >> 20) - (120u << 3);  // rebias exponent 127 -> 7
  } else {                          // subnormal grid k * 2^-9, k = 0..8
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  }
  return code | s;
}

// E2M1 code (4 bits) of q: nearest of {0,.5,1,1.5,2,3,4,6}, ties to the
// even code, saturating at 6; a NaN gives 0x7 (E2M1 has no NaN).
__device__ __forceinline__ uint32_t enc_e2m1_sw(float q) {
  if (q != q) return 0x7u;
  const float a = __builtin_fabsf(q);
  const uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                     (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                     (uint32_t)(a > 5.0f);
  return c | ((__float_as_uint(q) >> 28) & 0x8u);
}

// e8m0 exponent: smallest E in [-127, 127] with amax <= fmax * 2^E, for
// fmax = 1.m * 2^FE given as its exponent FE and mantissa bits FM.
template <int FE, uint32_t FM>
__device__ __forceinline__ int e8m0_exp(float amax) {
  const uint32_t u = __float_as_uint(amax);
  const int eb = (int)(u >> 23);
  if (eb == 0) return -127;   // zero or subnormal amax: below fmax * 2^-127
  if (eb == 255) return 127;  // infinite amax: the largest scale
  const int E = eb - 127 - FE + (int)((u & 0x7FFFFFu) > FM);
  return E < -127 ? -127 : (E > 127 ? 127 : E);
}

// 2^-E as an exact float, E in [-127, 127].
__device__ __forceinline__ float exp2_neg(int E) {
  return E == 127 ? __uint_as_float(0x00400000u) : __uint_as_float((uint32_t)(127 - E) << 23);
}

}  // namespace kvepi
