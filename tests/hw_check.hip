// hw_check.hip -- GPU check of the gfx950 instructions the epilog's fast paths
// rely on, against IEEE arithmetic or references written here from the
// format definitions (the FP8 and FP4 codes by a nearest-value search over
// the decoded code table, not the kernels' software encoders), over every
// input the kernels can give them:
//   rcp     rcp_rn(b) == 1/b for every fp32 significand, exponents [-100, 100]
//   sqrt    sqrt_rn(x) == sqrtf(x) for every fp32 x in [2^-96, 2^127]
//   fp8     v_cvt_pk_fp8_f32(q) == E4M3 search, every fp32 |q| <= 456 (a
//           quotient by a scale rounded to bf16 exceeds 448 by at most a
//           factor 1 / (1 - 2^-8), below 450; from 464 on the convert no
//           longer saturates to 448, so the kernels never give it such values)
//   fp8s    v_cvt_scalef32_pk_fp8_f32(v, 2^E) == E4M3 search of v / 2^E, every
//           bf16 v with |v / 2^E| <= 448, E in [-100, 100]
//   fp4s    v_cvt_scalef32_pk_fp4_f32(v, 2^E) == E2M1 search of v / 2^E, every
//           bf16 v with |v / 2^E| <= 6, E in [-100, 100]
//   f16     f16_lo / f16_hi (v_cvt_f32_f16) == a bit-level binary16 decode, every
//           pattern
//   fp8s16, fp4s16  the scaled converts as above, every fp16 v
//   rn16    fp32 -> fp16 ((_Float16), v_cvt_f16_f32) and fp32 -> bf16
//           (pack_bf16_rn, v_cvt_pk_bf16_f32) == round to nearest even done
//           on the bits, for every non-NaN fp32 value
//   fp4q    v_cvt_scalef32_pk_fp4_f32(q, 1.0) == the nearest E2M1 value found
//           by a search over the eight magnitudes (ties to the even code,
//           saturating at 6), every fp32 |q| <= 6.0625: the FP4 nope mode
//           converts quotients by a scale rounded to bf16, which exceed 6 by
//           at most a factor 1 / (1 - 2^-8) < 1.004
//   fp8sq, fp4sq  the scaled converts of fp32 inputs (the quotients by a
//           scale's significand that the staged quantisers convert with the
//           scale's exponent): v_cvt_scalef32_pk_{fp8,fp4}_f32(u 2^E, 2^E) ==
//           the search of u, every fp32 u in [2^-12, 456] (FP8) or
//           [2^-4, 6.0625] (FP4) and zero, every E in [-100, 100] with u 2^E
//           normal; below those ranges, where every code is +-0, inputs q with
//           |q| < 2^(E-12) (every 1021st pattern, subnormals included) give
//           +-0 with the sign of q
//   div16   div_fast(a, b, rcp_rn(b)) == a / b for every fp16 significand a
//           against every fp32 significand b (quotient in (1/2, 2); exponents
//           are a pure scaling while the quotient stays normal)
// Prints one line per check and exits with status 1 if anything differs.
// Every launch covers at most 2^28 indices and each thread checks its index
// against the count; results go to a 64-word counter buffer.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#include "kvepi_arith.h"

using namespace kvepi;

__global__ void k_rcp(uint32_t n, unsigned *bad) {
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint32_t mant = i & 0x7FFFFFu;
  const int e = (int)(i >> 23) - 100;  // exponent in [-100, 100]
  const float b = __uint_as_float((uint32_t)(e + 127) << 23 | mant);
  if (rcp_rn(b) != 1.0f / b) atomicAdd(bad, 1u);
}

__global__ void k_sqrt(uint32_t base, uint32_t n, unsigned *bad) {
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float x = __uint_as_float(base + i);
  if (sqrt_rn(x) != __builtin_sqrtf(x)) atomicAdd(bad, 1u);
}

// E4M3FN magnitude of code c in 0..126 (bias 7, 3 fraction bits; exponent
// field 0 holds the subnormals c * 2^-9; code 127 is NaN and not a value)
__device__ float e4m3_value(uint32_t c) {
  if (c < 8u) return (float)c * 0x1p-9f;
  return __uint_as_float(((c >> 3) + 120u) << 23 | (c & 7u) << 20);
}

// E4M3FN code of q by search: the largest magnitude not above |q| (binary
// search over the 127 increasing values), then the nearer of it and the next
// one, the even code on a tie, 448 above 448 (callers keep |q| <= 456, below
// the point 464 where a saturating rounding could differ); the sign bit from
// q.  The two distances are exact in fp32 (Sterbenz: the neighbours lie within
// a factor 2 of |q|, or one of them is 0).
__device__ uint32_t e4m3_by_search(float q) {
  const float a = __builtin_fabsf(q);
  uint32_t lo = 0, hi = 126;  // e4m3_value(lo) <= a
  while (lo < hi) {
    const uint32_t mid = (lo + hi + 1) >> 1;
    if (e4m3_value(mid) <= a) lo = mid; else hi = mid - 1;
  }
  uint32_t best = lo;
  if (lo < 126u) {
    const float d0 = a - e4m3_value(lo), d1 = e4m3_value(lo + 1) - a;
    if (d1 < d0 || (d1 == d0 && ((lo + 1) & 1u) == 0u)) best = lo + 1;
  }
  return best | ((__float_as_uint(q) >> 24) & 0x80u);
}

// E2M1 code of q by search: the nearest of the eight magnitudes, the even
// code on a tie, 6 above 6; the sign bit from q
__device__ uint32_t e2m1_by_search(float q) {
  const float mag[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
  const float a = __builtin_fabsf(q);
  uint32_t best = 7;
  if (a <= 6.0f) {
    float bd = __builtin_inff();
    for (uint32_t c = 0; c < 8; ++c) {
      const float dist = __builtin_fabsf(a - mag[c]);  // exact for the two nearest
      if (dist < bd || (dist == bd && (c & 1u) == 0u)) {
        bd = dist;
        best = c;
      }
    }
  }
  return best | ((__float_as_uint(q) >> 28) & 0x8u);
}

__global__ void k_fp8(uint32_t base, uint32_t n, unsigned *bad) {
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float q = __uint_as_float(base + i);
  const uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q, -q, 0, false);
  if ((w & 0xFFu) != e4m3_by_search(q) || ((w >> 8) & 0xFFu) != e4m3_by_search(-q))
    atomicAdd(bad, 1u);
}

typedef short s16x2_t __attribute__((ext_vector_type(2)));

// binary16 from its definition: sign, 5-bit exponent (bias 15), 10-bit
// fraction; exponent 0: f * 2^-24; exponent 31: infinity or NaN
__device__ float f16_ref(uint32_t h) {
  const uint32_t e = (h >> 10) & 0x1Fu, f = h & 0x3FFu;
  float mag;
  if (e == 0)
    mag = (float)f * 0x1p-24f;
  else if (e == 31)
    mag = f == 0 ? __builtin_inff() : __builtin_nanf("");
  else
    mag = __uint_as_float((e + 112u) << 23 | f << 13);
  return (h & 0x8000u) ? -mag : mag;
}

__global__ void k_f16(uint32_t n, unsigned *bad) {
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint32_t w = i | ((i ^ 0x5A5Au) << 16);
  const float lo = f16_lo(w), hi = f16_hi(w);
  const float rl = f16_ref(i), rh = f16_ref(i ^ 0x5A5Au);
  const bool ok_lo = (lo != lo && rl != rl) || __float_as_uint(lo) == __float_as_uint(rl);
  const bool ok_hi = (hi != hi && rh != rh) || __float_as_uint(hi) == __float_as_uint(rh);
  if (!ok_lo || !ok_hi) atomicAdd(bad, 1u);
}

// round to nearest even on the bits: binary16 (overflow to infinity from
// 65520; below 2^-14 the subnormal count f * 2^24, exact, rounded) and bfloat16
__device__ uint32_t f16_rn_ref(uint32_t u) {
  const uint32_t sign = (u >> 16) & 0x8000u, a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a >= 0x477FF000u) {
    code = 0x7C00u;
  } else if (a >= 0x38800000u) {
    const uint32_t r = a + 0xFFFu + ((a >> 13) & 1u);
    code = (r >> 13) - (112u << 10);
  } else {
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 0x1p24f);
  }
  return sign | code;
}

__global__ void k_rn16(uint32_t base, uint32_t n, unsigned *bad) {
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint32_t u = base + i;
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return;  // NaN
  const float f = __uint_as_float(u);
  const _Float16 h = (_Float16)f;
  const uint32_t got16 = __builtin_bit_cast(unsigned short, h);
  const uint32_t gotb = pack_bf16_rn(f, 0.0f) & 0xFFFFu;
  const uint32_t wantb = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  if (got16 != f16_rn_ref(u) || gotb != wantb) atomicAdd(bad, 1u);
}

// one fp32 divisor significand per thread, every fp16 numerator significand
__global__ void k_div16(uint32_t n, unsigned *bad) {
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float b = __uint_as_float(0x3F800000u | i);
  const float y = rcp_rn(b);
  unsigned nb = 0;
  for (uint32_t m = 0; m < 1024; ++m) {
    const float a = __uint_as_float(0x3F800000u | (m << 13));
    if (div_fast(a, b, y) != a / b) ++nb;
  }
  if (nb) atomicAdd(bad, nb);
}

__global__ void k_fp4q(uint32_t base, uint32_t n, unsigned *bad) {
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float q = __uint_as_float(base + i);
  const uint32_t got = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, q, -q, 1.0f, 0) & 0xFFu;
  if (got != (e2m1_by_search(q) | (e2m1_by_search(-q) << 4))) atomicAdd(bad, 1u);
}

// index = (E + 100) * 65536 + bf16 (or fp16) bits
__global__ void k_scaled(uint32_t n, int fp4, int f16, unsigned *bad, unsigned *count) {
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int E = (int)(i >> 16) - 100;
  const float v = f16 ? f16_lo(i & 0xFFFFu) : __uint_as_float((i & 0xFFFFu) << 16);
  const float f = exp2_neg(E);
  const float q = v * f;  // exact: a power-of-two scaling of a bf16 value
  const float lim = fp4 ? 6.0f : 448.0f;
  if (!(__builtin_fabsf(q) <= lim)) return;  // also skips NaN
  const float sc = __uint_as_float((uint32_t)(E + 127) << 23);
  uint32_t got, want;
  if (fp4) {
    got = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v, -v, sc, 0) & 0xFFu;
    want = e2m1_by_search(q) | (e2m1_by_search(-q) << 4);
  } else {
    s16x2_t w = {0, 0};
    w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, v, -v, sc, false);
    got = (uint32_t)(uint16_t)w[0];
    want = e4m3_by_search(q) | (e4m3_by_search(-q) << 8);
  }
  atomicAdd(count, 1u);
  if (got != want) atomicAdd(bad, 1u);
}

// index i: u = bits base + i; q = u 2^E (skipped where not normal)
__global__ void k_scaledq(uint32_t base, uint32_t n, int E, int fp4, unsigned *bad,
                          unsigned long long *count) {
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  bool checked = false;
  if (i < n) {
    const float u = __uint_as_float(base + i);
    const float q = u * __uint_as_float((uint32_t)(E + 127) << 23);  // exact when normal
    if (u == 0.0f || __builtin_fabsf(q) >= 0x1p-126f) {
      const float sc = __uint_as_float((uint32_t)(E + 127) << 23);
      uint32_t got, want;
      if (fp4) {
        got = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, q, -q, sc, 0) & 0xFFu;
        want = e2m1_by_search(u) | (e2m1_by_search(-u) << 4);
      } else {
        s16x2_t w = {0, 0};
        w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, q, -q, sc, false);
        got = (uint32_t)(uint16_t)w[0];
        want = e4m3_by_search(u) | (e4m3_by_search(-u) << 8);
      }
      checked = true;
      if (got != want) atomicAdd(bad, 1u);
    }
  }
  const uint64_t b = __builtin_amdgcn_ballot_w64(checked);
  if ((threadIdx.x & 63) == 0 && b != 0)
    atomicAdd(count, (unsigned long long)__builtin_popcountll(b));
}

// tiny inputs: q bits = 1021 i below 2^(E-12); codes +-0 with q's sign
__global__ void k_scaledtiny(uint32_t n, int E, int fp4, unsigned *bad,
                             unsigned long long *count) {
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  const uint32_t lim = (uint32_t)(E - 12 + 127) << 23;
  bool checked = false;
  if (i < n && (uint64_t)i * 1021u < lim) {
    const float q = __uint_as_float(i * 1021u);
    const float sc = __uint_as_float((uint32_t)(E + 127) << 23);
    uint32_t got, want;
    if (fp4) {
      got = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, q, -q, sc, 0) & 0xFFu;
      want = 0x80u;
    } else {
      s16x2_t w = {0, 0};
      w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, q, -q, sc, false);
      got = (uint32_t)(uint16_t)w[0];
      want = 0x8000u;
    }
    checked = true;
    if (got != want) atomicAdd(bad, 1u);
  }
  const uint64_t b = __builtin_amdgcn_ballot_w64(checked);
  if ((threadIdx.x & 63) == 0 && b != 0)
    atomicAdd(count, (unsigned long long)__builtin_popcountll(b));
}

static void launch_scaledq(uint32_t lo, uint32_t hi, int fp4, unsigned *bad,
                           unsigned long long *count) {
  for (int E = -100; E <= 100; ++E) {
    hipLaunchKernelGGL(k_scaledq, dim3(1), dim3(64), 0, 0, 0u, 1u, E, fp4, bad, count);  // zero
    for (uint64_t b = lo; b <= hi; b += (1ull << 28)) {
      const uint32_t n = (uint32_t)((hi + 1 - b) < (1ull << 28) ? (hi + 1 - b) : (1ull << 28));
      hipLaunchKernelGGL(k_scaledq, dim3((n + 255) / 256), dim3(256), 0, 0, (uint32_t)b, n, E,
                         fp4, bad, count);
    }
    const uint32_t nt = (uint32_t)((((uint64_t)(E - 12 + 127) << 23) + 1020) / 1021);
    hipLaunchKernelGGL(k_scaledtiny, dim3((nt + 255) / 256), dim3(256), 0, 0, nt, E, fp4, bad,
                       count + 1);
  }
}

static void launch_range(void (*fn)(uint32_t, uint32_t, unsigned *), uint64_t lo, uint64_t hi,
                         unsigned *bad) {
  for (uint64_t b = lo; b <= hi; b += (1ull << 28)) {
    const uint32_t n = (uint32_t)((hi + 1 - b) < (1ull << 28) ? (hi + 1 - b) : (1ull << 28));
    hipLaunchKernelGGL(fn, dim3((n + 255) / 256), dim3(256), 0, 0, (uint32_t)b, n, bad);
  }
}

int main() {
  unsigned *d = nullptr;
  if (hipMalloc(&d, 64 * sizeof(unsigned)) != hipSuccess) return 2;
  (void)hipMemset(d, 0, 64 * sizeof(unsigned));
  const uint32_t n_rcp = 201u << 23;
  hipLaunchKernelGGL(k_rcp, dim3((n_rcp + 255) / 256), dim3(256), 0, 0, n_rcp, d + 0);
  launch_range(k_sqrt, 0x0F800000u, 0x7F000000u, d + 1);      // [2^-96, 2^127]
  launch_range(k_fp8, 0x00000000u, 0x43E40000u, d + 2);       // [0, 456]
  const uint32_t n_sc = 201u << 16;
  hipLaunchKernelGGL(k_scaled, dim3((n_sc + 255) / 256), dim3(256), 0, 0, n_sc, 0, 0, d + 3, d + 4);
  hipLaunchKernelGGL(k_scaled, dim3((n_sc + 255) / 256), dim3(256), 0, 0, n_sc, 1, 0, d + 5, d + 6);
  hipLaunchKernelGGL(k_f16, dim3(65536 / 256), dim3(256), 0, 0, 65536u, d + 7);
  hipLaunchKernelGGL(k_scaled, dim3((n_sc + 255) / 256), dim3(256), 0, 0, n_sc, 0, 1, d + 8, d + 9);
  hipLaunchKernelGGL(k_scaled, dim3((n_sc + 255) / 256), dim3(256), 0, 0, n_sc, 1, 1, d + 10,
                     d + 11);
  for (uint64_t b = 0; b < (1ull << 32); b += (1ull << 28))
    hipLaunchKernelGGL(k_rn16, dim3((1u << 28) / 256), dim3(256), 0, 0, (uint32_t)b, 1u << 28,
                       d + 13);
  launch_range(k_fp4q, 0x00000000u, 0x40C20000u, d + 14);     // [0, 6.0625]
  unsigned long long *dc = nullptr;  // checks counted by k_scaledq / k_scaledtiny
  if (hipMalloc(&dc, 4 * sizeof(unsigned long long)) != hipSuccess) return 2;
  (void)hipMemset(dc, 0, 4 * sizeof(unsigned long long));
  launch_scaledq(0x39800000u, 0x43E40000u, 0, d + 15, dc + 0);  // [2^-12, 456]
  launch_scaledq(0x3D800000u, 0x40C20000u, 1, d + 16, dc + 2);  // [2^-4, 6.0625]
  const uint32_t n_div = 1u << 23;
  hipLaunchKernelGGL(k_div16, dim3(n_div / 256), dim3(256), 0, 0, n_div, d + 12);
  const hipError_t e = hipDeviceSynchronize();
  unsigned h[17] = {0};
  unsigned long long hc[4] = {0, 0, 0, 0};
  (void)hipMemcpy(h, d, sizeof(h), hipMemcpyDeviceToHost);
  (void)hipMemcpy(hc, dc, sizeof(hc), hipMemcpyDeviceToHost);
  (void)hipFree(d);
  (void)hipFree(dc);
  if (e != hipSuccess) {
    printf("hip error %d\n", (int)e);
    return 2;
  }
  printf("rcp: %u mismatches of %u\n", h[0], n_rcp);
  printf("sqrt: %u mismatches of %u\n", h[1], 0x7F000000u - 0x0F800000u + 1u);
  printf("fp8: %u mismatches of %u\n", h[2], 0x43E40000u + 1u);
  printf("fp8s: %u mismatches of %u\n", h[3], h[4]);
  printf("fp4s: %u mismatches of %u\n", h[5], h[6]);
  printf("f16: %u mismatches of %u\n", h[7], 65536u);
  printf("fp8s16: %u mismatches of %u\n", h[8], h[9]);
  printf("fp4s16: %u mismatches of %u\n", h[10], h[11]);
  printf("div16: %u mismatches of %llu\n", h[12], 1024ull << 23);
  printf("rn16: %u mismatches of %llu\n", h[13], 1ull << 32);
  printf("fp4q: %u mismatches of %u\n", h[14], 0x40C20000u + 1u);
  printf("fp8sq: %u mismatches of %llu (+ %llu tiny)\n", h[15], hc[0], hc[1]);
  printf("fp4sq: %u mismatches of %llu (+ %llu tiny)\n", h[16], hc[2], hc[3]);
  const bool none_checked = hc[0] == 0 || hc[1] == 0 || hc[2] == 0 || hc[3] == 0;
  return (h[0] | h[1] | h[2] | h[3] | h[5] | h[7] | h[8] | h[10] | h[12] | h[13] | h[14] |
          h[15] | h[16]) || none_checked ? 1 : 0;
}
