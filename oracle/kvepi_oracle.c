/*
 * kvepi_oracle.c -- plain CPU oracle of the fused KV-cache write epilog.
 *
 * TEST INFRASTRUCTURE ONLY (tests, smoke check and the benchmark's CPU
 * baseline leg).  It shares no code with the HIP path.  Every function says
 * which passage it follows; the page titles are those of the vendor operator
 * documentation pages this method comes from.
 *
 * Build: gcc -O2 -std=c99 -ffp-contract=off -fno-fast-math -fPIC -shared.
 * All floating point is IEEE binary32 evaluated in source order (x86-64 SSE,
 * no excess precision, no contraction); binary64 is used only where a value
 * is exact in it (comparisons against fmax*2^E, scaled code search).
 *
 * Parity unpinned: the codes of quantMode 0, of quantMode 2's FP4 nope
 * segment and of the indexer fp8 mode divide each value by the scale as it
 * is stored (bf16 in quantMode 0 and 2, fp32 in the fp8 mode), not by the
 * unrounded amax / FP_MAX.  The pages print no example that tells the two
 * apart; the tests pin this choice only where the two agree (power-of-two
 * scales) and otherwise check the reading's own hand-worked codes.
 */
#include "kvepi_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ======================================================================== */
/* bf16                                                                      */
/* ======================================================================== */

float kvo_bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* IEEE binary16 ("indexer_quant_cache" 接口功能: the indexer also takes
 * float16 activations), decoded from its definition: sign, 5-bit exponent
 * with bias 15, 10-bit fraction; exponent 0 holds the subnormals f * 2^-24,
 * exponent 31 the infinities and NaNs.  Every value is exact in binary32. */
float kvo_fp16_to_f32(uint16_t h) {
  const int sign = h >> 15, e = (h >> 10) & 0x1F, f = h & 0x3FF;
  float mag;
  if (e == 0)
    mag = ldexpf((float)f, -24);
  else if (e == 31)
    mag = f == 0 ? INFINITY : NAN;
  else
    mag = ldexpf((float)(1024 + f), e - 25);
  return sign ? -mag : mag;
}

/* Round a binary32 value to binary16, to nearest with ties to the even
 * significand, overflowing to infinity from 65520 (the midpoint between the
 * largest finite value 65504 and 2^16).  Written from the definition: the
 * two binary16 neighbours of |f| are built from its binade (or the
 * subnormal step 2^-24), compared exactly in binary64. */
uint16_t kvo_f32_to_fp16(float f) {
  if (isnan(f)) return 0x7E00u;
  const uint16_t sign = signbit(f) ? 0x8000u : 0u;
  const double a = fabs((double)f);
  if (a >= 65520.0) return (uint16_t)(sign | 0x7C00u);
  uint16_t lo;
  if (a < ldexp(1.0, -14)) {
    lo = (uint16_t)floor(a / ldexp(1.0, -24)); /* subnormal count */
  } else {
    int e;
    frexp(a, &e); /* a = m * 2^e, m in [0.5, 1) */
    e -= 1;       /* a in [2^e, 2^(e+1)) */
    const double step = ldexp(1.0, e - 10);
    const int k = (int)floor(a / step); /* 1024 .. 2047 */
    lo = (uint16_t)(((e + 15) << 10) | (k - 1024));
  }
  const uint16_t hi = (uint16_t)(lo + 1u); /* next magnitude (0x7C00 = inf) */
  const double dlo = fabs((double)kvo_fp16_to_f32(lo));
  const double dhi = hi == 0x7C00u ? 65536.0 : fabs((double)kvo_fp16_to_f32(hi));
  const double elo = a - dlo, ehi = dhi - a;
  uint16_t r;
  if (elo < ehi)
    r = lo;
  else if (ehi < elo)
    r = hi;
  else
    r = (lo & 1u) ? hi : lo;
  return (uint16_t)(sign | r);
}

static uint32_t f32_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

/* Round a binary32 value to bfloat16, to nearest with ties to the even
 * significand.  Written from the definition: take the two bf16 neighbours of
 * f (truncated towards zero, and one bf16 ulp further from zero), pick the
 * nearer one, exactly compared in binary64, and the even one on a tie. */
uint16_t kvo_f32_to_bf16(float f) {
  uint32_t u = f32_bits(f);
  if (isnan(f)) return (uint16_t)((u >> 16) | 0x0040u); /* quiet NaN */
  if (isinf(f)) return (uint16_t)(u >> 16);
  uint16_t lo = (uint16_t)(u >> 16);     /* towards zero */
  uint16_t hi = (uint16_t)(lo + 1u);     /* away from zero (may become inf) */
  double dlo = (double)kvo_bf16_to_f32(lo);
  double dhi = (double)kvo_bf16_to_f32(hi);
  double df = (double)f;
  double elo = fabs(df - dlo);
  double ehi = fabs(dhi - df);
  if (isinf(dhi)) {
    /* hi would be the overflow: the rounding boundary is the midpoint
     * between the largest finite bf16 and 2^128. */
    double mid = dlo + (ldexp(1.0, 128) * (dlo < 0 ? -1.0 : 1.0) - dlo) / 2.0;
    if (fabs(df) < fabs(mid)) return lo;
    if (fabs(df) > fabs(mid)) return hi;
    return (lo & 1u) ? hi : lo;
  }
  if (elo < ehi) return lo;
  if (ehi < elo) return hi;
  return (lo & 1u) ? hi : lo;
}

/* ======================================================================== */
/* FP8 E4M3FN and FP4 E2M1 encoders                                          */
/* ======================================================================== */

/* Round-half-even of a binary64 value that is exact (the callers only pass
 * v * 2^k of a binary32 v).  nearbyint follows the default to-nearest-even
 * rounding mode. */
static double rne(double a) { return nearbyint(a); }

/* E4M3FN (OCP 8-bit floating point): sign, 4 exponent bits with bias 7, 3
 * mantissa bits; subnormals m * 2^-9; no infinities; S.1111.111 is NaN so the
 * largest finite magnitude is 1.75 * 2^8 = 448.  Values are rounded to the
 * nearest representable magnitude, ties to the even code, and magnitudes
 * beyond 448 saturate to 448.  The sign of zero is kept.
 *
 * This is the round() of "aclnnKvCompressEpilog" 计算公式 (q_i =
 * round(x_i / scale_g)) with the FP8 format named by "aclnnKvRmsNormRopeCache"
 * 约束说明 (FLOAT8E4M3FN); round-half-even is the CAST_RINT of the
 * "aclnnDequantRopeQuantKvcache" kernel walkthrough. */
uint8_t kvo_enc_e4m3(float v) {
  uint8_t sign = signbit(v) ? 0x80 : 0x00;
  /* A NaN quotient (inf / inf, when an infinite RMSNorm output meets an
   * infinite bf16 scale) gets the format's positive NaN code 0x7F: the sign
   * of a NaN produced by an invalid operation differs between processors,
   * so it carries no information. */
  if (isnan(v)) return 0x7F;
  double a = fabs((double)v);
  if (a > 448.0) return (uint8_t)(sign | 0x7E);
  if (a < ldexp(1.0, -6)) {
    /* subnormal range: magnitude = k * 2^-9, k = 0..8 (k == 8 is the
     * smallest normal 2^-6, whose code is also 8) */
    int k = (int)rne(a * 512.0);
    return (uint8_t)(sign | k);
  }
  int e;
  double m = frexp(a, &e); /* a = m * 2^e, m in [0.5, 1) */
  e -= 1;                  /* a = (2m) * 2^e, 2m in [1, 2) */
  double frac = 2.0 * m - 1.0;
  int mm = (int)rne(frac * 8.0);
  if (mm == 8) {
    mm = 0;
    e += 1;
  }
  if (e > 8 || (e == 8 && mm == 7)) return (uint8_t)(sign | 0x7E);
  return (uint8_t)(sign | ((e + 7) << 3) | mm);
}

/* E2M1 (OCP MX FP4): sign, 2 exponent bits with bias 1, 1 mantissa bit;
 * magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}.  Nearest, ties to the even code,
 * saturating at 6 ("aclnnKvCompressEpilog" 计算公式 FLOAT4_E2M1(x / scale);
 * "indexer_quant_cache" 接口功能 MX-FP4).  Returns the 4-bit code. */
uint8_t kvo_enc_e2m1(float v) {
  /* E2M1 has no NaN: a NaN takes one canonical code, 0x7 (+6), whatever its
   * sign bit (the sign of a NaN made by an invalid operation is
   * processor-dependent) */
  if (isnan(v)) return 0x7;
  uint8_t sign = signbit(v) ? 0x8 : 0x0;
  double a = fabs((double)v);
  if (a > 6.0) return (uint8_t)(sign | 0x7);
  if (a < 1.0) {
    int k = (int)rne(a * 2.0); /* 0, 0.5 or (k == 2) the smallest normal 1.0 */
    return (uint8_t)(sign | k);
  }
  int e;
  double m = frexp(a, &e);
  e -= 1; /* a = (2m) * 2^e, e in {0, 1, 2} */
  double frac = 2.0 * m - 1.0;
  int mm = (int)rne(frac * 2.0);
  if (mm == 2) {
    mm = 0;
    e += 1;
  }
  if (e > 2) return (uint8_t)(sign | 0x7);
  return (uint8_t)(sign | ((e + 1) << 1) | mm);
}

/* e8m0 scale exponent: the smallest integer E with amax <= fmax * 2^E, i.e.
 * the scale amax / fmax rounded up to a power of two ("aclnnKvCompressEpilog"
 * 计算公式, quantMode=1: the e8m0 scale is rounded up to a power of two).
 * Clamped to the e8m0 range [-127, 127] (byte E + 127; 255 is NaN and never
 * produced).  amax == 0 gives -127. */
int kvo_e8m0_exponent(float amax, float fmax) {
  if (!(amax > 0.0f)) return -127;
  if (isinf(amax)) return 127;
  double a = (double)amax, f = (double)fmax;
  int E;
  frexp(a / f, &E); /* a/f in [2^(E-1), 2^E) up to binary64 rounding */
  /* settle E with exact binary64 comparisons (f * 2^E is exact) */
  while (E > -127 && ldexp(f, E - 1) >= a) E--;
  while (E < 127 && ldexp(f, E) < a) E++;
  if (E < -127) E = -127;
  if (E > 127) E = 127;
  return E;
}

void kvo_enc_e4m3_batch(const float *v, uint8_t *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = kvo_enc_e4m3(v[i]);
}
void kvo_enc_e2m1_batch(const float *v, uint8_t *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = kvo_enc_e2m1(v[i]);
}
void kvo_f32_to_bf16_batch(const float *v, uint16_t *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = kvo_f32_to_bf16(v[i]);
}
void kvo_e8m0_exponent_batch(const float *amax, float fmax, int32_t *out,
                             int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = kvo_e8m0_exponent(amax[i], fmax);
}

/* ======================================================================== */
/* RMSNorm and RoPE ("aclnnKvRmsNormRopeCache", 计算公式)                    */
/* ======================================================================== */

/* Balanced pairwise sum of v[0..n), n a power of two. */
static float tree_sum(const float *v, int64_t n) {
  if (n == 1) return v[0];
  return tree_sum(v, n / 2) + tree_sum(v + n / 2, n / 2);
}

float kvo_sumsq_tree(const uint16_t *x, int64_t n) {
  int64_t p = 1;
  while (p < n) p <<= 1;
  float *sq = (float *)calloc((size_t)p, sizeof(float));
  for (int64_t i = 0; i < n; ++i) {
    float xi = kvo_bf16_to_f32(x[i]);
    sq[i] = xi * xi; /* square_x = x * x, one fp32 rounding (exact when |x| >= 2^-67) */
  }
  float ss = tree_sum(sq, p);
  free(sq);
  return ss;
}

/* (2) rmsNorm: square_x = x*x; mean_square_x = mean(square_x);
 * rms = sqrt(mean_square_x + epsilon); y = (x / rms) * gamma, written in
 * binary32 and rounded once more to the bf16 output. */
void kvo_rmsnorm_row(const uint16_t *x, const uint16_t *gamma, int64_t n,
                     float eps, uint16_t *y) {
  float ss = kvo_sumsq_tree(x, n);
  float mean_sq = ss / (float)n;
  float rms = sqrtf(mean_sq + eps);
  for (int64_t i = 0; i < n; ++i) {
    float xi = kvo_bf16_to_f32(x[i]);
    float t = xi / rms;
    float u = t * kvo_bf16_to_f32(gamma[i]);
    y[i] = kvo_f32_to_bf16(u);
  }
}

/* (1) interleaveRope on the 64 rope columns: x1 = x[0::2], x2 = x[1::2];
 * y = cat(x1, x2) * cos + cat(-x2, x1) * sin.  The output is half-split:
 * y[j] = x1[j]*cos[j] - x2[j]*sin[j], y[32+j] = x2[j]*cos[32+j] +
 * x1[j]*sin[32+j]. */
void kvo_rope_row_n(const uint16_t *x, const uint16_t *cos, const uint16_t *sin, int64_t n,
                    uint16_t *y) {
  const int64_t h = n / 2;
  for (int64_t j = 0; j < h; ++j) {
    float x1 = kvo_bf16_to_f32(x[2 * j]);
    float x2 = kvo_bf16_to_f32(x[2 * j + 1]);
    float c0 = kvo_bf16_to_f32(cos[j]), s0 = kvo_bf16_to_f32(sin[j]);
    float c1 = kvo_bf16_to_f32(cos[h + j]), s1 = kvo_bf16_to_f32(sin[h + j]);
    float p1 = x1 * c0;
    float p2 = (-x2) * s0;
    y[j] = kvo_f32_to_bf16(p1 + p2);
    float p3 = x2 * c1;
    float p4 = x1 * s1;
    y[h + j] = kvo_f32_to_bf16(p3 + p4);
  }
}

void kvo_rope_row(const uint16_t *x, const uint16_t *cos, const uint16_t *sin,
                  uint16_t *y) {
  kvo_rope_row_n(x, cos, sin, 64, y);
}

/* ======================================================================== */
/* Row geometry ("aclnnKvCompressEpilog" 约束说明; "indexer_quant_cache" 约束) */
/* ======================================================================== */

int kvo_row_bytes(int mode, int64_t d, int32_t group_size, int64_t *concat_col,
                  int64_t *kv_cache_col, int64_t *scale_col) {
  int64_t cc = 0, kc = 0, sc = 0;
  if (mode == KVO_MODE_FP8_BF16SCALE || mode == KVO_MODE_FP8_E8M0) {
    if (group_size != 64 || d % 64 != 0 || d <= 64 || d > 8192) return -1;
    int64_t nope = d - 64;
    int64_t groups = (nope + 63) / 64;
    int64_t sbytes = mode == KVO_MODE_FP8_BF16SCALE ? 2 : 1;
    cc = nope + 128 + groups * sbytes;
    kc = mode == KVO_MODE_FP8_E8M0 ? cc : (cc + 31) / 32 * 32;
    sc = groups;
  } else if (mode == KVO_MODE_MXFP4) {
    if (group_size != 32 || d % 32 != 0 || d < 32 || d > 8192) return -1;
    cc = (d + 1) / 2;
    kc = cc;
    sc = (d + 31) / 32;
  } else if (mode == KVO_MODE_MXFP8) {
    if (group_size != 32 || d % 32 != 0 || d < 32 || d > 8192) return -1;
    cc = d;
    kc = d;
    sc = (d + 31) / 32;
  } else if (mode == KVO_MODE_FP8_ROW) {
    /* the whole row is one group: group_size 0 (or d) */
    if ((group_size != 0 && group_size != d) || d % 32 != 0 || d < 32 || d > 8192) return -1;
    cc = d;
    kc = d;
    sc = 1; /* one FLOAT per row */
  } else if (mode == KVO_MODE_FP4_NOPE) {
    /* quantMode=2: concatCol = 64 + (d-64)/2 + ((d-64)/G)*2, aligned to
     * 32 bytes; G in {16, 32, 64} dividing d-64 */
    if (d % 64 != 0 || d <= 64 || d > 8192) return -1;
    if (group_size != 16 && group_size != 32 && group_size != 64) return -1;
    if ((d - 64) % group_size != 0) return -1;
    cc = 64 + (d - 64) / 2 + ((d - 64) / group_size) * 2;
    kc = (cc + 31) / 32 * 32;
    sc = (d - 64) / group_size;
  } else if (mode == KVO_MODE_BF16_SPLIT) {
    if (d % 64 != 0 || d <= 64 || d > 8192) return -1;
    cc = d - 64; /* ckv elements per row */
    kc = d - 64;
    sc = 64; /* k elements per row */
  } else {
    return -1;
  }
  if (concat_col) *concat_col = cc;
  if (kv_cache_col) *kv_cache_col = kc;
  if (scale_col) *scale_col = sc;
  return 0;
}

/* ======================================================================== */
/* Quantisation of one prepared row                                          */
/* ======================================================================== */

static void put_u16le(uint8_t *p, uint16_t v) {
  p[0] = (uint8_t)(v & 0xFF);
  p[1] = (uint8_t)(v >> 8);
}

/* "aclnnKvCompressEpilog" 计算公式 scenes 1 and 2, with the row layout of
 * 约束说明 (nope codes | rope at 16 bit | one scale per group | zero padding
 * to kvCacheCol), and "indexer_quant_cache" mxfp4 (codes of the whole row,
 * two per byte, scales to cache_scale). */
/* value i of an input row: bf16, or (indexer modes) fp16 bits */
static float in_f32(const uint16_t *v, int64_t i, int fp16) {
  return fp16 ? kvo_fp16_to_f32(v[i]) : kvo_bf16_to_f32(v[i]);
}

int kvo_quant_row_x(int mode, const uint16_t *v, int64_t d, int32_t group_size, int x_fp16,
                    uint8_t *out, uint8_t *scale_out) {
  int64_t cc, kc, sc;
  if (kvo_row_bytes(mode, d, group_size, &cc, &kc, &sc) != 0) return -1;
  const int fp16 = x_fp16 != 0;
  if (fp16 && mode != KVO_MODE_MXFP4 && mode != KVO_MODE_MXFP8 && mode != KVO_MODE_FP8_ROW)
    return -1; /* fp16 rows only in the indexer modes */
  if (mode == KVO_MODE_FP8_BF16SCALE || mode == KVO_MODE_FP8_E8M0) {
    int64_t nope = d - 64;
    memset(out, 0, (size_t)kc);
    for (int64_t g = 0; g < sc; ++g) {
      int64_t i0 = g * 64, i1 = i0 + 64 < nope ? i0 + 64 : nope;
      float amax = 0.0f;
      for (int64_t i = i0; i < i1; ++i) {
        float a = fabsf(in_f32(v, i, fp16));
        if (a > amax) amax = a;
      }
      float s_use;
      if (mode == KVO_MODE_FP8_BF16SCALE) {
        float s32 = amax / 448.0f; /* scale_g = max|x_g| / FP8_MAX */
        uint16_t sb = kvo_f32_to_bf16(s32);
        put_u16le(out + nope + 128 + 2 * g, sb);
        s_use = kvo_bf16_to_f32(sb); /* divide by the scale as stored */
      } else {
        int E = kvo_e8m0_exponent(amax, 448.0f);
        out[nope + 128 + g] = (uint8_t)(E + 127);
        s_use = ldexpf(1.0f, E);
      }
      for (int64_t i = i0; i < i1; ++i) {
        if (s_use == 0.0f) {
          out[i] = 0x00;
        } else {
          float q = in_f32(v, i, fp16) / s_use;
          out[i] = kvo_enc_e4m3(q);
        }
      }
    }
    for (int64_t j = 0; j < 64; ++j) put_u16le(out + nope + 2 * j, v[nope + j]);
    return 0;
  }
  if (mode == KVO_MODE_FP4_NOPE) {
    /* "aclnnKvCompressEpilog" scene 3, nope segment: per group of
     * group_size values scale_g = max|x_g| / 6, stored as bf16 (2 bytes,
     * little-endian, after the codes), codes E2M1(x_i / scale_g) dividing
     * by the scale as stored, two per byte (element 2j in the low nibble);
     * an all-zero group has scale 0 and codes 0.  Bytes [0, 64) are the
     * rope segment's and are not written here. */
    if (fp16) return -1; /* x must be bf16 (约束说明) */
    const int64_t nope = d - 64;
    memset(out + 64, 0, (size_t)(kc - 64));
    for (int64_t g = 0; g < sc; ++g) {
      const int64_t i0 = g * group_size, i1 = i0 + group_size;
      float amax = 0.0f;
      for (int64_t i = i0; i < i1; ++i) {
        float a = fabsf(kvo_bf16_to_f32(v[i]));
        if (a > amax) amax = a;
      }
      const float s32 = amax / 6.0f; /* scale_g = max|x_g| / FP4_MAX */
      const uint16_t sb = kvo_f32_to_bf16(s32);
      put_u16le(out + 64 + nope / 2 + 2 * g, sb);
      const float s_use = kvo_bf16_to_f32(sb);
      for (int64_t i = i0; i < i1; ++i) {
        const uint8_t c = s_use == 0.0f ? 0x0 : kvo_enc_e2m1(kvo_bf16_to_f32(v[i]) / s_use);
        uint8_t *b = out + 64 + i / 2;
        *b = (i % 2 == 0) ? (uint8_t)((*b & 0xF0) | c) : (uint8_t)((*b & 0x0F) | (c << 4));
      }
    }
    return 0;
  }
  if (mode == KVO_MODE_MXFP4) {
    memset(out, 0, (size_t)kc);
    for (int64_t g = 0; g < sc; ++g) {
      int64_t i0 = g * 32, i1 = i0 + 32 < d ? i0 + 32 : d;
      float amax = 0.0f;
      for (int64_t i = i0; i < i1; ++i) {
        float a = fabsf(in_f32(v, i, fp16));
        if (a > amax) amax = a;
      }
      int E = kvo_e8m0_exponent(amax, 6.0f);
      scale_out[g] = (uint8_t)(E + 127);
      float s_use = ldexpf(1.0f, E);
      for (int64_t i = i0; i < i1; ++i) {
        uint8_t c = kvo_enc_e2m1(in_f32(v, i, fp16) / s_use);
        /* element 2j in the low nibble, 2j+1 in the high nibble */
        if (i % 2 == 0)
          out[i / 2] = (uint8_t)((out[i / 2] & 0xF0) | c);
        else
          out[i / 2] = (uint8_t)((out[i / 2] & 0x0F) | (c << 4));
      }
    }
    return 0;
  }
  if (mode == KVO_MODE_MXFP8) {
    /* "indexer_quant_cache" mxfp8: groups of 32, e8m0 scale, E4M3 codes */
    for (int64_t g = 0; g < sc; ++g) {
      int64_t i0 = g * 32, i1 = i0 + 32 < d ? i0 + 32 : d;
      float amax = 0.0f;
      for (int64_t i = i0; i < i1; ++i) {
        float a = fabsf(in_f32(v, i, fp16));
        if (a > amax) amax = a;
      }
      int E = kvo_e8m0_exponent(amax, 448.0f);
      scale_out[g] = (uint8_t)(E + 127);
      float s_use = ldexpf(1.0f, E);
      for (int64_t i = i0; i < i1; ++i) out[i] = kvo_enc_e4m3(in_f32(v, i, fp16) / s_use);
    }
    return 0;
  }
  if (mode == KVO_MODE_FP8_ROW) {
    /* "indexer_quant_cache" fp8: the whole row one group; the scale
     * max|x| / 448 is kept as FLOAT and the codes divide by it */
    float amax = 0.0f;
    for (int64_t i = 0; i < d; ++i) {
      float a = fabsf(in_f32(v, i, fp16));
      if (a > amax) amax = a;
    }
    float s = amax / 448.0f;
    memcpy(scale_out, &s, 4); /* little-endian fp32 */
    for (int64_t i = 0; i < d; ++i)
      out[i] = s == 0.0f ? 0x00 : kvo_enc_e4m3(in_f32(v, i, fp16) / s);
    return 0;
  }
  return -1;
}

int kvo_quant_row(int mode, const uint16_t *v, int64_t d, int32_t group_size,
                  uint8_t *out, uint8_t *scale_out) {
  return kvo_quant_row_x(mode, v, d, group_size, 0, out, scale_out);
}

/* ======================================================================== */
/* Whole epilog                                                              */
/* ======================================================================== */

static uint8_t *row_ptr(const kvo_cache *c, int64_t slot, int64_t esz) {
  int64_t blk = slot / c->block_size;
  int64_t pos = slot % c->block_size;
  return c->data + (blk * c->block_stride + pos * c->head_dim) * esz;
}

/* Cache row of token t, or -1 when the token is skipped.  Tokens are
 * batch-major (t = b * seq_len + s) in the index modes other than SLOT.
 *  SLOT:  index[t] is the token's slot ("aclnnKvCompressEpilog" 约束说明;
 *         "aclnnKvRmsNormRopeCache" index constraints, PA_BNSD/PA_NZ;
 *         "indexer_quant_cache" 约束).
 *  BATCH: index [B, S]; index[b, s] is the row inside batch b's own
 *         block_size rows ("aclnnKvRmsNormRopeCache" index constraints,
 *         Norm: values in [-1, Scache), repeats across batches allowed).
 *  BLOCK: index [B, ceil(S / block_size)]; entry c names the block (value /
 *         block_size) that takes tokens c*block_size .. of the batch, token
 *         s at row s % block_size of it ("aclnnKvRmsNormRopeCache" index
 *         constraints, PA_BLK_BNSD/PA_BLK_NZ: value / BlockSize distinct).
 *  BATCH_START: index [B]; token s of batch b goes to row index[b] + s of
 *         batch b's rows (the blog on aclnnDequantRopeQuantKvcache, cache
 *         modes: the contiguous mode's offset).
 * -1, and any value that would leave the cache, skip the token. */
int64_t kvo_token_slot(int index_mode, const int32_t *index, int64_t t, int64_t seq_len,
                       int64_t block_num, int64_t block_size) {
  const int64_t num_slots = block_num * block_size;
  if (index_mode == KVO_INDEX_SLOT) {
    int64_t v = index[t];
    return (v >= 0 && v < num_slots) ? v : -1;
  }
  if (seq_len <= 0) return -1;
  const int64_t b = t / seq_len, s = t % seq_len;
  if (index_mode == KVO_INDEX_BATCH) {
    int64_t v = index[t];
    if (v < 0 || v >= block_size || b >= block_num) return -1;
    return b * block_size + v;
  }
  if (index_mode == KVO_INDEX_BLOCK) {
    const int64_t nc = (seq_len + block_size - 1) / block_size;
    int64_t v = index[b * nc + s / block_size];
    if (v < 0 || v >= num_slots) return -1;
    return (v / block_size) * block_size + s % block_size;
  }
  if (index_mode == KVO_INDEX_BATCH_START) {
    int64_t v = index[b];
    if (v < 0 || v + s >= block_size || b >= block_num) return -1;
    return b * block_size + v + s;
  }
  return -1;
}

int kvo_epilog(int mode, int64_t T, int64_t d, const uint16_t *x,
               int64_t x_row_stride, const uint16_t *gamma,
               const uint16_t *cos, const uint16_t *sin, float eps,
               const int32_t *slot_mapping, int32_t group_size,
               const kvo_cache *cache, const kvo_cache *aux) {
  return kvo_epilog_ex(mode, T, d, x, x_row_stride, 0, gamma, cos, sin, eps, slot_mapping,
                       KVO_INDEX_SLOT, 0, 64, group_size, cache, aux);
}

int kvo_epilog_ex(int mode, int64_t T, int64_t d, const uint16_t *x, int64_t x_row_stride,
                  int x_fp16, const uint16_t *gamma, const uint16_t *cos, const uint16_t *sin,
                  float eps, const int32_t *index, int index_mode, int64_t seq_len,
                  int rope_dim, int32_t group_size, const kvo_cache *cache,
                  const kvo_cache *aux) {
  int64_t cc, kc, sc;
  /* the rope segment: the last 64 columns ("aclnnKvCompressEpilog" 接口功能),
   * or in the bf16 split mode any even Dk with Dk + Dv = d
   * ("aclnnKvRmsNormRopeCache", shape notes: Dk even) */
  if (mode == KVO_MODE_BF16_SPLIT) {
    if (rope_dim < 2 || rope_dim % 2 || d - rope_dim < 8 || (d - rope_dim) % 8 || d > 8192)
      return -1;
    cc = kc = d - rope_dim;
    sc = rope_dim;
  } else {
    if (rope_dim != 64) return -1;
    if (kvo_row_bytes(mode, d, group_size, &cc, &kc, &sc) != 0) return -1;
  }
  if (index_mode != KVO_INDEX_SLOT && (seq_len <= 0 || T % seq_len != 0)) return -1;
  if ((cos == NULL) != (sin == NULL)) return -1;
  const int indexer = mode == KVO_MODE_MXFP4 || mode == KVO_MODE_MXFP8 ||
                      mode == KVO_MODE_FP8_ROW;
  if (indexer && (gamma || cos)) return -1;
  if (mode == KVO_MODE_BF16_SPLIT && (!gamma || !cos)) return -1;
  if (mode == KVO_MODE_FP4_NOPE && (cos || aux)) return -1; /* rope bytes not written */
  if ((indexer || mode == KVO_MODE_BF16_SPLIT) && !aux) return -1;
  if (x_fp16 && !indexer) return -1;
  /* every row written must fit its cache row, and the rows of a block its
   * block: headDim >= kvCacheCol ("aclnnKvCompressEpilog", 约束说明;
   * "indexer_quant_cache", 约束 for cache_scale); in the split mode the ckv
   * rows hold Dv and the k rows Dk bf16 elements */
  if (!cache || cache->head_dim < kc || cache->block_stride < cache->block_size * cache->head_dim)
    return -1;
  if (aux) {
    const int64_t need = mode == KVO_MODE_FP8_ROW ? 1 : sc;
    if (aux->head_dim < need || aux->block_stride < aux->block_size * aux->head_dim ||
        aux->block_num != cache->block_num || aux->block_size != cache->block_size)
      return -1;
  }
  const int64_t dk = rope_dim;
  int64_t nope = d - dk;
  uint16_t *v = (uint16_t *)malloc((size_t)d * sizeof(uint16_t));
  uint8_t *row = (uint8_t *)malloc((size_t)kc + 64);
  uint8_t *srow = (uint8_t *)malloc((size_t)sc + 64);
  for (int64_t t = 0; t < T; ++t) {
    int64_t s = kvo_token_slot(index_mode, index, t, seq_len, cache->block_num,
                               cache->block_size);
    if (s < 0) continue; /* -1: token skipped */
    const uint16_t *xr = x + t * x_row_stride;
    if (indexer) {
      kvo_quant_row_x(mode, xr, d, group_size, x_fp16, row, srow);
      memcpy(row_ptr(cache, s, 1), row, (size_t)kc);
      if (mode == KVO_MODE_FP8_ROW)
        memcpy(row_ptr(aux, s, 4), srow, 4);
      else
        memcpy(row_ptr(aux, s, 1), srow, (size_t)sc);
      continue;
    }
    if (gamma)
      kvo_rmsnorm_row(xr, gamma, nope, eps, v);
    else
      memcpy(v, xr, (size_t)nope * sizeof(uint16_t));
    if (mode == KVO_MODE_FP4_NOPE) {
      kvo_quant_row(mode, v, d, group_size, row, NULL);
      memcpy(row_ptr(cache, s, 1) + 64, row + 64, (size_t)(kc - 64));
      continue;
    }
    if (cos)
      kvo_rope_row_n(xr + nope, cos + t * dk, sin + t * dk, dk, v + nope);
    else
      memcpy(v + nope, xr + nope, (size_t)dk * sizeof(uint16_t));
    if (mode == KVO_MODE_BF16_SPLIT) {
      uint8_t *ckv = row_ptr(cache, s, 2);
      uint8_t *k = row_ptr(aux, s, 2);
      for (int64_t i = 0; i < nope; ++i) put_u16le(ckv + 2 * i, v[i]);
      for (int64_t j = 0; j < dk; ++j) put_u16le(k + 2 * j, v[nope + j]);
      continue;
    }
    kvo_quant_row(mode, v, d, group_size, row, NULL);
    memcpy(row_ptr(cache, s, 1), row, (size_t)kc);
  }
  free(v);
  free(row);
  free(srow);
  return 0;
}

/* ======================================================================== */
/* Dequant -> RoPE -> static int8 quantisation -> KV cache (the blog on      */
/* aclnnDequantRopeQuantKvcache: 计算步骤公式 steps 1-5, 约束说明)           */
/* ======================================================================== */

static float val16(uint16_t h, int dtype) {
  return dtype == KVO_DT_FP16 ? kvo_fp16_to_f32(h) : kvo_bf16_to_f32(h);
}
static uint16_t round16(float f, int dtype) {
  return dtype == KVO_DT_FP16 ? kvo_f32_to_fp16(f) : kvo_f32_to_bf16(f);
}

/* Static int8 quantisation of one value (step 4): v / scale, plus the
 * offset when there is one, rounded half to even, saturated to [-128, 127]. */
int8_t kvo_quant_int8(float v, float scale, const float *offset) {
  float q = v / scale;
  if (offset) q = q + *offset;
  const double r = nearbyint((double)q); /* exact: q is a binary32 value */
  if (r > 127.0) return 127;
  if (r < -128.0) return -128;
  return (int8_t)r;
}

int kvo_drq(int64_t T, int nq, int nkv, int D, const void *x, int x_dtype, int64_t x_row_stride,
            const uint16_t *cos, const uint16_t *sin, int out_dtype, const float *weight_scale,
            const float *act_scale, const void *bias, int bias_dtype, const float *scale_k,
            const float *scale_v, const float *offset_k, const float *offset_v,
            const int32_t *index, int index_mode, int64_t seq_len, const kvo_cache *k_cache,
            const kvo_cache *v_cache, uint16_t *q_out, uint16_t *k_out, uint16_t *v_out) {
  if (nq < 1 || nkv < 1 || D < 2 || D % 2) return -1;
  if (out_dtype != KVO_DT_BF16 && out_dtype != KVO_DT_FP16) return -1;
  const int dequant = x_dtype == KVO_DT_INT32;
  if (!dequant && x_dtype != out_dtype) return -1; /* 约束说明 4 */
  if (dequant && !weight_scale) return -1;         /* 约束说明 5 */
  if (!dequant && (weight_scale || act_scale || bias)) return -1;
  if (index_mode != KVO_INDEX_SLOT && index_mode != KVO_INDEX_BATCH_START) return -1;
  if (index_mode != KVO_INDEX_SLOT && (seq_len <= 0 || T % seq_len != 0)) return -1;
  const int64_t H = (int64_t)(nq + 2 * nkv) * D, HK = (int64_t)nkv * D;
  float *dq = (float *)malloc((size_t)H * sizeof(float));
  float *ko = (float *)malloc((size_t)HK * sizeof(float));
  for (int64_t t = 0; t < T; ++t) {
    /* step 1: dequantX (cast, * weight_scale, * activation scale, + bias),
     * held in the output dtype like every tensor of the chain */
    for (int64_t h = 0; h < H; ++h) {
      float v;
      if (dequant) {
        v = (float)((const int32_t *)x)[t * x_row_stride + h];
        v = v * weight_scale[h];
        if (act_scale) v = v * act_scale[t];
        if (bias) {
          float b;
          if (bias_dtype == KVO_DT_FP32)
            b = ((const float *)bias)[h];
          else if (bias_dtype == KVO_DT_INT32)
            b = (float)((const int32_t *)bias)[h];
          else
            b = val16(((const uint16_t *)bias)[h], bias_dtype);
          v = v + b;
        }
        v = val16(round16(v, out_dtype), out_dtype);
      } else {
        v = val16(((const uint16_t *)x)[t * x_row_stride + h], x_dtype);
      }
      dq[h] = v;
    }
    /* steps 2-3: split into q | k | v heads; rotate-half RoPE of q and k
     * with the token's cos / sin [D] (each product exact in binary32 for
     * 16-bit operands, one rounding for the sum, then the output dtype) */
    const uint16_t *c = cos + t * D, *sn = sin + t * D;
    for (int h = 0; h < nq + nkv; ++h) {
      const float *in = dq + (int64_t)h * D;
      for (int j = 0; j < D / 2; ++j) {
        const float a = in[j], b = in[j + D / 2];
        const float y1 = a * val16(c[j], out_dtype) - b * val16(sn[j], out_dtype);
        const float y2 = b * val16(c[j + D / 2], out_dtype) + a * val16(sn[j + D / 2], out_dtype);
        const uint16_t r1 = round16(y1, out_dtype), r2 = round16(y2, out_dtype);
        if (h < nq) {
          q_out[t * nq * D + (int64_t)h * D + j] = r1;
          q_out[t * nq * D + (int64_t)h * D + j + D / 2] = r2;
        } else {
          const int64_t o = (int64_t)(h - nq) * D;
          if (k_out) {
            k_out[t * HK + o + j] = r1;
            k_out[t * HK + o + j + D / 2] = r2;
          }
          ko[o + j] = val16(r1, out_dtype);
          ko[o + j + D / 2] = val16(r2, out_dtype);
        }
      }
    }
    const float *vv = dq + (int64_t)(nq + nkv) * D;
    if (v_out)
      for (int64_t i = 0; i < HK; ++i) v_out[t * HK + i] = round16(vv[i], out_dtype);
    /* steps 4-5: static int8 quantisation of kOut and vOut, written to the
     * token's cache row (-1, or a row outside the cache, skips the write) */
    const int64_t slot = kvo_token_slot(index_mode, index, t, seq_len, k_cache->block_num,
                                        k_cache->block_size);
    if (slot < 0) continue;
    int8_t *kr = (int8_t *)(k_cache->data + (slot / k_cache->block_size) * k_cache->block_stride +
                            (slot % k_cache->block_size) * k_cache->head_dim);
    int8_t *vr = (int8_t *)(v_cache->data + (slot / v_cache->block_size) * v_cache->block_stride +
                            (slot % v_cache->block_size) * v_cache->head_dim);
    for (int64_t i = 0; i < HK; ++i) {
      kr[i] = kvo_quant_int8(ko[i], scale_k[i], offset_k ? offset_k + i : NULL);
      vr[i] = kvo_quant_int8(vv[i], scale_v[i], offset_v ? offset_v + i : NULL);
    }
  }
  free(dq);
  free(ko);
  return 0;
}

