// kvepi_kernels.hip -- gfx950 kernels of the fused KV-cache write epilog.
//
// One kernel template covers every mode.  A token row is handled by a group
// of L lanes of one 64-lane wavefront (L = 64 for the d = 576 rows, 16 for
// the d = 128 indexer rows, so a wave carries 64/L rows at once); each lane
// owns C 16-byte chunks of 8 bf16 values, chunk index li + L*j, so every
// load instruction of a wave reads L*16 contiguous bytes of a row.
//
// Steps per row (sources cited by page title and section):
//  1. slot = slot_mapping[t]; -1 (or any value outside [0, num_slots)) skips
//     the token: nothing is read or written for it
//     ("aclnnKvCompressEpilog", 约束说明).
//  2. RMSNorm of the nope segment ("aclnnKvRmsNormRopeCache", 计算公式 (2)):
//     squares summed as a balanced pairwise tree -- within a lane over its 8
//     values, then across lanes by a DPP / ds_swizzle butterfly whose
//     pairing is exactly the tree's (fp32 addition is commutative, so both
//     lanes of a pair hold the same node), then over the chunk index j;
//     mean = sum / n, rms = sqrt(mean + eps), t = x / rms, u = t * gamma,
//     bf16 output.  All in IEEE fp32; x / rms uses the reciprocal with one
//     FMA correction (Markstein), which returns the correctly rounded
//     quotient for a bf16 numerator and a normal result -- the row falls
//     back to full division when that cannot be guaranteed.
//  3. Interleaved RoPE of the last 64 columns, half-split output
//     ("aclnnKvRmsNormRopeCache", 计算公式 (1)).
//  4. Per-group amax (DPP max over the 8 or 4 lanes of a group), the scale
//     ("aclnnKvCompressEpilog", 计算公式: amax / 448 as bf16, or the e8m0
//     power of two rounded up; "indexer_quant_cache": e8m0 over groups of
//     32 with FP4 max 6) and the codes, round-to-nearest-even with
//     saturation.
//  5. Stores of exactly kvCacheCol bytes at the slot's row; the widest store
//     the row alignment allows is used (16/8/4/2/1 bytes), so odd headDim
//     such as 323 works.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvepi_plan.h"

namespace kvepi {

struct KArgs {
  const uint16_t *x, *gamma, *cos, *sin;
  const int32_t *slots;
  uint8_t *cache, *aux;
  int64_t x_stride;            // elements
  int64_t c_pitch, c_bstride;  // bytes
  int64_t a_pitch, a_bstride;  // bytes
  uint64_t bs_magic;           // slot / block_size == (slot * magic) >> shift
  int32_t bs_shift, block_size;
  int32_t T, num_slots;
  int32_t nseg;    // values in the quantised/normalised segment (d-64, or d)
  int32_t nchunk;  // nseg / 8
  int32_t concat_col, kv_cache_col;
  int32_t c_align, a_align;
  float eps, nseg_f;
  int32_t nwaves;      // waves in the grid
  int32_t xcd_blocks;  // blocks per XCD for the XCD-major remap, 0 = off
};

// ------------------------------------------------------------------------
// bit-level helpers
// ------------------------------------------------------------------------
__device__ __forceinline__ float lo_f(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 (round to nearest even; v_cvt_pk_bf16_f32), a low.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// lane ^ 16 inside each half of the wave (ds_swizzle bit-mask mode)
__device__ __forceinline__ float swz_xor16(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
}
__device__ __forceinline__ float rdlane(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// Sum over aligned groups of G lanes; every lane of a group receives the
// balanced-tree sum of the group's values in lane order.  Steps: lane^1,
// lane^2 (quad permutes), then the half-row and row mirrors, which pair the
// same blocks as lane^4 and lane^8 once each block holds one value.
template <int G>
__device__ __forceinline__ float grp_sum(float v) {
  if constexpr (G >= 2) v = v + dpp<0xB1>(v);
  if constexpr (G >= 4) v = v + dpp<0x4E>(v);
  if constexpr (G >= 8) v = v + dpp<0x141>(v);
  if constexpr (G >= 16) v = v + dpp<0x140>(v);
  if constexpr (G >= 32) v = v + swz_xor16(v);
  if constexpr (G >= 64) v = rdlane(v, 0) + rdlane(v, 32);
  return v;
}

template <int G>
__device__ __forceinline__ float grp_max(float v) {
  if constexpr (G >= 2) v = fmaxf(v, dpp<0xB1>(v));
  if constexpr (G >= 4) v = fmaxf(v, dpp<0x4E>(v));
  if constexpr (G >= 8) v = fmaxf(v, dpp<0x141>(v));
  return v;
}

// Correctly rounded a / b from rcp = RN(1 / b) with one FMA correction.
// Exact for a bf16 numerator whenever the quotient is a normal fp32 number
// (checked over every bf16 significand against every fp32 divisor
// significand); the sign of a zero quotient is restored explicitly.
__device__ __forceinline__ float div_fast(float a, float b, float rcp) {
  const float q0 = a * rcp;
  const float r = __builtin_fmaf(-q0, b, a);
  return __builtin_copysignf(__builtin_fmaf(r, rcp, q0), a);
}

// E4M3FN code of q: round to nearest even, |q| > 448 saturates to 448,
// sign kept (also for zero).
__device__ __forceinline__ uint32_t enc_e4m3(float q) {
  const uint32_t u = __float_as_uint(q);
  const uint32_t s = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a > 0x43E00000u) {          // > 448
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
// even code, saturating at 6.
__device__ __forceinline__ uint32_t enc_e2m1(float q) {
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
  int E = eb - 127 - FE + (int)((u & 0x7FFFFFu) > FM);
  return E < -127 ? -127 : (E > 127 ? 127 : E);
}

// 2^-E as an exact float, E in [-127, 127].
__device__ __forceinline__ float exp2_neg(int E) {
  return E == 127 ? __uint_as_float(0x00400000u) : __uint_as_float((uint32_t)(127 - E) << 23);
}

// ------------------------------------------------------------------------
// stores honouring the row alignment `al` (a power of two, uniform)
// ------------------------------------------------------------------------
__device__ __forceinline__ void st_u8(uint8_t *p, uint32_t v) { *p = (uint8_t)v; }
__device__ __forceinline__ void st_u16(uint8_t *p, uint32_t v, int al) {
  if (al >= 2) {
    *reinterpret_cast<uint16_t *>(p) = (uint16_t)v;
  } else {
    p[0] = (uint8_t)v;
    p[1] = (uint8_t)(v >> 8);
  }
}
__device__ __forceinline__ void st_u32(uint8_t *p, uint32_t v, int al) {
  if (al >= 4) {
    *reinterpret_cast<uint32_t *>(p) = v;
  } else if (al >= 2) {
    reinterpret_cast<uint16_t *>(p)[0] = (uint16_t)v;
    reinterpret_cast<uint16_t *>(p)[1] = (uint16_t)(v >> 16);
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) p[k] = (uint8_t)(v >> (8 * k));
  }
}
__device__ __forceinline__ void st_u64(uint8_t *p, uint2 v, int al) {
  if (al >= 8) {
    *reinterpret_cast<uint2 *>(p) = v;
  } else {
    st_u32(p, v.x, al);
    st_u32(p + 4, v.y, al);
  }
}
__device__ __forceinline__ void st_u128(uint8_t *p, uint4 v, int al) {
  if (al >= 16) {
    *reinterpret_cast<uint4 *>(p) = v;
  } else {
    st_u64(p, make_uint2(v.x, v.y), al);
    st_u64(p + 8, make_uint2(v.z, v.w), al);
  }
}

__device__ __forceinline__ uint8_t *row_addr(uint8_t *base, uint32_t s, const KArgs &a,
                                             int64_t pitch, int64_t bstride) {
  const uint32_t blk = (uint32_t)(((uint64_t)s * a.bs_magic) >> a.bs_shift);
  const uint32_t pos = s - blk * (uint32_t)a.block_size;
  return base + (int64_t)blk * bstride + (int64_t)pos * pitch;
}

__device__ __forceinline__ uint4 ld16(const uint16_t *p) {
  return *reinterpret_cast<const uint4 *>(p);
}
__device__ __forceinline__ uint2 ld8(const uint16_t *p) {
  return *reinterpret_cast<const uint2 *>(p);
}

__device__ __forceinline__ void unpack8(const uint4 w, float (&v)[8]) {
  v[0] = lo_f(w.x); v[1] = hi_f(w.x);
  v[2] = lo_f(w.y); v[3] = hi_f(w.y);
  v[4] = lo_f(w.z); v[5] = hi_f(w.z);
  v[6] = lo_f(w.w); v[7] = hi_f(w.w);
}

// ------------------------------------------------------------------------
// the epilog kernel
// ------------------------------------------------------------------------
enum { M_FP8_BF16 = 0, M_FP8_E8M0 = 1, M_MXFP4 = 3, M_SPLIT = 4 };

template <int MODE, bool NORM, bool ROPE, int L, int C>
__global__ __launch_bounds__(256) void epilog_kernel(const KArgs a) {
  constexpr int R = 64 / L;  // rows per wave per iteration
  const int lane = threadIdx.x & 63;
  const int li = lane & (L - 1);
  const int sub = lane / L;
  int blk = blockIdx.x;
  if (a.xcd_blocks > 0) blk = (blk & 7) * a.xcd_blocks + (blk >> 3);
  const int wave = blk * 4 + (threadIdx.x >> 6);

  // gamma of this lane's chunks, kept in registers across rows
  constexpr bool KEEP_G = NORM && C <= 2;
  uint4 gw[KEEP_G ? C : 1];
  if constexpr (KEEP_G) {
#pragma unroll
    for (int j = 0; j < C; ++j) {
      const int c = li + L * j;
      gw[j] = c < a.nchunk ? ld16(a.gamma + 8 * c) : make_uint4(0, 0, 0, 0);
    }
  }

  for (int64_t rg = wave; rg * R < a.T; rg += a.nwaves) {
    const int64_t row = rg * R + sub;
    int slot = row < a.T ? a.slots[row] : -1;
    if constexpr (L == 64) slot = __builtin_amdgcn_readfirstlane(slot);
    if ((uint32_t)slot >= (uint32_t)a.num_slots) continue;

    const uint16_t *xr = a.x + row * a.x_stride;
    uint4 xw[C];
#pragma unroll
    for (int j = 0; j < C; ++j) {
      const int c = li + L * j;
      xw[j] = c < a.nchunk ? ld16(xr + 8 * c) : make_uint4(0, 0, 0, 0);
    }
    // rope chunk (lanes li < 8): 4 interleaved (a, b) pairs
    uint4 rw = make_uint4(0, 0, 0, 0);
    uint2 c0w, c1w, s0w, s1w;
    if constexpr (MODE != M_MXFP4) {
      if (li < 8) {
        rw = ld16(xr + a.nseg + 8 * li);
        if constexpr (ROPE) {
          const uint16_t *cr = a.cos + row * 64;
          const uint16_t *sr = a.sin + row * 64;
          c0w = ld8(cr + 4 * li);
          c1w = ld8(cr + 32 + 4 * li);
          s0w = ld8(sr + 4 * li);
          s1w = ld8(sr + 32 + 4 * li);
        }
      }
    }

    // ---- RMSNorm -> packed bf16 yw ----
    uint4 yw[C];
    if constexpr (NORM) {
      float part[C];
#pragma unroll
      for (int j = 0; j < C; ++j) {
        float v[8];
        unpack8(xw[j], v);
        float s01 = v[0] * v[0] + v[1] * v[1];
        float s23 = v[2] * v[2] + v[3] * v[3];
        float s45 = v[4] * v[4] + v[5] * v[5];
        float s67 = v[6] * v[6] + v[7] * v[7];
        part[j] = grp_sum<L>((s01 + s23) + (s45 + s67));
      }
#pragma unroll
      for (int w = 1; w < C; w *= 2)
#pragma unroll
        for (int j = 0; j < C; j += 2 * w) part[j] = part[j] + part[j + w];
      const float ss = part[0];
      const float mean = ss / a.nseg_f;
      const float rms = __builtin_sqrtf(mean + a.eps);
      const float rcp = 1.0f / rms;
      // The fast division needs a normal rms with a normal reciprocal, a
      // normal quotient (|x| >= 2^(e(rms) - 252) guarantees it) and an exact
      // FMA residual (|x| >= 2^-100 keeps it far from underflow).  Zeros are
      // exact either way, so the scan is over nonzero magnitudes (packed
      // 16-bit: magnitude - 1 wraps zero to 0xFFFF).
      const int re = (int)(__float_as_uint(rms) >> 23);
      bool fast = re >= 127 - 100 && re <= 127 + 100;
      const int k = re - 252 > -100 ? re - 252 : -100;
      const uint32_t thr = (uint32_t)(k + 127) << 7;  // bf16 bits of 2^k
      u16x2_t mn = {0xFFFF, 0xFFFF};
#pragma unroll
      for (int j = 0; j < C; ++j) {
        const int c = li + L * j;
        if (c < a.nchunk) {
          const uint32_t ws[4] = {xw[j].x, xw[j].y, xw[j].z, xw[j].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const u16x2_t m = __builtin_bit_cast(u16x2_t, ws[q] & 0x7FFF7FFFu);
            const u16x2_t one = {1, 1};
            mn = __builtin_elementwise_min(mn, (u16x2_t)(m - one));
          }
        }
      }
      const uint32_t mnl = (uint32_t)(mn.x < mn.y ? mn.x : mn.y);
      const bool tiny = mnl < thr - 1;
      if constexpr (L == 64) {
        fast = fast && __builtin_amdgcn_ballot_w64(tiny) == 0;
      } else {
        const uint64_t bal = __builtin_amdgcn_ballot_w64(tiny);
        fast = fast && ((bal >> (sub * L)) & ((1ull << L) - 1)) == 0;
      }
#pragma unroll
      for (int j = 0; j < C; ++j) {
        const int c = li + L * j;
        float v[8], g[8], y[8];
        unpack8(xw[j], v);
        if constexpr (KEEP_G) {
          unpack8(gw[j], g);
        } else {
          unpack8(c < a.nchunk ? ld16(a.gamma + 8 * c) : make_uint4(0, 0, 0, 0), g);
        }
        if (fast) {
#pragma unroll
          for (int k = 0; k < 8; ++k) y[k] = div_fast(v[k], rms, rcp) * g[k];
        } else {
#pragma unroll
          for (int k = 0; k < 8; ++k) y[k] = (v[k] / rms) * g[k];
        }
        yw[j] = make_uint4(pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3]), pack_bf16(y[4], y[5]),
                           pack_bf16(y[6], y[7]));
      }
    } else {
#pragma unroll
      for (int j = 0; j < C; ++j) yw[j] = xw[j];
    }

    // ---- RoPE -> packed bf16 halves (rope lanes) ----
    uint2 y0w = make_uint2(0, 0), y1w = make_uint2(0, 0);
    if constexpr (MODE != M_MXFP4 && ROPE) {
      if (li < 8) {
        const uint32_t xs[4] = {rw.x, rw.y, rw.z, rw.w};
        const float c0[4] = {lo_f(c0w.x), hi_f(c0w.x), lo_f(c0w.y), hi_f(c0w.y)};
        const float c1[4] = {lo_f(c1w.x), hi_f(c1w.x), lo_f(c1w.y), hi_f(c1w.y)};
        const float s0[4] = {lo_f(s0w.x), hi_f(s0w.x), lo_f(s0w.y), hi_f(s0w.y)};
        const float s1[4] = {lo_f(s1w.x), hi_f(s1w.x), lo_f(s1w.y), hi_f(s1w.y)};
        float o0[4], o1[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float xa = lo_f(xs[k]), xb = hi_f(xs[k]);
          o0[k] = xa * c0[k] + (-xb) * s0[k];  // both products exact
          o1[k] = xb * c1[k] + xa * s1[k];
        }
        y0w = make_uint2(pack_bf16(o0[0], o0[1]), pack_bf16(o0[2], o0[3]));
        y1w = make_uint2(pack_bf16(o1[0], o1[1]), pack_bf16(o1[2], o1[3]));
      }
    }

    // ---- outputs ----
    if constexpr (MODE == M_SPLIT) {
      uint8_t *ck = row_addr(a.cache, (uint32_t)slot, a, a.c_pitch, a.c_bstride);
      uint8_t *kk = row_addr(a.aux, (uint32_t)slot, a, a.a_pitch, a.a_bstride);
#pragma unroll
      for (int j = 0; j < C; ++j) {
        const int c = li + L * j;
        if (c < a.nchunk) st_u128(ck + 16 * c, yw[j], a.c_align);
      }
      if (li < 8) {
        st_u64(kk + 8 * li, y0w, a.a_align);
        st_u64(kk + 64 + 8 * li, y1w, a.a_align);
      }
    } else if constexpr (MODE == M_MXFP4) {
      uint8_t *cr = row_addr(a.cache, (uint32_t)slot, a, a.c_pitch, a.c_bstride);
      uint8_t *sr = row_addr(a.aux, (uint32_t)slot, a, a.a_pitch, a.a_bstride);
#pragma unroll
      for (int j = 0; j < C; ++j) {
        const int c = li + L * j;
        float v[8];
        unpack8(yw[j], v);
        float m = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) m = fmaxf(m, __builtin_fabsf(v[k]));
        m = grp_max<4>(m);  // 32 values = 4 lanes
        const int E = e8m0_exp<2, 0x400000u>(m);  // FP4 max 6 = 1.5 * 2^2
        const float f = exp2_neg(E);
        uint32_t word = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) word |= enc_e2m1(v[k] * f) << (4 * k);
        if (c < a.nchunk) {
          st_u32(cr + 4 * c, word, a.c_align);
          if ((li & 3) == 0) st_u8(sr + (c >> 2), (uint32_t)(E + 127));
        }
      }
    } else {  // FP8 modes
      uint8_t *cr = row_addr(a.cache, (uint32_t)slot, a, a.c_pitch, a.c_bstride);
#pragma unroll
      for (int j = 0; j < C; ++j) {
        const int c = li + L * j;
        float v[8];
        unpack8(yw[j], v);
        float m = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) m = fmaxf(m, __builtin_fabsf(v[k]));
        m = grp_max<8>(m);  // 64 values = 8 lanes
        uint32_t q[8];
        uint32_t sbits;
        if constexpr (MODE == M_FP8_E8M0) {
          const int E = e8m0_exp<8, 0x600000u>(m);  // FP8 max 448 = 1.75 * 2^8
          const float f = exp2_neg(E);
#pragma unroll
          for (int k = 0; k < 8; ++k) q[k] = enc_e4m3(v[k] * f);
          sbits = (uint32_t)(E + 127);
        } else {
          // scale = amax / 448 (IEEE), stored as bf16; codes divide by the
          // stored value
          const float s32 =
              (m >= 0x1p-100f && m <= 0x1p+100f) ? div_fast(m, 448.0f, 1.0f / 448.0f) : m / 448.0f;
          sbits = pack_bf16(s32, 0.0f) & 0xFFFFu;
          const float su = __uint_as_float(sbits << 16);
          // Outside [2^-80, 2^100] a residual or the reciprocal of the fast
          // division could leave the normal range; such groups divide
          // exactly.  An infinite scale (an infinite RMSNorm output) gives
          // +-0 for finite values and the NaN code 0x7F for inf / inf.
          if (su >= 0x1p-80f && su <= 0x1p+100f) {
            const float rs = 1.0f / su;
#pragma unroll
            for (int k = 0; k < 8; ++k) q[k] = enc_e4m3(div_fast(v[k], su, rs));
          } else if (su > 0.0f) {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
              const float qq = v[k] / su;
              q[k] = qq != qq ? 0x7Fu : enc_e4m3(qq);
            }
          } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) q[k] = 0u;
          }
        }
        if (c < a.nchunk) {
          const uint2 codes = make_uint2(q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24),
                                         q[4] | (q[5] << 8) | (q[6] << 16) | (q[7] << 24));
          st_u64(cr + 8 * c, codes, a.c_align);
          if ((li & 7) == 0) {
            const int g = c >> 3;
            if constexpr (MODE == M_FP8_E8M0)
              st_u8(cr + a.nseg + 128 + g, sbits);
            else
              st_u16(cr + a.nseg + 128 + 2 * g, sbits, a.c_align);
          }
        }
      }
      if (li < 8) {
        if constexpr (ROPE) {
          st_u64(cr + a.nseg + 8 * li, y0w, a.c_align);
          st_u64(cr + a.nseg + 64 + 8 * li, y1w, a.c_align);
        } else {
          st_u128(cr + a.nseg + 16 * li, rw, a.c_align);
        }
      }
      if constexpr (MODE == M_FP8_BF16) {
        for (int b = a.concat_col + li; b < a.kv_cache_col; b += L) st_u8(cr + b, 0u);
      }
    }
  }
}

// ------------------------------------------------------------------------
// dispatch
// ------------------------------------------------------------------------
typedef void (*kfn_t)(const KArgs);

template <int MODE, bool NORM, bool ROPE>
kfn_t pick_layout(int L, int C) {
  if (L == 8) return epilog_kernel<MODE, NORM, ROPE, 8, 1>;
  if (L == 16) return epilog_kernel<MODE, NORM, ROPE, 16, 1>;
  if (L == 32) return epilog_kernel<MODE, NORM, ROPE, 32, 1>;
  switch (C) {
    case 1: return epilog_kernel<MODE, NORM, ROPE, 64, 1>;
    case 2: return epilog_kernel<MODE, NORM, ROPE, 64, 2>;
    case 4: return epilog_kernel<MODE, NORM, ROPE, 64, 4>;
    case 8: return epilog_kernel<MODE, NORM, ROPE, 64, 8>;
    default: return epilog_kernel<MODE, NORM, ROPE, 64, 16>;
  }
}

kfn_t pick(int mode, bool norm, bool rope, int L, int C) {
  switch (mode) {
    case M_FP8_BF16:
      if (norm) return rope ? pick_layout<M_FP8_BF16, true, true>(L, C)
                            : pick_layout<M_FP8_BF16, true, false>(L, C);
      return rope ? pick_layout<M_FP8_BF16, false, true>(L, C)
                  : pick_layout<M_FP8_BF16, false, false>(L, C);
    case M_FP8_E8M0:
      if (norm) return rope ? pick_layout<M_FP8_E8M0, true, true>(L, C)
                            : pick_layout<M_FP8_E8M0, true, false>(L, C);
      return rope ? pick_layout<M_FP8_E8M0, false, true>(L, C)
                  : pick_layout<M_FP8_E8M0, false, false>(L, C);
    case M_MXFP4:
      return pick_layout<M_MXFP4, false, false>(L, C);
    default:
      return pick_layout<M_SPLIT, true, true>(L, C);
  }
}

int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

}  // namespace kvepi

kvepi_status kvepi_launch(const kvepi_plan &p, void *stream) {
  using namespace kvepi;
  KArgs a{};
  a.x = p.x;
  a.gamma = p.gamma;
  a.cos = p.cos;
  a.sin = p.sin;
  a.slots = p.slots;
  a.cache = p.cache;
  a.aux = p.aux;
  a.x_stride = p.x_stride;
  a.c_pitch = p.c_pitch;
  a.c_bstride = p.c_bstride;
  a.a_pitch = p.a_pitch;
  a.a_bstride = p.a_bstride;
  // slot / block_size for slot < 2^31: m = ceil(2^(31+l) / bs), l = ceil(log2 bs)
  int l = 0;
  while ((INT64_C(1) << l) < p.block_size) ++l;
  const int shift = 31 + l;
  const unsigned __int128 num = (unsigned __int128)1 << shift;
  a.bs_magic = (uint64_t)((num + (unsigned __int128)p.block_size - 1) / (unsigned __int128)p.block_size);
  a.bs_shift = shift;
  a.block_size = (int32_t)p.block_size;
  a.T = (int32_t)p.T;
  a.num_slots = (int32_t)p.num_slots;
  a.nseg = (int32_t)p.nope;
  a.nchunk = (int32_t)(p.nope / 8);
  a.concat_col = (int32_t)p.concat_col;
  a.kv_cache_col = (int32_t)p.kv_cache_col;
  a.c_align = p.c_align;
  a.a_align = p.mode == KVEPI_MODE_MXFP4 || p.mode == KVEPI_MODE_BF16_SPLIT ? p.a_align : 16;
  a.eps = p.eps;
  a.nseg_f = (float)p.nope;

  // layout: L lanes per row (power of two, 8..64), C chunks per lane
  int L = 8;
  while (L < 64 && L < a.nchunk) L *= 2;
  int C = 1;
  while (C * L < a.nchunk) C *= 2;

  const int rows_per_wave = 64 / L;
  const int64_t waves_needed = (p.T + rows_per_wave - 1) / rows_per_wave;
  const int cus = device_cus();
  const int64_t max_waves = (int64_t)cus * 32;  // 8 blocks of 4 waves per CU
  int64_t waves = waves_needed < max_waves ? waves_needed : max_waves;
  int64_t blocks = (waves + 3) / 4;
  a.nwaves = (int32_t)(blocks * 4);
  a.xcd_blocks = (blocks % 8 == 0) ? (int32_t)(blocks / 8) : 0;

  kfn_t fn = pick(p.mode, p.norm, p.rope, L, C);
  void *args[] = {&a};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(fn), dim3((unsigned)blocks),
                                 dim3(256), args, 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVEPI_OK : KVEPI_ERR_RUNTIME;
}
