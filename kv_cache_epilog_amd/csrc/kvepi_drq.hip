// kvepi_drq.hip -- gfx950 kernel of the dequant -> RoPE -> static int8
// quantisation -> KV cache operator (the blog on
// aclnnDequantRopeQuantKvcache: 计算步骤公式 steps 1-5).
//
// The work is elementwise except for the rotate-half RoPE, which pairs value
// j of a head with value j + D/2.  One thread owns a "unit" of 16 values of
// one head: 8 consecutive values of its first half and the 8 values D/2
// further on, so the rotation needs no exchange between lanes.  Consecutive
// threads take consecutive units of a token (and heads follow each other),
// so every load and store instruction covers contiguous 16-byte pieces.
// The path is bound by HBM bandwidth: each value is read once (2 or 4 bytes)
// and written once or twice (the 16-bit outputs and the int8 cache).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvepi_arith.h"
#include "kvepi_drq_plan.h"

namespace kvepi_drq {

struct DArgs {
  const uint8_t *x;
  int64_t x_pitch;  // bytes between rows of x
  const uint8_t *cos, *sin;
  const float *w, *act;
  const uint8_t *bias;
  int32_t bias_dt;  // -1: no bias
  const float *sk, *sv, *ok, *ov;
  const int32_t *idx;
  uint8_t *kc, *vc;
  int64_t k_pitch, k_bstride, v_pitch, v_bstride;
  uint8_t *q_out, *k_out, *v_out;
  uint64_t u_magic;  // token = unit / U
  int32_t u_shift, U;
  uint64_t h_magic;  // head = unit-in-token / (D / 16)
  int32_t h_shift, upH;
  uint64_t s_magic;  // batch = token / seq_len (contiguous mode)
  int32_t s_shift, S;
  uint64_t bs_magic;  // block = slot / block_size
  int32_t bs_shift, bs_log2, block_size;
  int32_t num_slots;
  int32_t nq, nkv, D;
  int32_t contiguous;
  uint32_t total;  // units
};

typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4v_t __attribute__((ext_vector_type(4)));

// streamed 16-byte loads (x is read once)
__device__ __forceinline__ int4 ldnt_i4(const uint8_t *p) {
  const i32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const i32x4_t *>(p));
  return make_int4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 ldnt_u4(const uint8_t *p) {
  const u32x4v_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4v_t *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint32_t mdiv(uint32_t n, uint64_t m, int s) {
  return (uint32_t)(((uint64_t)n * m) >> s);
}

template <int DT>
__device__ __forceinline__ void unpack16(const uint4 w, float (&v)[8]) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if constexpr (DT == KVEPI_DT_FP16) {
      v[2 * k] = kvepi::f16_lo(ws[k]);
      v[2 * k + 1] = kvepi::f16_hi(ws[k]);
    } else {
      v[2 * k] = __uint_as_float(ws[k] << 16);
      v[2 * k + 1] = __uint_as_float(ws[k] & 0xFFFF0000u);
    }
  }
}

// fp32 -> the 16-bit output type, round to nearest even (v_cvt_pk_bf16_f32 /
// v_cvt_f16_f32; tests/hw_check.hip compares both with a software rounding
// for every fp32 value)
template <int DT>
__device__ __forceinline__ uint32_t pack16(float a, float b) {
  if constexpr (DT == KVEPI_DT_FP16) {
    const _Float16 ha = (_Float16)a, hb = (_Float16)b;
    return (uint32_t)__builtin_bit_cast(unsigned short, ha) |
           ((uint32_t)__builtin_bit_cast(unsigned short, hb) << 16);
  } else {
    return kvepi::pack_bf16_rn(a, b);
  }
}
template <int DT>
__device__ __forceinline__ uint4 pack8(const float (&v)[8]) {
  return make_uint4(pack16<DT>(v[0], v[1]), pack16<DT>(v[2], v[3]), pack16<DT>(v[4], v[5]),
                    pack16<DT>(v[6], v[7]));
}

__device__ __forceinline__ void load8f(const float *p, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4 *>(p);
  const float4 b = *reinterpret_cast<const float4 *>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// bias values h .. h+7 as fp32
__device__ __forceinline__ void load_bias(const DArgs &a, int64_t h, float (&v)[8]) {
  if (a.bias_dt == KVEPI_DT_FP32) {
    load8f(reinterpret_cast<const float *>(a.bias) + h, v);
  } else if (a.bias_dt == KVEPI_DT_INT32) {
    const int4 p = *reinterpret_cast<const int4 *>(a.bias + 4 * h);
    const int4 q = *reinterpret_cast<const int4 *>(a.bias + 4 * h + 16);
    v[0] = (float)p.x; v[1] = (float)p.y; v[2] = (float)p.z; v[3] = (float)p.w;
    v[4] = (float)q.x; v[5] = (float)q.y; v[6] = (float)q.z; v[7] = (float)q.w;
  } else {
    const uint4 w = *reinterpret_cast<const uint4 *>(a.bias + 2 * h);
    if (a.bias_dt == KVEPI_DT_FP16)
      unpack16<KVEPI_DT_FP16>(w, v);
    else
      unpack16<KVEPI_DT_BF16>(w, v);
  }
}

// step 1 for values h .. h+7 of token t: x, or its dequantisation rounded to
// the output type (then read back as fp32)
template <int XT, int OT>
__device__ __forceinline__ void dequant8(const DArgs &a, uint32_t t, int64_t h, float (&v)[8]) {
  const uint8_t *xr = a.x + (int64_t)t * a.x_pitch;
  if constexpr (XT == KVEPI_DT_INT32) {
    const int4 p = ldnt_i4(xr + 4 * h);
    const int4 q = ldnt_i4(xr + 4 * h + 16);
    const int xi[8] = {p.x, p.y, p.z, p.w, q.x, q.y, q.z, q.w};
    float w[8];
    load8f(a.w + h, w);
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = (float)xi[k] * w[k];
    if (a.act != nullptr) {
      const float s = a.act[t];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = v[k] * s;
    }
    if (a.bias_dt >= 0) {
      float b[8];
      load_bias(a, h, b);
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = v[k] + b[k];
    }
    unpack16<OT>(pack8<OT>(v), v);
  } else {
    const uint4 w = ldnt_u4(xr + 2 * h);
    unpack16<XT>(w, v);
  }
}

// step 4 for 8 channels: rint(v / scale + offset) saturated to int8, packed
__device__ __forceinline__ uint2 quant8(const float (&v)[8], const float *sc, const float *of) {
  float s[8], o[8];
  load8f(sc, s);
  if (of != nullptr) load8f(of, o);
  uint32_t b[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    float q = v[k] / s[k];
    if (of != nullptr) q = q + o[k];
    const float r = __builtin_fminf(__builtin_fmaxf(__builtin_rintf(q), -128.0f), 127.0f);
    b[k] = (uint32_t)(int32_t)r & 0xFFu;
  }
  return make_uint2(b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24),
                    b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24));
}

template <int XT, int OT>
__global__ __launch_bounds__(256) void drq_kernel(const DArgs a) {
  const uint32_t i = blockIdx.x * 256u + threadIdx.x;
  if (i >= a.total) return;
  const uint32_t t = mdiv(i, a.u_magic, a.u_shift);
  const uint32_t u = i - t * (uint32_t)a.U;
  const uint32_t head = mdiv(u, a.h_magic, a.h_shift);
  const int32_t j0 = 8 * (int32_t)(u - head * (uint32_t)a.upH);
  const int32_t D = a.D, half = D / 2;
  const int64_t h0 = (int64_t)head * D + j0, h1 = h0 + half;

  float x0[8], x1[8];
  dequant8<XT, OT>(a, t, h0, x0);
  dequant8<XT, OT>(a, t, h1, x1);

  const int32_t nq = a.nq, nkv = a.nkv;
  float y0[8], y1[8];
  if ((int32_t)head < nq + nkv) {
    // rotate-half RoPE with the token's cos / sin: two products, one sum
    float c0[8], c1[8], s0[8], s1[8];
    const int64_t cb = 2 * ((int64_t)t * D + j0);
    unpack16<OT>(*reinterpret_cast<const uint4 *>(a.cos + cb), c0);
    unpack16<OT>(*reinterpret_cast<const uint4 *>(a.cos + cb + 2 * half), c1);
    unpack16<OT>(*reinterpret_cast<const uint4 *>(a.sin + cb), s0);
    unpack16<OT>(*reinterpret_cast<const uint4 *>(a.sin + cb + 2 * half), s1);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float p0 = x0[k] * c0[k], q0 = x1[k] * s0[k];
      const float p1 = x1[k] * c1[k], q1 = x0[k] * s1[k];
      y0[k] = p0 - q0;
      y1[k] = p1 + q1;
    }
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      y0[k] = x0[k];
      y1[k] = x1[k];
    }
  }
  const uint4 w0 = pack8<OT>(y0), w1 = pack8<OT>(y1);
  if ((int32_t)head < nq) {
    uint8_t *qo = a.q_out + 2 * ((int64_t)t * nq * D + h0);
    *reinterpret_cast<uint4 *>(qo) = w0;
    *reinterpret_cast<uint4 *>(qo + 2 * half) = w1;
    return;
  }
  // k or v head: the 16-bit output, then the int8 codes of the rounded values
  const bool is_k = (int32_t)head < nq + nkv;
  const int32_t hk = (int32_t)head - (is_k ? nq : nq + nkv);
  const int64_t c = (int64_t)hk * D + j0;  // channel in [nkv * D]
  uint8_t *out = is_k ? a.k_out : a.v_out;
  if (out != nullptr) {
    uint8_t *o = out + 2 * ((int64_t)t * nkv * D + c);
    *reinterpret_cast<uint4 *>(o) = w0;
    *reinterpret_cast<uint4 *>(o + 2 * half) = w1;
  }
  // the token's cache row (page: its slot; contiguous: row start[b] + s of
  // block b); -1 or a row outside the cache skips the write
  uint32_t slot;
  if (a.contiguous) {
    const uint32_t b = mdiv(t, a.s_magic, a.s_shift);
    const uint32_t s = t - b * (uint32_t)a.S;
    const uint32_t v = (uint32_t)a.idx[b];
    const uint32_t bs = (uint32_t)a.block_size;
    slot = v < bs && v + s < bs ? b * bs + v + s : 0xFFFFFFFFu;
  } else {
    slot = (uint32_t)a.idx[t];
  }
  if (slot >= (uint32_t)a.num_slots) return;
  const uint32_t blk =
      a.bs_log2 >= 0 ? slot >> a.bs_log2 : mdiv(slot, a.bs_magic, a.bs_shift);
  const uint32_t pos = slot - blk * (uint32_t)a.block_size;
  unpack16<OT>(w0, y0);  // quantise the values as output (rounded)
  unpack16<OT>(w1, y1);
  const float *sc = is_k ? a.sk : a.sv;
  const float *of = is_k ? a.ok : a.ov;
  uint8_t *row = is_k ? a.kc + (int64_t)blk * a.k_bstride + (int64_t)pos * a.k_pitch
                      : a.vc + (int64_t)blk * a.v_bstride + (int64_t)pos * a.v_pitch;
  *reinterpret_cast<uint2 *>(row + c) = quant8(y0, sc + c, of ? of + c : nullptr);
  *reinterpret_cast<uint2 *>(row + c + half) =
      quant8(y1, sc + c + half, of ? of + c + half : nullptr);
}

// n / d == (n * m) >> s for every n < 2^31 (m = ceil(2^(31+l) / d), l =
// ceil(log2 d))
void magic(uint32_t d, uint64_t *m, int32_t *s) {
  int l = 0;
  while ((UINT64_C(1) << l) < d) ++l;
  const unsigned __int128 n = (unsigned __int128)1 << (31 + l);
  *m = (uint64_t)((n + d - 1) / d);
  *s = 31 + l;
}

typedef void (*kfn_t)(const DArgs);

}  // namespace kvepi_drq

kvepi_status kvepi_drq_launch(const kvepi_drq_plan &pl, void *stream) {
  using namespace kvepi_drq;
  const kvepi_drq_params &p = pl.p;
  DArgs a{};
  const int xb = p.x_dtype == KVEPI_DT_INT32 ? 4 : 2;
  a.x = static_cast<const uint8_t *>(p.x);
  a.x_pitch = p.x_row_stride * xb;
  a.cos = static_cast<const uint8_t *>(p.cos);
  a.sin = static_cast<const uint8_t *>(p.sin);
  a.w = p.weight_scale;
  a.act = p.act_scale;
  a.bias = static_cast<const uint8_t *>(p.bias);
  a.bias_dt = p.bias ? p.bias_dtype : -1;
  a.sk = p.scale_k;
  a.sv = p.scale_v;
  a.ok = p.offset_k;
  a.ov = p.offset_v;
  a.idx = p.indices;
  a.kc = static_cast<uint8_t *>(p.k_cache.data);
  a.vc = static_cast<uint8_t *>(p.v_cache.data);
  a.k_pitch = pl.k_pitch;
  a.k_bstride = pl.k_bstride;
  a.v_pitch = pl.v_pitch;
  a.v_bstride = pl.v_bstride;
  a.q_out = static_cast<uint8_t *>(p.q_out);
  a.k_out = static_cast<uint8_t *>(p.k_out);
  a.v_out = static_cast<uint8_t *>(p.v_out);
  a.U = (int32_t)(pl.H / 16);
  magic((uint32_t)a.U, &a.u_magic, &a.u_shift);
  a.upH = p.head_dim / 16;
  magic((uint32_t)a.upH, &a.h_magic, &a.h_shift);
  a.contiguous = p.cache_mode == KVEPI_DRQ_CONTIGUOUS;
  a.S = a.contiguous ? (int32_t)p.seq_len : 1;
  magic((uint32_t)a.S, &a.s_magic, &a.s_shift);
  a.block_size = (int32_t)p.k_cache.block_size;
  magic((uint32_t)a.block_size, &a.bs_magic, &a.bs_shift);
  a.bs_log2 = -1;
  for (int l = 0; l < 31; ++l)
    if ((INT64_C(1) << l) == p.k_cache.block_size) a.bs_log2 = l;
  a.num_slots = (int32_t)(p.k_cache.block_num * p.k_cache.block_size);
  a.nq = p.nq;
  a.nkv = p.nkv;
  a.D = p.head_dim;
  a.total = (uint32_t)pl.units;

  kfn_t fn;
  if (p.x_dtype == KVEPI_DT_INT32)
    fn = p.out_dtype == KVEPI_DT_FP16 ? drq_kernel<KVEPI_DT_INT32, KVEPI_DT_FP16>
                                      : drq_kernel<KVEPI_DT_INT32, KVEPI_DT_BF16>;
  else
    fn = p.out_dtype == KVEPI_DT_FP16 ? drq_kernel<KVEPI_DT_FP16, KVEPI_DT_FP16>
                                      : drq_kernel<KVEPI_DT_BF16, KVEPI_DT_BF16>;
  const uint32_t blocks = (a.total + 255u) / 256u;
  void *args[] = {&a};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(fn), dim3(blocks),
                                       dim3(256), args, 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVEPI_OK : KVEPI_ERR_RUNTIME;
}
