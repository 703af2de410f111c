// kvepi_drq.hip -- gfx950 kernel of the dequant -> RoPE -> static int8
// quantisation -> KV cache operator (the blog on
// aclnnDequantRopeQuantKvcache: 计算步骤公式 steps 1-5).
//
// The work is elementwise except for the rotate-half RoPE, which pairs value
// j of a head with value j + D/2.  One thread owns a "unit" of 2V values of
// one head: V consecutive values of its first half and the V values D/2
// further on, so the rotation needs no exchange between lanes.  Consecutive
// threads take consecutive units of a token (and heads follow each other).
// V is 8: a half of a unit is one 16-byte piece of 16-bit x or two of int32
// x, and a wave's loads cover contiguous bytes.  (Four int32 values per half,
// one piece, measured 3.5 % slower: twice the threads, and with them twice
// the scale, bias, cos and sin loads per byte of x.)
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
  uint64_t u_magic;  // token = thread / U
  int32_t u_shift, U;
  uint64_t h_magic;  // head = unit-in-token / (units per head)
  int32_t h_shift, upH;
  uint64_t s_magic;  // batch = token / seq_len (contiguous mode)
  int32_t s_shift, S;
  uint64_t bs_magic;  // block = slot / block_size
  int32_t bs_shift, bs_log2, block_size;
  int32_t num_slots;
  int32_t nq, nkv, D;
  int32_t contiguous;
  uint32_t total;  // threads (units)
};

typedef unsigned int u32x4v_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t mdiv(uint32_t n, uint64_t m, int s) {
  return (uint32_t)(((uint64_t)n * m) >> s);
}

// NW consecutive 32-bit words (NW = 1, 2 or 4) from p; NT: streamed load
template <int NW, bool NT = false>
__device__ __forceinline__ void ldw(const uint8_t *p, uint32_t (&w)[NW]) {
  if constexpr (NW == 4) {
    if constexpr (NT) {
      const u32x4v_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4v_t *>(p));
      w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    } else {
      const uint4 v = *reinterpret_cast<const uint4 *>(p);
      w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    }
  } else if constexpr (NW == 2) {
    const uint2 v = *reinterpret_cast<const uint2 *>(p);
    w[0] = v.x; w[1] = v.y;
  } else {
    w[0] = *reinterpret_cast<const uint32_t *>(p);
  }
}
template <int NW>
__device__ __forceinline__ void stw(uint8_t *p, const uint32_t (&w)[NW]) {
  if constexpr (NW == 4)
    *reinterpret_cast<uint4 *>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  else if constexpr (NW == 2)
    *reinterpret_cast<uint2 *>(p) = make_uint2(w[0], w[1]);
  else
    *reinterpret_cast<uint32_t *>(p) = w[0];
}

// V 16-bit values of type DT (V / 2 words) as fp32
template <int DT, int V>
__device__ __forceinline__ void unpack(const uint32_t (&w)[V / 2], float (&v)[V]) {
#pragma unroll
  for (int k = 0; k < V / 2; ++k) {
    if constexpr (DT == KVEPI_DT_FP16) {
      v[2 * k] = kvepi::f16_lo(w[k]);
      v[2 * k + 1] = kvepi::f16_hi(w[k]);
    } else {
      v[2 * k] = __uint_as_float(w[k] << 16);
      v[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
    }
  }
}

// fp32 -> the 16-bit output type, round to nearest even (v_cvt_pk_bf16_f32 /
// v_cvt_f16_f32; tests/hw_check.hip compares both with a software rounding
// for every fp32 value)
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

template <int DT>
__device__ __forceinline__ uint32_t pack16(float a, float b) {
  if constexpr (DT == KVEPI_DT_FP16) {
    const f32x2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
  } else {
    return kvepi::pack_bf16_rn(a, b);
  }
}
template <int DT, int V>
__device__ __forceinline__ void pack(const float (&v)[V], uint32_t (&w)[V / 2]) {
#pragma unroll
  for (int k = 0; k < V / 2; ++k) w[k] = pack16<DT>(v[2 * k], v[2 * k + 1]);
}

template <int V>
__device__ __forceinline__ void loadf(const float *p, float (&v)[V]) {
  uint32_t w[V];
  if constexpr (V == 8) {
    uint32_t a[4], b[4];
    ldw<4>(reinterpret_cast<const uint8_t *>(p), a);
    ldw<4>(reinterpret_cast<const uint8_t *>(p + 4), b);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      w[k] = a[k];
      w[k + 4] = b[k];
    }
  } else {
    ldw<V>(reinterpret_cast<const uint8_t *>(p), w);
  }
#pragma unroll
  for (int k = 0; k < V; ++k) v[k] = __uint_as_float(w[k]);
}

// bias values h .. h+V-1 as fp32
template <int V>
__device__ __forceinline__ void load_bias(const DArgs &a, int64_t h, float (&v)[V]) {
  if (a.bias_dt == KVEPI_DT_FP32 || a.bias_dt == KVEPI_DT_INT32) {
    loadf<V>(reinterpret_cast<const float *>(a.bias) + h, v);
    if (a.bias_dt == KVEPI_DT_INT32) {
#pragma unroll
      for (int k = 0; k < V; ++k) v[k] = (float)(int32_t)__float_as_uint(v[k]);
    }
  } else {
    uint32_t w[V / 2];
    ldw<V / 2>(a.bias + 2 * h, w);
    if (a.bias_dt == KVEPI_DT_FP16)
      unpack<KVEPI_DT_FP16, V>(w, v);
    else
      unpack<KVEPI_DT_BF16, V>(w, v);
  }
}

// step 1 for values h .. h+V-1 of token t: x, or its dequantisation rounded
// to the output type (then read back as fp32)
template <int XT, int OT, int V>
__device__ __forceinline__ void dequant(const DArgs &a, uint32_t t, int64_t h, float (&v)[V]) {
  const uint8_t *xr = a.x + (int64_t)t * a.x_pitch;
  if constexpr (XT == KVEPI_DT_INT32) {
    static_assert(V == 8, "int32 rows: 8 values (two 16-byte pieces) per half");
    uint32_t xa[4], xb[4], xi[V];
    ldw<4, true>(xr + 4 * h, xa);
    ldw<4, true>(xr + 4 * h + 16, xb);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      xi[k] = xa[k];
      xi[k + 4] = xb[k];
    }
    float w[V];
    loadf<V>(a.w + h, w);
#pragma unroll
    for (int k = 0; k < V; ++k) v[k] = (float)(int32_t)xi[k] * w[k];
    if (a.act != nullptr) {
      const float s = a.act[t];
#pragma unroll
      for (int k = 0; k < V; ++k) v[k] = v[k] * s;
    }
    if (a.bias_dt >= 0) {
      float b[V];
      load_bias<V>(a, h, b);
#pragma unroll
      for (int k = 0; k < V; ++k) v[k] = v[k] + b[k];
    }
    uint32_t p[V / 2];
    pack<OT, V>(v, p);
    unpack<OT, V>(p, v);
  } else {
    static_assert(V == 8, "16-bit rows: 8 values (16 bytes) per half");
    uint32_t w[4];
    ldw<4, true>(xr + 2 * h, w);
    unpack<XT, V>(w, v);
  }
}

// step 4 for V channels: rint(v / scale + offset) saturated to int8, packed
// (IEEE division: a reciprocal with one correction, guarded to the range
// where it is exact, measured no faster here)
template <int V>
__device__ __forceinline__ void quant(const float (&v)[V], const float *sc, const float *of,
                                      uint32_t (&out)[V / 4]) {
  float s[V], o[V];
  loadf<V>(sc, s);
  if (of != nullptr) loadf<V>(of, o);
#pragma unroll
  for (int k = 0; k < V / 4; ++k) out[k] = 0;
#pragma unroll
  for (int k = 0; k < V; ++k) {
    float q = v[k] / s[k];
    if (of != nullptr) q = q + o[k];
    const float r = __builtin_fminf(__builtin_fmaxf(__builtin_rintf(q), -128.0f), 127.0f);
    out[k / 4] |= ((uint32_t)(int32_t)r & 0xFFu) << (8 * (k % 4));
  }
}

template <int XT, int OT, int V>
__global__ __launch_bounds__(256) void drq_kernel(const DArgs a) {
  const uint32_t i = blockIdx.x * 256u + threadIdx.x;
  if (i >= a.total) return;
  const uint32_t t = mdiv(i, a.u_magic, a.u_shift);
  const uint32_t u = i - t * (uint32_t)a.U;
  const uint32_t head = mdiv(u, a.h_magic, a.h_shift);
  const int32_t j0 = V * (int32_t)(u - head * (uint32_t)a.upH);
  const int32_t D = a.D, half = D / 2;
  const int64_t h0 = (int64_t)head * D + j0, h1 = h0 + half;

  float x0[V], x1[V];
  dequant<XT, OT, V>(a, t, h0, x0);
  dequant<XT, OT, V>(a, t, h1, x1);

  const int32_t nq = a.nq, nkv = a.nkv;
  float y0[V], y1[V];
  if ((int32_t)head < nq + nkv) {
    // rotate-half RoPE with the token's cos / sin: two products, one sum
    float c0[V], c1[V], s0[V], s1[V];
    uint32_t w[V / 2];
    const int64_t cb = 2 * ((int64_t)t * D + j0);
    ldw<V / 2>(a.cos + cb, w);
    unpack<OT, V>(w, c0);
    ldw<V / 2>(a.cos + cb + 2 * half, w);
    unpack<OT, V>(w, c1);
    ldw<V / 2>(a.sin + cb, w);
    unpack<OT, V>(w, s0);
    ldw<V / 2>(a.sin + cb + 2 * half, w);
    unpack<OT, V>(w, s1);
#pragma unroll
    for (int k = 0; k < V; ++k) {
      if constexpr (OT == KVEPI_DT_FP16) {
        // fp16 products are exact in fp32 (22 significant bits, never
        // below 2^-48), so one FMA gives the rounded sum of the two
        y0[k] = __builtin_fmaf(x0[k], c0[k], -(x1[k] * s0[k]));
        y1[k] = __builtin_fmaf(x1[k], c1[k], x0[k] * s1[k]);
      } else {
        // bf16 products can fall below the fp32 normal range: round each
        const float p0 = x0[k] * c0[k], q0 = x1[k] * s0[k];
        const float p1 = x1[k] * c1[k], q1 = x0[k] * s1[k];
        y0[k] = p0 - q0;
        y1[k] = p1 + q1;
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < V; ++k) {
      y0[k] = x0[k];
      y1[k] = x1[k];
    }
  }
  uint32_t w0[V / 2], w1[V / 2];
  pack<OT, V>(y0, w0);
  pack<OT, V>(y1, w1);
  if ((int32_t)head < nq) {
    uint8_t *qo = a.q_out + 2 * ((int64_t)t * nq * D + h0);
    stw<V / 2>(qo, w0);
    stw<V / 2>(qo + 2 * half, w1);
    return;
  }
  // k or v head: the 16-bit output, then the int8 codes of the rounded values
  const bool is_k = (int32_t)head < nq + nkv;
  const int32_t hk = (int32_t)head - (is_k ? nq : nq + nkv);
  const int64_t c = (int64_t)hk * D + j0;  // channel in [nkv * D]
  uint8_t *out = is_k ? a.k_out : a.v_out;
  if (out != nullptr) {
    uint8_t *o = out + 2 * ((int64_t)t * nkv * D + c);
    stw<V / 2>(o, w0);
    stw<V / 2>(o + 2 * half, w1);
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
  unpack<OT, V>(w0, y0);  // quantise the values as output (rounded)
  unpack<OT, V>(w1, y1);
  const float *sc = is_k ? a.sk : a.sv;
  const float *of = is_k ? a.ok : a.ov;
  uint8_t *row = is_k ? a.kc + (int64_t)blk * a.k_bstride + (int64_t)pos * a.k_pitch
                      : a.vc + (int64_t)blk * a.v_bstride + (int64_t)pos * a.v_pitch;
  uint32_t q0[V / 4], q1[V / 4];
  quant<V>(y0, sc + c, of ? of + c : nullptr, q0);
  quant<V>(y1, sc + c + half, of ? of + c + half : nullptr, q1);
  stw<V / 4>(row + c, q0);
  stw<V / 4>(row + c + half, q1);
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
  const bool i32 = p.x_dtype == KVEPI_DT_INT32;
  const int V = 8;  // values per half-unit
  a.x = static_cast<const uint8_t *>(p.x);
  a.x_pitch = p.x_row_stride * (i32 ? 4 : 2);
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
  a.U = (int32_t)(pl.H / (2 * V));
  magic((uint32_t)a.U, &a.u_magic, &a.u_shift);
  a.upH = p.head_dim / (2 * V);
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
  a.total = (uint32_t)(p.num_tokens * a.U);

  kfn_t fn;
  if (i32)
    fn = p.out_dtype == KVEPI_DT_FP16 ? drq_kernel<KVEPI_DT_INT32, KVEPI_DT_FP16, 8>
                                      : drq_kernel<KVEPI_DT_INT32, KVEPI_DT_BF16, 8>;
  else
    fn = p.out_dtype == KVEPI_DT_FP16 ? drq_kernel<KVEPI_DT_FP16, KVEPI_DT_FP16, 8>
                                      : drq_kernel<KVEPI_DT_BF16, KVEPI_DT_BF16, 8>;
  const uint32_t blocks = (a.total + 255u) / 256u;
  void *args[] = {&a};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(fn), dim3(blocks),
                                       dim3(256), args, 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVEPI_OK : KVEPI_ERR_RUNTIME;
}
