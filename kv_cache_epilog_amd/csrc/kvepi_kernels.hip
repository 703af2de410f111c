// kvepi_kernels.hip -- gfx950 kernels of the fused KV-cache write epilog.
//
// One kernel template covers every mode.  A token row is handled by a group
// of L lanes of one 64-lane wavefront (64/L rows per wave-iteration: L = 32,
// two rows per wave, for the d = 576 rows; L = 16, four rows, for the d = 128
// indexer rows).  Each lane owns C 16-byte chunks of 8 16-bit values, chunk
// li + L*j, so every load instruction reads L*16 contiguous bytes of a row.
// The path is bound by HBM bandwidth; the design keeps the VALU work and the
// number of memory instructions per row small:
//  - waves are persistent (one block per resident slot of the device); each
//    wave loads its slots ahead and issues the loads of the row two steps
//    ahead before storing the current one (two register sets);
//  - the 64-column rope segment is spread over 32 tasks of two outputs each
//    (a rope segment of another length, in the bf16 split mode, over one
//    task per output pair);
//  - codes come from the gfx950 converts v_cvt_pk_fp8_f32 /
//    v_cvt_scalef32_pk_fp8_f32 / v_cvt_scalef32_pk_fp4_f32, which round to
//    nearest even exactly like the reference encoders over the value ranges
//    used here (|q| <= 456 for FP8 -- the unscaled convert stops saturating
//    at 464 --, |q| <= 6 for FP4, power-of-two scales in [2^-100, 2^100]);
//    outside those ranges a group falls back to software encoding.
//
// Steps per row (sources cited by page title and section):
//  1. The token's slot: slot_mapping[t], or from the index modes (a row of
//     the token's batch, one block per chunk of block_size tokens, a start
//     row per batch; "aclnnKvRmsNormRopeCache", index constraints); -1, or
//     any value that would leave the cache, skips the token: nothing is
//     written for it ("aclnnKvCompressEpilog", 约束说明).
//  2. RMSNorm of the nope segment ("aclnnKvRmsNormRopeCache", 计算公式 (2)):
//     squares summed as a balanced pairwise tree -- within a lane over its 8
//     values, then across lanes by a DPP / ds_swizzle butterfly whose pairing
//     is exactly the tree's (fp32 addition is commutative, so both lanes of a
//     pair hold the same node), then over the chunk index j; mean = sum / n,
//     rms = sqrt(mean + eps), t = x / rms, u = t * gamma, bf16 output.  All in
//     IEEE fp32; x / rms uses the reciprocal with one FMA correction
//     (Markstein), which returns the correctly rounded quotient for a bf16
//     numerator and a normal result -- a row falls back to full division when
//     that cannot be guaranteed.
//  3. Interleaved RoPE of the rope segment (the last 64 columns, or Dk
//     columns in the bf16 split mode), half-split output
//     ("aclnnKvRmsNormRopeCache", 计算公式 (1)).
//  4. Per-group amax (DPP max over the lanes of a group, or of the whole row
//     for the per-row FP8 mode), the scale ("aclnnKvCompressEpilog",
//     计算公式: amax / 448 as bf16, or the e8m0 power of two rounded up;
//     "indexer_quant_cache": e8m0 over groups of 32 with FP4 max 6 or FP8
//     max 448, or amax / 448 in fp32 for the whole row) and the codes,
//     round-to-nearest-even with saturation.  The indexer modes also read
//     fp16 rows ("indexer_quant_cache", 接口功能).
//  5. Stores of exactly kvCacheCol bytes at the slot's row (plus the scale
//     row or the k row in the second cache).  Mode 0 rows laid out as one or
//     two chunks on each of 32 lanes (d = 320 and d = 576, 16-byte aligned
//     rows) are assembled in LDS and leave as one 16-byte store per lane;
//     otherwise the widest store the row alignment allows is used
//     (16/8/4/2/1 bytes), so odd headDim such as 323 works.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "kvepi_arith.h"
#include "kvepi_plan.h"

namespace kvepi {

struct KArgs {
  const uint16_t *x, *gamma, *cos, *sin;
  const int32_t *slots;
  uint8_t *cache, *aux;
  int64_t x_stride;            // elements
  uint32_t x_pitch;            // bytes between rows of x (2 * x_stride < 2^28)
  int64_t c_pitch, c_bstride;  // bytes
  int64_t a_pitch, a_bstride;  // bytes
  uint64_t bs_magic;           // slot / block_size == (slot * magic) >> shift
  int32_t bs_shift, block_size;
  int32_t bs_log2;  // log2(block_size) if a power of two, else -1
  int32_t T, num_slots;
  int32_t nseg;    // values in the quantised/normalised segment (d-64, or d)
  int32_t nchunk;  // nseg / 8
  int32_t concat_col, kv_cache_col;
  int32_t pad16;  // zero padding as whole 16-byte stores (count), -1: bytes
  int32_t c_align, a_align;
  float eps, inv_nseg;  // inv_nseg != 0: nseg is a power of two, mean = ss*inv
  float nseg_f;
  int32_t index_mode;  // KVEPI_INDEX_*: how a token's cache row is found
  int32_t seq_len;     // tokens per batch (index modes other than SLOT)
  uint64_t sq_magic;   // row / seq_len == (row * sq_magic) >> sq_shift
  int32_t sq_shift;
  int32_t n_chunk_b;   // index entries per batch in the block-index mode
  int32_t glog;        // M_FP4_NOPE: log2(group size / 8), chunks per group 2^glog
  int32_t img_bytes;   // FAST == 2: bytes of a row image staged in LDS
  int32_t img_off;     // FAST == 2: where the image goes in the cache row
  int32_t rope_half;   // M_SPLIT_G: rope_dim / 2 output pairs per row
  int32_t rope_pitch;  // M_SPLIT_G: bytes per cos / sin row (2 * rope_dim)
  int32_t nwaves;      // waves in the grid
  int32_t n_groups;    // row groups (wave-iterations) = ceil(T / rows per wave)
};

// ------------------------------------------------------------------------
// bit-level helpers
// ------------------------------------------------------------------------
__device__ __forceinline__ float lo_f(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 (round to nearest even; v_cvt_pk_bf16_f32), a low.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// y rounded to bf16 (nearest even) and read back as fp32: a zero low half
// next to the bf16 code makes the word that value's fp32 bits.
__device__ __forceinline__ float round_bf16(float y) {
  return __uint_as_float(pack_bf16(0.0f, y));
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
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

// Max of non-negative floats over aligned groups of G lanes, as unsigned
// integers (same order for non-negative IEEE values); the lane pairings are
// those of grp_sum.
template <int G>
__device__ __forceinline__ float grp_max(float f) {
  uint32_t v = __float_as_uint(f);
  if constexpr (G >= 2) v = max(v, dpp_u<0xB1>(v));
  if constexpr (G >= 4) v = max(v, dpp_u<0x4E>(v));
  if constexpr (G >= 8) v = max(v, dpp_u<0x141>(v));
  if constexpr (G >= 16) v = max(v, dpp_u<0x140>(v));
  if constexpr (G >= 32) v = max(v, (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F));
  if constexpr (G >= 64)
    v = max((uint32_t)__builtin_amdgcn_readlane((int)v, 0),
            (uint32_t)__builtin_amdgcn_readlane((int)v, 32));
  return __uint_as_float(v);
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
  uint32_t blk, pos;
  if (a.bs_log2 >= 0) {
    blk = s >> a.bs_log2;
    pos = s & ((1u << a.bs_log2) - 1u);
  } else {
    blk = (uint32_t)(((uint64_t)s * a.bs_magic) >> a.bs_shift);
    pos = s - blk * (uint32_t)a.block_size;
  }
  return base + (int64_t)blk * bstride + (int64_t)pos * pitch;
}

// Streamed inputs (read once) use nontemporal loads.
__device__ __forceinline__ uint4 ld16(const uint8_t *p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld8(const uint8_t *p) {
  const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t *>(p));
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint32_t ld4(const uint8_t *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p));
}
__device__ __forceinline__ uint32_t ld2(const uint8_t *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint16_t *>(p));
}
// gamma is shared by every row: a plain (cached) load.
__device__ __forceinline__ uint4 ld16_cached(const uint16_t *p) {
  return *reinterpret_cast<const uint4 *>(p);
}

// gamma in LDS as fp32, in two planes of L*C float4 (values 0-3 and 4-7 of
// each chunk), entry j*L + li holding the chunk lane li keeps in register j:
// every read is 16 contiguous bytes per lane.
template <int PLANE>
__device__ __forceinline__ void gamma8(const float4 *g_lds, int e, float (&g)[8]) {
  const float4 lo = g_lds[e];
  const float4 hi = g_lds[e + PLANE];
  g[0] = lo.x; g[1] = lo.y; g[2] = lo.z; g[3] = lo.w;
  g[4] = hi.x; g[5] = hi.y; g[6] = hi.z; g[7] = hi.w;
}

// the same for fp16 rows (XF16) or bf16 rows
template <bool XF16>
__device__ __forceinline__ void unpack8x(const uint4 w, float (&v)[8]);

__device__ __forceinline__ void unpack8(const uint4 w, float (&v)[8]) {
  v[0] = lo_f(w.x); v[1] = hi_f(w.x);
  v[2] = lo_f(w.y); v[3] = hi_f(w.y);
  v[4] = lo_f(w.z); v[5] = hi_f(w.z);
  v[6] = lo_f(w.w); v[7] = hi_f(w.w);
}

template <bool XF16>
__device__ __forceinline__ void unpack8x(const uint4 w, float (&v)[8]) {
  if constexpr (XF16) {
    v[0] = f16_lo(w.x); v[1] = f16_hi(w.x);
    v[2] = f16_lo(w.y); v[3] = f16_hi(w.y);
    v[4] = f16_lo(w.z); v[5] = f16_hi(w.z);
    v[6] = f16_lo(w.w); v[7] = f16_hi(w.w);
  } else {
    unpack8(w, v);
  }
}

// ------------------------------------------------------------------------
// the epilog kernel
// ------------------------------------------------------------------------

// Write sink for skipped tokens: their (discarded) row goes here instead of
// being branched around, so that every loop iteration issues the same
// stores.  Its contents are never read.  Half for the main row (at most
// 16256 bytes, a bf16 ckv row of d = 8192), half for the aux row, then 16
// bytes per lane for lanes with nothing to store.
constexpr int kSinkHalf = 16384;
__device__ __attribute__((aligned(256))) uint8_t g_sink[2 * kSinkHalf + 64 * 16];
enum { M_FP8_BF16 = 0, M_FP8_E8M0 = 1, M_MXFP4 = 3, M_SPLIT = 4, M_MXFP8 = 5, M_FP8_ROW = 6,
       M_FP4_NOPE = 7 /* quantMode 2's nope segment: FP4 codes, bf16 scales */,
       M_SPLIT_G = 8 /* the bf16 split with a rope segment of another length */ };
// the indexer modes quantise the whole row (no rope segment)
constexpr bool whole_row(int m) { return m == M_MXFP4 || m == M_MXFP8 || m == M_FP8_ROW; }
// modes writing a second cache (scales or the k rows)
constexpr bool has_aux(int m) { return m != M_FP8_BF16 && m != M_FP8_E8M0; }
// the rope segment: the last 64 columns, or (M_SPLIT_G) rope_dim columns;
// M_FP4_NOPE leaves the rope bytes of its rows alone and does not read them
constexpr bool fixed_rope(int m) { return !whole_row(m) && m != M_SPLIT_G && m != M_FP4_NOPE; }
// modes whose rows are assembled in LDS when the layout allows (FAST == 2)
constexpr bool staged_mode(int m) { return m == M_FP8_BF16 || m == M_FP4_NOPE; }
// Speculative rows (staged rows of mode 0 and of the FP4 nope mode after
// RMSNorm): the row is computed with the fast arithmetic only, while a flag
// records whether any input is outside the ranges where that arithmetic is
// exact; a wave-iteration with such a row computes its rows again with exact
// arithmetic (exact_row).  This keeps the checks off the branches of the
// common path.
constexpr bool spec_rows(int m, bool norm, int fast) {
  return staged_mode(m) && norm && fast == 2;
}
constexpr bool gen_rope(int m) { return m == M_SPLIT_G; }

// Rope work is split into 32 tasks: task tau = 16h + p produces outputs
// y[32h + 2p] and y[32h + 2p + 1] from the interleaved pairs 2p and 2p+1
// (x[4p..4p+3]) and cos/sin[32h + 2p .. +1]; its 4 output bytes sit at rope
// byte 4*tau, so the 32 tasks write the 128 rope bytes contiguously.
template <int L>
struct RopeShape {
  static constexpr int TPL = L >= 32 ? 1 : 32 / L;  // tasks per lane
  // rope segments of another length (M_SPLIT_G): one task per output pair
  // (y[p], y[p + Dk/2]), up to 64 pairs (Dk <= 128)
  static constexpr int TPG = (64 + L - 1) / L;
};

// Chunk layout: lane li of a row owns C chunks of 16 bytes (8 values),
// chunk li + L*j in register j.  Each load instruction then reads L*16
// contiguous bytes of the row, the L lanes of a register j cover an aligned
// block of the row (the RMSNorm tree and the quantisation groups stay
// lane-aligned) and a lane's codes of one chunk are contiguous.
template <int L>
__device__ __forceinline__ int chunk_of(int li, int j) {
  return li + L * j;
}

template <int MODE, bool ROPE, int L, int C>
struct RowBuf {
  static constexpr bool HAS_ROPE_SEG = fixed_rope(MODE);
  static constexpr int TPL = RopeShape<L>::TPL;
  static constexpr int TPG = gen_rope(MODE) ? RopeShape<L>::TPG : 1;
  uint4 xw[C];
  uint2 rx[HAS_ROPE_SEG ? TPL : 1];             // x[4p .. 4p+3] (or 2 copied values)
  uint32_t rc[HAS_ROPE_SEG && ROPE ? TPL : 1];  // cos pair
  uint32_t rs[HAS_ROPE_SEG && ROPE ? TPL : 1];  // sin pair
  uint32_t gx[TPG];  // M_SPLIT_G: x[2p], x[2p+1]
  uint32_t gc[TPG];  // cos[p] | cos[p + Dk/2] << 16
  uint32_t gs[TPG];  // sin[p] | sin[p + Dk/2] << 16
};

// Loads one row into registers.  xr, cr and sr are the wave-uniform bases of
// the first row loaded by the wave in this iteration (x, cos, sin); dr is the
// lane's row relative to it (0 for lanes of a skipped token, which read that
// first row again).  Every lane always issues the same loads (chunk indices
// beyond the row are clamped and their values cleared), so the number of
// memory operations per iteration is fixed -- see the pipeline in the kernel.
template <int MODE, bool NORM, bool ROPE, int L, int C, int FAST>
__device__ __forceinline__ void load_row(const KArgs &a, const uint8_t *xr, const uint8_t *cr,
                                         const uint8_t *sr, uint32_t dr, int li,
                                         RowBuf<MODE, ROPE, L, C> &b) {
  const uint32_t xo = dr * a.x_pitch;
#pragma unroll
  for (int j = 0; j < C; ++j) {
    const int c = chunk_of<L>(li, j);
    if constexpr (FAST) {
      b.xw[j] = ld16(xr + (xo + 16u * (uint32_t)c));
    } else {
      const uint4 v = ld16(xr + (xo + 16u * (uint32_t)min(c, a.nchunk - 1)));
      b.xw[j] = c < a.nchunk ? v : make_uint4(0, 0, 0, 0);
    }
  }
  if constexpr (RowBuf<MODE, ROPE, L, C>::HAS_ROPE_SEG) {
    constexpr int TPL = RowBuf<MODE, ROPE, L, C>::TPL;
    const uint32_t ro = xo + 2u * (uint32_t)a.nseg;
#pragma unroll
    for (int k = 0; k < TPL; ++k) {
      const int tau = (li + L * k) & 31;
      if constexpr (ROPE) {
        const int p = tau & 15;
        b.rx[k] = ld8(xr + (ro + 8u * (uint32_t)p));
        b.rc[k] = ld4(cr + (128u * dr + 4u * (uint32_t)tau));
        b.rs[k] = ld4(sr + (128u * dr + 4u * (uint32_t)tau));
      } else {
        b.rx[k] = make_uint2(ld4(xr + (ro + 4u * (uint32_t)tau)), 0u);
      }
    }
  }
  if constexpr (gen_rope(MODE)) {
    // task p (lanes past the last pair read pair 0 again)
    const uint32_t ro = xo + 2u * (uint32_t)a.nseg;
    const uint32_t half = (uint32_t)a.rope_half;
    const uint32_t cb = (uint32_t)a.rope_pitch * dr;
#pragma unroll
    for (int k = 0; k < RowBuf<MODE, ROPE, L, C>::TPG; ++k) {
      const uint32_t p0 = (uint32_t)(li + L * k);
      const uint32_t p = p0 < half ? p0 : 0u;
      b.gx[k] = ld4(xr + (ro + 4u * p));
      b.gc[k] = ld2(cr + (cb + 2u * p)) | (ld2(cr + (cb + 2u * (p + half))) << 16);
      b.gs[k] = ld2(sr + (cb + 2u * p)) | (ld2(sr + (cb + 2u * (p + half))) << 16);
    }
  }
}

// A computed row waiting to be stored: destination pointers, code words
// (or the bf16 ckv chunks), scale bits and rope words.
template <int MODE, int L, int C>
struct RowOut {
  uint8_t *p0, *p1;
  uint4 w[C];
  uint32_t sb[C];
  bool redo;  // (speculative rows) the fast arithmetic may be inexact here
  uint32_t ry[whole_row(MODE) ? 1 : (gen_rope(MODE) ? RopeShape<L>::TPG : RopeShape<L>::TPL)];
};

// E4M3 codes of v / 2^E (E the group's e8m0 exponent, -127..127) as two
// words of four codes.
__device__ __forceinline__ void codes_e8m0_fp8(const float (&v)[8], int E, uint32_t (&cw)[2]) {
  if (E >= -100 && E <= 100) {
    const float sc = __uint_as_float((uint32_t)(E + 127) << 23);
    s16x2_t w0 = {0, 0}, w1 = {0, 0};
    w0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w0, v[0], v[1], sc, false);
    w0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w0, v[2], v[3], sc, true);
    w1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w1, v[4], v[5], sc, false);
    w1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w1, v[6], v[7], sc, true);
    cw[0] = __builtin_bit_cast(uint32_t, w0);
    cw[1] = __builtin_bit_cast(uint32_t, w1);
  } else {
    const float f = exp2_neg(E);
    uint32_t q[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) q[t] = enc_e4m3_sw(v[t] * f);
    cw[0] = q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24);
    cw[1] = q[4] | (q[5] << 8) | (q[6] << 16) | (q[7] << 24);
  }
}

// E4M3 codes of eight quotients, each of magnitude at most 456 or NaN (the
// hardware convert rounds to nearest even and, below 464, saturates to 448;
// tests/hw_check.hip).
__device__ __forceinline__ void codes_fp8(const float (&q)[8], uint32_t (&cw)[2]) {
  // (any initial words: the two converts of each fill both halves)
  int w0 = __builtin_bit_cast(int, q[0]), w1 = __builtin_bit_cast(int, q[4]);
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], w0, false);
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], w0, true);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(q[4], q[5], w1, false);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(q[6], q[7], w1, true);
  cw[0] = (uint32_t)w0;
  cw[1] = (uint32_t)w1;
}

// E4M3 codes of eight values q_i / sc, sc a power of two in [2^-100, 2^100]
// (v_cvt_scalef32_pk_fp8_f32 takes the exponent of sc); every |q_i / sc| at
// most 456 (tests/hw_check.hip checks the convert for fp32 inputs against the
// software encoder of the scaled value).
__device__ __forceinline__ void codes_fp8_scaled(const float (&q)[8], float sc,
                                                 uint32_t (&cw)[2]) {
  s16x2_t w0 = {0, 0}, w1 = {0, 0};
  w0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w0, q[0], q[1], sc, false);
  w0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w0, q[2], q[3], sc, true);
  w1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w1, q[4], q[5], sc, false);
  w1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w1, q[6], q[7], sc, true);
  cw[0] = __builtin_bit_cast(uint32_t, w0);
  cw[1] = __builtin_bit_cast(uint32_t, w1);
}

// Reciprocals of the 128 significands of bf16 scales, kept in LDS by the
// staged instances: entry k holds, for m = 1 + k/128, rs = 1/m rounded
// downwards and rl = RN((1 - m rs) rs), the double-length reciprocal the
// quotient v / m = fma(v, rs, v rl) takes.  They are computed at block start
// with the very arithmetic the per-group path uses (rcp_rn, then one step
// down when it rounded up).  A scale s = m 2^e then divides as v / m with the
// convert scaled by 2^e: v / s and (v / m) 2^-e are the same fp32 value
// wherever it is normal, and below that every code is +-0.
__device__ __forceinline__ float2 recip_entry(int k) {
  const float m = 1.0f + (float)k * 0x1p-7f;
  float rs = rcp_rn(m);
  if (__builtin_fmaf(-m, rs, 1.0f) < 0.0f) rs = __uint_as_float(__float_as_uint(rs) - 1u);
  return make_float2(rs, __builtin_fmaf(-m, rs, 1.0f) * rs);
}

// The table sits at the start of the block's dynamic LDS (every extern
// shared array names that same start).
__device__ __forceinline__ const float2 *recip_table() {
  extern __shared__ float2 kvepi_recip_lds[];
  return kvepi_recip_lds;
}
constexpr int RECIP_BYTES = 128 * 8;

// the table entry of a positive normal bf16-valued scale su, and 2^e(su)
__device__ __forceinline__ float2 recip_of(float su, float &pow2) {
  const uint32_t sb = __float_as_uint(su);
  pow2 = __uint_as_float(sb & 0x7F800000u);
  return recip_table()[__builtin_amdgcn_ubfe(sb, 16, 7)];
}

// m / 448 correctly rounded for a bf16 m in [2^-71, 2^100]: fma(m, H, m*Lo)
// with H + Lo a double-length 1/448 (tests/fastdiv_check.c compares it with
// the IEEE quotient for every such m).
__device__ __forceinline__ float div448_fast(float m) {
  constexpr float H448 = 1.0f / 448.0f;
  constexpr float L448 = (float)(1.0 / 448.0 - (double)H448);
  return __builtin_fmaf(m, H448, m * L448);
}

// Mode 0 codes of one group of 8 values per lane (v, group maximum m);
// returns the stored bf16 scale bits.  The scale is amax / 448 (IEEE),
// stored as bf16, and the codes divide by the stored value.
// fast (callers pass m in [2^-71, 2^100], which keeps m / 448 and the
// stored scale inside the range of the fast division and reciprocal):
// m / 448 = fma(m, H, m * Lo) with H + Lo a double-length 1/448, and v / su =
// fma(v, rs, v * rl) with rs + rl a double-length 1/su: both are exactly the
// IEEE quotient for bf16 operands (their distance to a rounding boundary is
// far above the error), except that v / su below 2^-100 may differ -- where
// every code is +-0.  rs is rounded downwards so that rl >= 0 and a zero v
// keeps its sign.  Otherwise the group divides exactly (an infinite scale,
// from an infinite RMSNorm output, gives +-0 for finite values and the NaN
// code for inf / inf).
// The exact codes of a chunk of 8 bf16 values (packed in w) divided by su:
// IEEE division and the software encoder, rolled over the four words (the
// rare branch: little code, few registers).  Code byte i is value i's.
__device__ __forceinline__ void codes_fp8_exact(uint4 w, float su, uint32_t (&cw)[2]) {
  uint32_t c0 = 0, c1 = 0;
#pragma unroll 1
  for (int q = 0; q < 4; ++q) {
    const uint32_t e0 = su > 0.0f ? enc_e4m3_sw(lo_f(w.x) / su) : 0u;
    const uint32_t e1 = su > 0.0f ? enc_e4m3_sw(hi_f(w.x) / su) : 0u;
    c0 = (c0 >> 16) | (c1 << 16);
    c1 = (c1 >> 16) | ((e0 | (e1 << 8)) << 16);
    w = make_uint4(w.y, w.z, w.w, w.x);
  }
  cw[0] = c0;
  cw[1] = c1;
}

// TBL (staged instances): rs and rl of the scale's significand from the LDS
// table, the exponent applied by the scaled convert.
template <bool TBL = false>
__device__ __forceinline__ uint32_t codes_fp8_bf16scale(const float (&v)[8], float m, bool fast,
                                                        uint32_t (&cw)[2],
                                                        uint4 packed = make_uint4(0, 0, 0, 0),
                                                        bool rolled = false) {
  const float su = round_bf16(fast ? div448_fast(m) : m / 448.0f);
  if (rolled && !fast) {
    codes_fp8_exact(packed, su, cw);
  } else if (TBL && fast) {
    float sc;
    const float2 r = recip_of(su, sc);
    float qv[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) qv[t] = __builtin_fmaf(v[t], r.x, v[t] * r.y);
    codes_fp8_scaled(qv, sc, cw);
  } else if (fast) {
    float rs = rcp_rn(su);
    if (__builtin_fmaf(-su, rs, 1.0f) < 0.0f) rs = __uint_as_float(__float_as_uint(rs) - 1u);
    const float rl = __builtin_fmaf(-su, rs, 1.0f) * rs;
    float qv[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) qv[t] = __builtin_fmaf(v[t], rs, v[t] * rl);
    codes_fp8(qv, cw);
  } else {
    uint32_t q[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) q[t] = su > 0.0f ? enc_e4m3_sw(v[t] / su) : 0u;
    cw[0] = q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24);
    cw[1] = q[4] | (q[5] << 8) | (q[6] << 16) | (q[7] << 24);
  }
  return __float_as_uint(su) >> 16;
}

// m / 6 correctly rounded for a bf16 m in [2^-90, 2^100]: fma(m, H, m*Lo)
// with H + Lo a double-length 1/6 (tests/fastdiv_check.c compares it with the
// IEEE quotient for every such m).
__device__ __forceinline__ float div6_fast(float m) {
  constexpr float H6 = 1.0f / 6.0f;
  constexpr float L6 = (float)(1.0 / 6.0 - (double)H6);
  return __builtin_fmaf(m, H6, m * L6);
}

// Max of non-negative floats over aligned groups of 2^k lanes, k in 1..3
// (wave-uniform); pairings as in grp_max.
__device__ __forceinline__ float grp_max_k(float f, int k) {
  uint32_t v = __float_as_uint(f);
  v = max(v, dpp_u<0xB1>(v));
  if (k >= 2) v = max(v, dpp_u<0x4E>(v));
  if (k >= 3) v = max(v, dpp_u<0x141>(v));
  return __uint_as_float(v);
}

// FP4 nope codes of one chunk of 8 values (v, group maximum m): the scale is
// amax / 6 (IEEE), stored as bf16, and the codes are E2M1(v / s) with the
// stored s; returns the bf16 scale bits and the 8 codes as one word (value 2i
// in the low nibble of byte i).
// fast (m in [2^-90, 2^100]): m / 6 from a double-length 1/6, v / s from a
// double-length reciprocal rounded downwards (both exactly the IEEE quotient
// for bf16 operands wherever a code can be nonzero, as in mode 0), codes from
// v_cvt_scalef32_pk_fp4_f32 with scale 1, which rounds every fp32 quotient up
// to 6.0625 to nearest even and saturates at 6 (tests/hw_check.hip); the
// quotients stay below 6 / (1 - 2^-8).  Otherwise the group divides exactly
// and encodes in software (a zero group: scale 0 and codes 0).
// TBL (staged instances): the significand's reciprocal from the LDS table and
// the scale's exponent applied by the convert, as in mode 0.
template <bool TBL = false>
__device__ __forceinline__ uint32_t codes_fp4_bf16scale(const float (&v)[8], float m, bool fast,
                                                        uint32_t &w) {
  const float su = round_bf16(fast ? div6_fast(m) : m / 6.0f);
  if (TBL && fast) {
    float sc;
    const float2 r = recip_of(su, sc);
    float q[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) q[t] = __builtin_fmaf(v[t], r.x, v[t] * r.y);
    uint32_t x = 0;
    x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, q[0], q[1], sc, 0);
    x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, q[2], q[3], sc, 1);
    x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, q[4], q[5], sc, 2);
    x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, q[6], q[7], sc, 3);
    w = x;
  } else if (fast) {
    float rs = rcp_rn(su);
    if (__builtin_fmaf(-su, rs, 1.0f) < 0.0f) rs = __uint_as_float(__float_as_uint(rs) - 1u);
    const float rl = __builtin_fmaf(-su, rs, 1.0f) * rs;
    float q[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) q[t] = __builtin_fmaf(v[t], rs, v[t] * rl);
    uint32_t x = 0;
    x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, q[0], q[1], 1.0f, 0);
    x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, q[2], q[3], 1.0f, 1);
    x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, q[4], q[5], 1.0f, 2);
    x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, q[6], q[7], 1.0f, 3);
    w = x;
  } else {
    uint32_t x = 0;
#pragma unroll
    for (int t = 0; t < 8; ++t) x |= (su > 0.0f ? enc_e2m1_sw(v[t] / su) : 0u) << (4 * t);
    w = x;
  }
  return __float_as_uint(su) >> 16;
}

template <int MODE, bool NORM, bool ROPE, int L, int C, int FAST, bool XF16>
__device__ __forceinline__ void compute_row(const KArgs &a, int li, int sub,
                                            const RowBuf<MODE, ROPE, L, C> &b,
                                            const float4 *g_lds, RowOut<MODE, L, C> &o) {
  // ---- RMSNorm -> packed bf16 yw ----
  // Speculative rows only quantise the normalised values, so they keep them
  // as fp32 holding the bf16-rounded value (one convert per value) instead of
  // packing pairs and unpacking them again.
  constexpr bool DIRECT = spec_rows(MODE, NORM, FAST);
  uint4 yw[C];
  float yf[DIRECT ? C : 1][8];
  if constexpr (NORM) {
    float s8[C];
    float mn = __builtin_inff();  // smallest magnitude of the lane's values
#pragma unroll
    for (int j = 0; j < C; ++j) {
      float v[8];
      unpack8(b.xw[j], v);
      // the square of a bf16 value with |v| >= 2^-67 is exact, so then
      // fma(b, b, a*a) is the rounded sum of the two rounded squares
      const float s01 = __builtin_fmaf(v[1], v[1], v[0] * v[0]);
      const float s23 = __builtin_fmaf(v[3], v[3], v[2] * v[2]);
      const float s45 = __builtin_fmaf(v[5], v[5], v[4] * v[4]);
      const float s67 = __builtin_fmaf(v[7], v[7], v[6] * v[6]);
      s8[j] = (s01 + s23) + (s45 + s67);
      const int c = chunk_of<L>(li, j);
      if (FAST || c < a.nchunk) {
#pragma unroll
        for (int q = 0; q < 8; ++q) mn = __builtin_fminf(mn, __builtin_fabsf(v[q]));
      }
    }
    // tree: the 8 values of a chunk, then the L lanes (butterfly), then the
    // C blocks of L chunks
    float part[C];
#pragma unroll
    for (int j = 0; j < C; ++j) part[j] = grp_sum<L>(s8[j]);
#pragma unroll
    for (int w = 1; w < C; w *= 2)
#pragma unroll
      for (int j = 0; j < C; j += 2 * w) part[j] = part[j] + part[j + w];
    float ss = part[0];
    constexpr bool SPEC = spec_rows(MODE, NORM, FAST);
    // A smaller magnitude (zeros included, which costs nothing) can have a
    // square that underflows and rounds, and the fused sum above would then
    // round once where the definition rounds the square first: such waves,
    // rare, sum the separately rounded squares.
    // (The rare branches below run as rolled loops over the words of a
    // chunk, rotating the words through one register set, so that they add
    // little code and few registers to the common path.)
    if (!SPEC && __builtin_amdgcn_ballot_w64(mn < 0x1p-67f) != 0) {
#pragma unroll
      for (int j = 0; j < C; ++j) {
        uint4 w = b.xw[j];
        float pr[4];  // pair sums (x[2q]^2 + x[2q+1]^2), each square rounded
#pragma unroll 1
        for (int q = 0; q < 4; ++q) {
          const float v0 = lo_f(w.x), v1 = hi_f(w.x);
          const float p2 = v0 * v0 + v1 * v1;
          w = make_uint4(w.y, w.z, w.w, __float_as_uint(p2));
        }
        pr[0] = __uint_as_float(w.x);
        pr[1] = __uint_as_float(w.y);
        pr[2] = __uint_as_float(w.z);
        pr[3] = __uint_as_float(w.w);
        s8[j] = (pr[0] + pr[1]) + (pr[2] + pr[3]);
      }
#pragma unroll
      for (int j = 0; j < C; ++j) part[j] = grp_sum<L>(s8[j]);
#pragma unroll
      for (int w = 1; w < C; w *= 2)
#pragma unroll
        for (int j = 0; j < C; j += 2 * w) part[j] = part[j] + part[j + w];
      ss = part[0];
    }
    const float mean = a.inv_nseg != 0.0f ? ss * a.inv_nseg : ss / a.nseg_f;
    const float xs = mean + a.eps;
    // (a wave-uniform choice, so only one of the two square roots runs)
    const bool xs_ok = xs >= 0x1p-96f && xs <= 0x1p+127f;
    const float rms = SPEC || __builtin_amdgcn_ballot_w64(!xs_ok) == 0 ? sqrt_rn(xs)
                                                                     : __builtin_sqrtf(xs);
    // The fast division needs a normal rms with a normal reciprocal, every
    // quotient normal (|x| >= 2^(e(rms) - 252) guarantees it) and an exact
    // FMA residual (|x| >= 2^-100).  Rows holding a smaller magnitude --
    // including an exact zero -- divide exactly instead.
    const int re = (int)(__float_as_uint(rms) >> 23);
    const int k = re - 252 > -100 ? re - 252 : -100;
    const float thr = __uint_as_float((uint32_t)(k + 127) << 23);  // 2^k
    const bool tiny = mn < thr;
    bool fast = re >= 127 - 100 && re <= 127 + 100;
    if constexpr (SPEC) {
      // checks the fast branches need, answered after the row is done
      o.redo = mn < 0x1p-67f || tiny || !xs_ok || !fast;
      fast = true;
    } else if constexpr (L == 64) {
      fast = fast && __builtin_amdgcn_ballot_w64(tiny) == 0;
    } else {
      const uint64_t bal = __builtin_amdgcn_ballot_w64(tiny);
      fast = fast && ((bal >> (sub * L)) & ((1ull << L) - 1)) == 0;
    }
    if (fast) {
      const float rcp = rcp_rn(rms);
#pragma unroll
      for (int j = 0; j < C; ++j) {
        float v[8], g[8], y[8];
        unpack8(b.xw[j], v);
        gamma8<L * C>(g_lds, j * L + li, g);
#pragma unroll
        for (int q = 0; q < 8; ++q) y[q] = div_fast(v[q], rms, rcp) * g[q];
        if constexpr (DIRECT) {
#pragma unroll
          for (int q = 0; q < 8; ++q) yf[j][q] = round_bf16(y[q]);
        } else {
          yw[j] = make_uint4(pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3]), pack_bf16(y[4], y[5]),
                             pack_bf16(y[6], y[7]));
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < C; ++j) {
        uint4 w = b.xw[j];
        const float *gp = reinterpret_cast<const float *>(g_lds + (j * L + li));
#pragma unroll 1
        for (int q = 0; q < 4; ++q) {
          // values 2q, 2q+1: gamma plane q / 2, entries 2 (q % 2) + {0, 1}
          const float *gq = gp + (q >> 1) * 4 * (L * C) + 2 * (q & 1);
          const float y0 = (lo_f(w.x) / rms) * gq[0];
          const float y1 = (hi_f(w.x) / rms) * gq[1];
          w = make_uint4(w.y, w.z, w.w, pack_bf16(y0, y1));
        }
        yw[j] = w;
        if constexpr (DIRECT) unpack8(w, yf[j]);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < C; ++j) yw[j] = b.xw[j];
  }

  // ---- RoPE: 4 output bytes per task ----
  constexpr int TPL = RopeShape<L>::TPL;
  uint32_t ry[RowBuf<MODE, ROPE, L, C>::HAS_ROPE_SEG ? TPL : 1];
  if constexpr (RowBuf<MODE, ROPE, L, C>::HAS_ROPE_SEG) {
#pragma unroll
    for (int k = 0; k < TPL; ++k) {
      const int tau = (li + L * k) & 31;  // lanes past 31 repeat tasks 0..31
      if constexpr (ROPE) {
        const bool hi = tau >= 16;
        const float a0 = lo_f(b.rx[k].x), b0 = hi_f(b.rx[k].x);
        const float a1 = lo_f(b.rx[k].y), b1 = hi_f(b.rx[k].y);
        const float c0 = lo_f(b.rc[k]), c1 = hi_f(b.rc[k]);
        const float s0 = lo_f(b.rs[k]), s1 = hi_f(b.rs[k]);
        // first half: a*c - b*s; second half: b*c + a*s.  Each product is
        // rounded on its own, as the definition has it: a product of two
        // bf16 values is exact unless it underflows, and there a fused
        // multiply-add would round once where the definition rounds twice.
        const float p0 = hi ? b0 : a0, q0 = hi ? a0 : -b0;
        const float p1 = hi ? b1 : a1, q1 = hi ? a1 : -b1;
        ry[k] = pack_bf16(p0 * c0 + q0 * s0, p1 * c1 + q1 * s1);
      } else {
        ry[k] = b.rx[k].x;
      }
    }
  }

  // ---- outputs (kept in registers; stored by store_row) ----
  if constexpr (MODE == M_SPLIT) {
#pragma unroll
    for (int j = 0; j < C; ++j) o.w[j] = yw[j];
#pragma unroll
    for (int k = 0; k < TPL; ++k) o.ry[k] = ry[k];
  } else if constexpr (MODE == M_SPLIT_G) {
#pragma unroll
    for (int j = 0; j < C; ++j) o.w[j] = yw[j];
    // y[p] = a c[p] - b s[p], y[p + Dk/2] = b c[p + Dk/2] + a s[p + Dk/2],
    // each product rounded on its own (as above)
#pragma unroll
    for (int k = 0; k < RowBuf<MODE, ROPE, L, C>::TPG; ++k) {
      const float xa = lo_f(b.gx[k]), xb = hi_f(b.gx[k]);
      const float c0 = lo_f(b.gc[k]), c1 = hi_f(b.gc[k]);
      const float s0 = lo_f(b.gs[k]), s1 = hi_f(b.gs[k]);
      o.ry[k] = pack_bf16(xa * c0 + -xb * s0, xb * c1 + xa * s1);
    }
  } else if constexpr (MODE == M_FP4_NOPE) {
    // "aclnnKvCompressEpilog" quantMode 2, nope segment: groups of 16, 32 or
    // 64 values (2, 4 or 8 lanes), scale amax / 6 as bf16, E2M1 codes
#pragma unroll
    for (int j = 0; j < C; ++j) {
      float v[8];
      if constexpr (DIRECT) {
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = yf[j][q];
      } else {
        unpack8(yw[j], v);
      }
      const float m = grp_max_k(amax8(v), a.glog);
      const bool fast = m >= 0x1p-90f && m <= 0x1p+100f;
      uint32_t w;
      if constexpr (spec_rows(MODE, NORM, FAST)) {
        o.redo = o.redo || !fast;
        o.sb[j] = codes_fp4_bf16scale<true>(v, m, true, w);
      } else {
        o.sb[j] = codes_fp4_bf16scale<FAST == 2>(v, m, fast, w);
      }
      o.w[j] = make_uint4(w, 0u, 0u, 0u);
    }
  } else if constexpr (MODE == M_MXFP4) {
#pragma unroll
    for (int j = 0; j < C; ++j) {
      float v[8];
      unpack8x<XF16>(yw[j], v);
      float m = amax8(v);
      m = grp_max<4>(m);  // 32 values = 4 lanes
      const int E = e8m0_exp<2, 0x400000u>(m);  // FP4 max 6 = 1.5 * 2^2
      uint32_t w = 0;
      if (E >= -100 && E <= 100) {
        const float sc = __uint_as_float((uint32_t)(E + 127) << 23);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0], v[1], sc, 0);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], sc, 1);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], sc, 2);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], sc, 3);
      } else {
        const float f = exp2_neg(E);
#pragma unroll
        for (int q = 0; q < 8; ++q) w |= enc_e2m1_sw(v[q] * f) << (4 * q);
      }
      o.w[j] = make_uint4(w, 0u, 0u, 0u);
      o.sb[j] = (uint32_t)(E + 127);
    }
  } else if constexpr (MODE == M_MXFP8) {
    // "indexer_quant_cache" mxfp8: e8m0 scale per group of 32, E4M3 codes
#pragma unroll
    for (int j = 0; j < C; ++j) {
      float v[8];
      unpack8x<XF16>(yw[j], v);
      const float m = grp_max<4>(amax8(v));  // 32 values = 4 lanes
      const int E = e8m0_exp<8, 0x600000u>(m);  // FP8 max 448 = 1.75 * 2^8
      uint32_t cw[2];
      codes_e8m0_fp8(v, E, cw);
      o.w[j] = make_uint4(cw[0], cw[1], 0u, 0u);
      o.sb[j] = (uint32_t)(E + 127);
    }
  } else if constexpr (MODE == M_FP8_ROW) {
    // "indexer_quant_cache" fp8: the whole row is one group; its scale
    // amax / 448 is kept in fp32 and the codes divide by it.  The fast path
    // (amax in [2^-71, 2^100], so that the scale and its reciprocal are
    // normal and inside the range of rcp_rn) divides with div_fast, exact
    // for bf16 numerators wherever a code can be nonzero; elsewhere the row
    // divides exactly (a zero row has scale 0 and all codes 0).
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < C; ++j) {
      float v[8];
      unpack8x<XF16>(yw[j], v);
      m = __builtin_fmaxf(m, amax8(v));
    }
    m = grp_max<L>(m);
    const bool fastq = m >= 0x1p-71f && m <= 0x1p+100f;
    const float s = fastq ? div448_fast(m) : m / 448.0f;
    const float rcp = rcp_rn(s);
#pragma unroll
    for (int j = 0; j < C; ++j) {
      float v[8];
      unpack8x<XF16>(yw[j], v);
      uint32_t cw[2];
      if (fastq) {
        float q[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) q[t] = div_fast(v[t], s, rcp);
        codes_fp8(q, cw);
      } else {
        uint32_t q[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) q[t] = s > 0.0f ? enc_e4m3_sw(v[t] / s) : 0u;
        cw[0] = q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24);
        cw[1] = q[4] | (q[5] << 8) | (q[6] << 16) | (q[7] << 24);
      }
      o.w[j] = make_uint4(cw[0], cw[1], 0u, 0u);
    }
    o.sb[0] = __float_as_uint(s);
  } else if constexpr (MODE == M_FP8_E8M0) {
#pragma unroll
    for (int j = 0; j < C; ++j) {
      float v[8];
      unpack8(yw[j], v);
      const float m = grp_max<8>(amax8(v));  // 64 values = 8 lanes
      const int E = e8m0_exp<8, 0x600000u>(m);  // FP8 max 448 = 1.75 * 2^8
      uint32_t cw[2];
      codes_e8m0_fp8(v, E, cw);
      o.w[j] = make_uint4(cw[0], cw[1], 0u, 0u);
      o.sb[j] = (uint32_t)(E + 127);
    }
#pragma unroll
    for (int k = 0; k < TPL; ++k) o.ry[k] = ry[k];
  } else {  // M_FP8_BF16
    // After an RMSNorm the chunks go in pairs: the two group maxima reduce
    // together and the fast-path choice is made once for the wave, so the
    // common case runs as one straight block (measured faster; without
    // RMSNorm the same form costs registers, and each lane chooses alone).
    constexpr int NB = (NORM && C >= 2) ? 2 : 1;
#pragma unroll
    for (int j0 = 0; j0 < C; j0 += NB) {
      float vv[NB][8], mm[NB];
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        if constexpr (DIRECT) {
#pragma unroll
          for (int q = 0; q < 8; ++q) vv[i][q] = yf[j0 + i][q];
        } else {
          unpack8(yw[j0 + i], vv[i]);
        }
        mm[i] = amax8(vv[i]);
      }
#pragma unroll
      for (int i = 0; i < NB; ++i) mm[i] = grp_max<8>(mm[i]);  // 64 values = 8 lanes
      bool inr[NB], all = true;
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        inr[i] = mm[i] >= 0x1p-71f && mm[i] <= 0x1p+100f;
        all = all && inr[i];
      }
      uint32_t cw[NB][2];
      if constexpr (spec_rows(MODE, NORM, FAST)) {
        o.redo = o.redo || !all;
#pragma unroll
        for (int i = 0; i < NB; ++i) o.sb[j0 + i] = codes_fp8_bf16scale<FAST == 2>(vv[i], mm[i], true, cw[i]);
      } else if (NORM && __builtin_amdgcn_ballot_w64(!all) == 0) {
#pragma unroll
        for (int i = 0; i < NB; ++i) o.sb[j0 + i] = codes_fp8_bf16scale<FAST == 2>(vv[i], mm[i], true, cw[i]);
      } else {
#pragma unroll
        for (int i = 0; i < NB; ++i)
          o.sb[j0 + i] = codes_fp8_bf16scale<FAST == 2>(vv[i], mm[i], inr[i], cw[i], yw[j0 + i], true);
      }
#pragma unroll
      for (int i = 0; i < NB; ++i) o.w[j0 + i] = make_uint4(cw[i][0], cw[i][1], 0u, 0u);
    }
#pragma unroll
    for (int k = 0; k < TPL; ++k) o.ry[k] = ry[k];
  }
}

// Exact arithmetic for a speculative row (mode 0 or the FP4 nope mode after
// RMSNorm): the sum of separately rounded squares, the library square root,
// IEEE division by rms, then per group the scale amax / 448 (amax / 6) by
// IEEE division and the codes of the exact quotients -- the definitions
// themselves, for rows holding inputs outside the ranges of the fast
// arithmetic.  Rewrites the codes and scales of o (mode 0's rope words are
// unchanged).  Rolled loops where they matter: rare, little code.
template <int MODE, int L, int C>
__device__ __forceinline__ void exact_row(const KArgs &a, int li, const uint4 (&xw)[C],
                                          const float4 *g_lds, RowOut<MODE, L, C> &o) {
  float part[C];
#pragma unroll
  for (int j = 0; j < C; ++j) {
    uint4 w = xw[j];
#pragma unroll 1
    for (int q = 0; q < 4; ++q) {
      const float v0 = lo_f(w.x), v1 = hi_f(w.x);
      w = make_uint4(w.y, w.z, w.w, __float_as_uint(v0 * v0 + v1 * v1));
    }
    const float s8 = (__uint_as_float(w.x) + __uint_as_float(w.y)) +
                     (__uint_as_float(w.z) + __uint_as_float(w.w));
    part[j] = grp_sum<L>(s8);
  }
#pragma unroll
  for (int w = 1; w < C; w *= 2)
#pragma unroll
    for (int j = 0; j < C; j += 2 * w) part[j] = part[j] + part[j + w];
  const float mean = a.inv_nseg != 0.0f ? part[0] * a.inv_nseg : part[0] / a.nseg_f;
  const float rms = __builtin_sqrtf(mean + a.eps);
#pragma unroll
  for (int j = 0; j < C; ++j) {
    uint4 w = xw[j];
    const float *gp = reinterpret_cast<const float *>(g_lds + (j * L + li));
#pragma unroll 1
    for (int q = 0; q < 4; ++q) {
      const float *gq = gp + (q >> 1) * 4 * (L * C) + 2 * (q & 1);
      const float y0 = (lo_f(w.x) / rms) * gq[0];
      const float y1 = (hi_f(w.x) / rms) * gq[1];
      w = make_uint4(w.y, w.z, w.w, pack_bf16(y0, y1));
    }
    float v[8];
    unpack8(w, v);
    if constexpr (MODE == M_FP4_NOPE) {
      const float m = grp_max_k(amax8(v), a.glog);
      uint32_t cw;
      o.sb[j] = codes_fp4_bf16scale<false>(v, m, false, cw);
      o.w[j] = make_uint4(cw, 0u, 0u, 0u);
    } else {
      const float m = grp_max<8>(amax8(v));  // 64 values = 8 lanes
      const float su = round_bf16(m / 448.0f);
      uint32_t cw[2];
      codes_fp8_exact(w, su, cw);
      o.w[j] = make_uint4(cw[0], cw[1], 0u, 0u);
      o.sb[j] = __float_as_uint(su) >> 16;
    }
  }
}

// FAST == 2 (mode 0, one or two rows per wave-iteration): each row is
// assembled in LDS and leaves as one store of 16-byte pieces, lane i storing
// piece i mod (kvCacheCol / 16) (lanes past the last piece repeat earlier
// ones: same bytes, same address).  This replaces the many narrow stores of
// a row (codes, scales, rope, pad) by one wide store per row.
// The largest mode-0 row of a layout of L lanes x C chunks: nope codes,
// rope, bf16 scales, padded to 32 bytes.
constexpr int max_row_bytes(int L, int C) {
  return ((8 * L * C + 128 + 2 * ((8 * L * C + 63) / 64) + 31) / 32) * 32;
}

// FAST == 2: writes the computed row into the wave's staging area (its own
// image at stage + sub * img_bytes).  Mode 0: codes, rope and scales; the FP4
// nope mode: codes and scales (its image starts after the row's 64 rope
// bytes).  The zero pad after the scales was written once when the wave
// started (every row writes the same fields, so the pad bytes are never
// overwritten).
template <int MODE, int L, int C>
__device__ __forceinline__ void stage_write(const KArgs &a, int li, int sub,
                                            const RowOut<MODE, L, C> &o, uint8_t *stage) {
  static_assert(staged_mode(MODE) && L >= 32, "staged rows: mode 0 and the FP4 nope mode");
  uint8_t *img = stage + sub * a.img_bytes;
  if constexpr (MODE == M_FP4_NOPE) {
#pragma unroll
    for (int j = 0; j < C; ++j) {
      const int c = li + L * j;
      *reinterpret_cast<uint32_t *>(img + 4 * c) = o.w[j].x;
      *reinterpret_cast<uint16_t *>(img + a.nseg / 2 + 2 * (c >> a.glog)) = (uint16_t)o.sb[j];
    }
  } else {
    constexpr int TPL = RopeShape<L>::TPL;
#pragma unroll
    for (int j = 0; j < C; ++j) {
      const int c = li + L * j;
      *reinterpret_cast<uint2 *>(img + 8 * c) = make_uint2(o.w[j].x, o.w[j].y);
    }
    const int tail = a.nseg + 128;
#pragma unroll
    for (int j = 0; j < C; ++j) {
      const int c = li + L * j;
      *reinterpret_cast<uint16_t *>(img + tail + 2 * (c >> 3)) = (uint16_t)o.sb[j];
    }
#pragma unroll
    for (int k = 0; k < TPL; ++k)
      *reinterpret_cast<uint32_t *>(img + a.nseg + 4 * ((li + L * k) & 31)) = o.ry[k];
  }
}

// Orders a wave's LDS accesses across its lanes: the writes (reads) of one
// lane before the reads (writes) of another that follow in program order.
__device__ __forceinline__ void lds_handover() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// FAST == 2: stores the staged rows of a wave-iteration, one instruction per
// row, 16 bytes per lane; dst[r] is where row r's image goes (wave-uniform),
// off the lane's piece offset, img the bytes per image.  (Destinations are
// pointers derived from the cache or the sink, never integers, so that the
// stores stay global ones.)
template <int R>
__device__ __forceinline__ void stage_store(const uint8_t *stage, int img, uint32_t off,
                                            uint8_t *const (&dst)[R]) {
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint4 v = *reinterpret_cast<const uint4 *>(stage + r * img + off);
    // a global-memory pointer (an integer cast would otherwise give a flat
    // store, which also counts against the LDS counter)
    *reinterpret_cast<uint4 *>(dst[r] + off) = v;
  }
}

// Zero padding of a row from concatCol to kvCacheCol (0..31 bytes): one store
// per lane, duplicates allowed (lanes with nothing to write use the sink).
template <int L>
__device__ __forceinline__ void store_pad(const KArgs &a, int li, uint8_t *lsink, uint8_t *row) {
  const int npad = a.kv_cache_col - a.concat_col;
  if (a.pad16 == 1) {
    *reinterpret_cast<uint4 *>(row + a.concat_col) = make_uint4(0, 0, 0, 0);
  } else {
    constexpr int PADIT = (31 + L - 1) / L;  // enough stores for 31 bytes
#pragma unroll
    for (int k = 0; k < PADIT; ++k) {
      const int b = li + L * k;
      st_u8(npad > 0 ? row + a.concat_col + (b < npad ? b : b % max(npad, 1)) : lsink + 12, 0u);
    }
  }
}

// Stores one computed row: exactly kvCacheCol bytes (plus the aux row).
// Every lane issues every store, so that the number of memory operations per
// iteration is fixed: lanes that carry a copy of a value another lane writes
// (the group scale, the pad, duplicated rope tasks) write the same bytes to
// the same address, and lanes with nothing to write (chunks past the row)
// write to a private slot of the sink.
template <int MODE, bool ROPE, int L, int C, int FAST>
__device__ __forceinline__ void store_row(const KArgs &a, int li, int lane,
                                          const RowOut<MODE, L, C> &o) {
  constexpr int TPL = RopeShape<L>::TPL;
  // in FAST mode every row start is 16-byte aligned (k rows 4-byte aligned):
  // the alignment is a constant and the store helpers reduce to one store
  const int c_al = FAST ? 16 : a.c_align;
  const int a_al = FAST ? 4 : a.a_align;
  uint8_t *lsink = g_sink + 2 * kSinkHalf + 16 * lane;
  if constexpr (MODE == M_SPLIT_G) {
#pragma unroll
    for (int j = 0; j < C; ++j) {
      const int c = chunk_of<L>(li, j);
      st_u128((FAST || c < a.nchunk) ? o.p0 + 16 * c : lsink, o.w[j], c_al);
    }
    const int half = a.rope_half;
#pragma unroll
    for (int k = 0; k < RowBuf<MODE, ROPE, L, C>::TPG; ++k) {
      const int p = li + L * k;
      const bool in = p < half;
      st_u16(in ? o.p1 + 2 * p : lsink + 4, o.ry[k], 2);
      st_u16(in ? o.p1 + 2 * (p + half) : lsink + 6, o.ry[k] >> 16, 2);
    }
  } else if constexpr (MODE == M_SPLIT) {
#pragma unroll
    for (int j = 0; j < C; ++j) {
      const int c = chunk_of<L>(li, j);
      st_u128((FAST || c < a.nchunk) ? o.p0 + 16 * c : lsink, o.w[j], c_al);
    }
#pragma unroll
    for (int k = 0; k < TPL; ++k) st_u32(o.p1 + 4 * ((li + L * k) & 31), o.ry[k], a_al);
  } else if constexpr (MODE == M_MXFP4) {
#pragma unroll
    for (int j = 0; j < C; ++j) {
      const int c = chunk_of<L>(li, j);
      const bool in = FAST || c < a.nchunk;
      st_u32(in ? o.p0 + 4 * c : lsink, o.w[j].x, c_al);
      st_u8(in ? o.p1 + (c >> 2) : lsink + 8, o.sb[j]);  // every lane of the group
    }
  } else if constexpr (MODE == M_FP4_NOPE) {
    // after the 64 rope bytes: the codes (4 bytes per chunk), the group
    // scales (every lane of a group writes its scale) and the zero pad
    uint8_t *r0 = o.p0 + 64;
#pragma unroll
    for (int j = 0; j < C; ++j) {
      const int c = chunk_of<L>(li, j);
      const bool in = FAST || c < a.nchunk;
      st_u32(in ? r0 + 4 * c : lsink, o.w[j].x, c_al);
      st_u16(in ? r0 + a.nseg / 2 + 2 * (c >> a.glog) : lsink + 8, o.sb[j], c_al);
    }
    store_pad<L>(a, li, lsink, o.p0);
  } else if constexpr (MODE == M_MXFP8 || MODE == M_FP8_ROW) {
#pragma unroll
    for (int j = 0; j < C; ++j) {
      const int c = chunk_of<L>(li, j);
      const bool in = FAST || c < a.nchunk;
      st_u64(in ? o.p0 + 8 * c : lsink, make_uint2(o.w[j].x, o.w[j].y), c_al);
      if constexpr (MODE == M_MXFP8)
        st_u8(in ? o.p1 + (c >> 2) : lsink + 8, o.sb[j]);  // every lane of the group
    }
    // every lane of the row writes the row's fp32 scale
    if constexpr (MODE == M_FP8_ROW) st_u32(o.p1, o.sb[0], a.a_align);
  } else {
#pragma unroll
    for (int j = 0; j < C; ++j) {
      const int c = chunk_of<L>(li, j);
      const bool in = FAST || c < a.nchunk;
      st_u64(in ? o.p0 + 8 * c : lsink, make_uint2(o.w[j].x, o.w[j].y), c_al);
      // every lane of the group writes the group's scale
      if constexpr (MODE == M_FP8_E8M0)
        st_u8(in ? o.p0 + a.nseg + 128 + (c >> 3) : lsink + 8, o.sb[j]);
      else
        st_u16(in ? o.p0 + a.nseg + 128 + 2 * (c >> 3) : lsink + 8, o.sb[j], c_al);
    }
#pragma unroll
    for (int k = 0; k < TPL; ++k)
      st_u32(o.p0 + a.nseg + 4 * ((li + L * k) & 31), o.ry[k], c_al);
    if constexpr (MODE == M_FP8_BF16) store_pad<L>(a, li, lsink, o.p0);
  }
}

// Description of one wave-iteration (R rows): which rows are live, the first
// live row (the one skipped tokens read instead of their own) and every
// row's slot, all wave-uniform for R <= 2.  For R > 2 each lane keeps its own
// row's slot (own) and only its own row's bit in live; sl is unused.
template <int R>
struct IterInfo {
  uint32_t live;   // bit r: row r is live
  uint32_t g;      // row group (rows g * R + r)
  uint32_t first;  // first live row, 0 if none
  uint32_t sl[R];  // slot of each row
  uint32_t own;    // (R > 2) slot of the lane's own row, per lane
};

template <int MODE, bool NORM, bool ROPE, int L, int C, int FAST, bool XF16 = false>
__global__ __launch_bounds__(256) void epilog_kernel(const KArgs a) {
  static_assert(!XF16 || whole_row(MODE), "fp16 rows: indexer modes");
  constexpr int R = 64 / L;  // rows per wave-iteration
  static_assert(FAST != 2 || (staged_mode(MODE) && R <= 2 && max_row_bytes(L, C) <= 1024),
                "staged rows");
  const int lane = threadIdx.x & 63;
  const int li = lane & (L - 1);
  const int sub = lane / L;
  // dynamic LDS: (FAST == 2) the reciprocal table; gamma (the same for every
  // row) staged once per block; (FAST == 2) the waves' row images
  extern __shared__ float4 lds_base[];
  if constexpr (FAST == 2) {
    float2 *tb = reinterpret_cast<float2 *>(lds_base);
    for (int k = threadIdx.x; k < 128; k += 256) tb[k] = recip_entry(k);
  }
  float4 *g_lds = lds_base + (FAST == 2 ? RECIP_BYTES / 16 : 0);
  if constexpr (NORM) {
    for (int i = threadIdx.x; i < L * C; i += 256) {
      const int c = chunk_of<L>(i % L, i / L);
      float g[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (c < a.nchunk) unpack8(ld16_cached(a.gamma + 8 * c), g);
      g_lds[i] = make_float4(g[0], g[1], g[2], g[3]);
      g_lds[i + L * C] = make_float4(g[4], g[5], g[6], g[7]);
    }
  }
  if constexpr (NORM || FAST == 2) __syncthreads();
  // per-wave staging area for FAST == 2, after gamma
  uint8_t *stage = reinterpret_cast<uint8_t *>(g_lds) + (NORM ? L * C * 32 : 0) +
                   (threadIdx.x >> 6) * R * a.img_bytes;
  const uint32_t piece = FAST == 2 ? 16u * (uint32_t)(lane % (a.img_bytes / 16)) : 0u;
  if constexpr (FAST == 2) {
    // the wave's R row images start as zeros: their pad stays zero
    for (int b = 16 * lane; b < R * a.img_bytes; b += 64 * 16)
      *reinterpret_cast<uint4 *>(stage + b) = make_uint4(0, 0, 0, 0);
    lds_handover();
  }
  // Blocks are dispatched round-robin over the 8 XCDs, so consecutive row
  // groups spread over all of them (an XCD-major remap, each XCD taking a
  // contiguous range, measured 0.3-4 % slower on every workload).
  const int wave = __builtin_amdgcn_readfirstlane((int)blockIdx.x * 4 + (int)(threadIdx.x >> 6));
  if (wave >= a.n_groups) return;
  const int n_it = (a.n_groups - wave + a.nwaves - 1) / a.nwaves;
  const uint32_t ns = (uint32_t)a.num_slots;

  // Slot of token row r < T from the index array; 0xFFFFFFFF (past every
  // slot) skips the token.  SLOT: index[r]; the other modes first split r
  // into batch b and position s (r = b * seq_len + s).
  //  BATCH:       row index[r] of batch b's rows (b * block_size ...);
  //  BLOCK:       entry b * n_chunk_b + s / block_size names the block, the
  //               row in it is s % block_size;
  //  BATCH_START: row index[b] + s of batch b's rows.
  auto token_slot = [&](uint32_t r) -> uint32_t {
    const uint32_t bs = (uint32_t)a.block_size;
    auto blk_of = [&](uint32_t v) -> uint32_t {
      return a.bs_log2 >= 0 ? v >> a.bs_log2 : (uint32_t)(((uint64_t)v * a.bs_magic) >> a.bs_shift);
    };
    const uint32_t b = (uint32_t)(((uint64_t)r * a.sq_magic) >> a.sq_shift);
    const uint32_t s = r - b * (uint32_t)a.seq_len;
    if (a.index_mode == KVEPI_INDEX_BATCH) {
      const uint32_t v = (uint32_t)a.slots[r];
      return v < bs ? b * bs + v : 0xFFFFFFFFu;
    }
    if (a.index_mode == KVEPI_INDEX_BLOCK) {
      const uint32_t c = blk_of(s);
      const uint32_t v = (uint32_t)a.slots[b * (uint32_t)a.n_chunk_b + c];
      return v < ns ? blk_of(v) * bs + (s - c * bs) : 0xFFFFFFFFu;
    }
    const uint32_t v = (uint32_t)a.slots[b];  // KVEPI_INDEX_BATCH_START
    return v < bs && v + s < bs ? b * bs + v + s : 0xFFFFFFFFu;
  };
  // Slots come in windows of L iterations: lane l of window w holds the
  // slot of row sub = l % R of iteration j = w * L + l / R.  Lanes past the
  // wave's rows read slot 0 (their value is never used).
  auto win_load = [&](int w) -> int {
    const int j = w * L + lane / R;
    const int64_t r = ((int64_t)wave + (int64_t)j * a.nwaves) * R + lane % R;
    const bool in = j < n_it && r < a.T;
    if (a.index_mode == KVEPI_INDEX_SLOT)
      return __builtin_nontemporal_load(a.slots + (in ? r : 0));
    return in ? (int)token_slot((uint32_t)r) : 0;
  };
  // iteration j's rows, from the window holding it
  // (32-bit row arithmetic: for j < n_it every row index is below T + R)
  auto prep = [&](int j, int win) -> IterInfo<R> {
    IterInfo<R> t;
    t.live = 0;
    t.first = 0;
    if constexpr (R > 2)
      t.own = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * ((j % L) * R + sub), win);
    t.g = (uint32_t)wave + (uint32_t)j * (uint32_t)a.nwaves;
    const bool in = j < n_it;
    if constexpr (R > 2) {
      // many rows per wave: each lane decides for its own row (live holds only
      // the lane's own bit), and the first live row comes from a ballot
      const uint32_t row = t.g * R + (uint32_t)sub;
      const bool lv = in && row < (uint32_t)a.T && t.own < ns;
      const uint64_t bal = __builtin_amdgcn_ballot_w64(lv);
      t.live = lv ? 1u << sub : 0u;
      t.first = bal != 0 ? t.g * R + (uint32_t)__builtin_ctzll(bal) / L : 0u;
    } else {
#pragma unroll
      for (int r = R - 1; r >= 0; --r) {
        const uint32_t sl = (uint32_t)__builtin_amdgcn_readlane(win, (j % L) * R + r);
        const uint32_t row = t.g * R + r;
        t.sl[r] = sl;
        if (in && row < (uint32_t)a.T && sl < ns) {
          t.live |= 1u << r;
          t.first = row;  // the loop runs downwards: the last assignment is the first row
        }
      }
    }
    return t;
  };
  const uint32_t subbit = 1u << sub;
  auto lane_live = [&](const IterInfo<R> &t) -> bool { return (t.live & subbit) != 0; };
  // issues the loads of iteration j's rows
  auto issue = [&](const IterInfo<R> &t, RowBuf<MODE, ROPE, L, C> &b) {
    const uint32_t dr = lane_live(t) ? t.g * R + sub - t.first : 0u;
    const uint8_t *xr = reinterpret_cast<const uint8_t *>(a.x) + (uint64_t)t.first * a.x_pitch;
    const uint64_t rp = gen_rope(MODE) ? (uint64_t)a.rope_pitch : 128u;  // cos / sin row bytes
    const uint8_t *cr = reinterpret_cast<const uint8_t *>(a.cos) + (uint64_t)t.first * rp;
    const uint8_t *sr = reinterpret_cast<const uint8_t *>(a.sin) + (uint64_t)t.first * rp;
    load_row<MODE, NORM, ROPE, L, C, FAST>(a, xr, cr, sr, dr, li, b);
  };
  // issues the loads of iteration j's own rows, whatever their slots (rows
  // past the tokens read the last token's row)
  auto issue_own = [&](int j, RowBuf<MODE, ROPE, L, C> &b) {
    const uint32_t base = j < n_it ? ((uint32_t)wave + (uint32_t)j * (uint32_t)a.nwaves) * R : 0u;
    const uint32_t dr = min((uint32_t)sub, (uint32_t)a.T - 1u - base);
    const uint8_t *xr = reinterpret_cast<const uint8_t *>(a.x) + (uint64_t)base * a.x_pitch;
    const uint64_t rp = gen_rope(MODE) ? (uint64_t)a.rope_pitch : 128u;
    const uint8_t *cr = reinterpret_cast<const uint8_t *>(a.cos) + (uint64_t)base * rp;
    const uint8_t *sr = reinterpret_cast<const uint8_t *>(a.sin) + (uint64_t)base * rp;
    load_row<MODE, NORM, ROPE, L, C, FAST>(a, xr, cr, sr, dr, li, b);
  };
  // computes iteration j's rows and stores them (after the caller has issued
  // the next loads)
  RowOut<MODE, L, C> out;
  auto compute = [&](const IterInfo<R> &t, const RowBuf<MODE, ROPE, L, C> &b) {
    out.redo = false;
    if (lane_live(t)) {
      compute_row<MODE, NORM, ROPE, L, C, FAST, XF16>(a, li, sub, b, g_lds, out);
      if constexpr (FAST == 2) stage_write<MODE, L, C>(a, li, sub, out, stage);
    }
    if constexpr (spec_rows(MODE, NORM, FAST)) {
      // a row whose inputs leave the fast ranges: both rows again, exactly
      if (__builtin_amdgcn_ballot_w64(out.redo) != 0 && lane_live(t)) {
        lds_handover();
        if constexpr (MODE == M_FP4_NOPE) {
          // the lane's x chunks again from memory: keeping them in registers
          // for this rare branch costs the FP4 nope kernel one wave per SIMD
          // (76 instead of 70 VGPRs; with them reloaded it measured 2.6 %
          // faster, while mode 0 measured 1 % slower at 71 VGPRs)
          const uint8_t *xr = reinterpret_cast<const uint8_t *>(a.x) +
                              (uint64_t)(t.g * R + sub) * a.x_pitch;
          uint4 xw[C];
#pragma unroll
          for (int j = 0; j < C; ++j)
            xw[j] = *reinterpret_cast<const uint4 *>(xr + 16u * (uint32_t)chunk_of<L>(li, j));
          exact_row<MODE, L, C>(a, li, xw, g_lds, out);
        } else {
          exact_row<MODE, L, C>(a, li, b.xw, g_lds, out);
        }
        stage_write<MODE, L, C>(a, li, sub, out, stage);
      }
    }
    // the staged bytes one lane writes are stored by another lane: order the
    // LDS writes before the reads in stage_store (wave scope)
    if constexpr (FAST == 2) lds_handover();
  };
  // destination of row r (the sink when it is not live)
  // (pointers, not integers, so that the compiler keeps them global)
  auto dst = [&](const IterInfo<R> &t, int r) -> uint8_t * {
    return (t.live >> r) & 1 ? row_addr(a.cache, t.sl[r], a, a.c_pitch, a.c_bstride) : g_sink;
  };
  auto adst = [&](const IterInfo<R> &t, int r) -> uint8_t * {
    return (t.live >> r) & 1 ? row_addr(a.aux, t.sl[r], a, a.a_pitch, a.a_bstride)
                             : g_sink + kSinkHalf;
  };
  auto store = [&](const IterInfo<R> &t) {
    if constexpr (FAST == 2) {
      uint8_t *d[R];
#pragma unroll
      for (int r = 0; r < R; ++r) d[r] = dst(t, r) + a.img_off;
      stage_store<R>(stage, a.img_bytes, piece, d);
      // ... and those reads before the next row's writes to the same image
      lds_handover();
    } else {
      uint8_t *d, *ad = nullptr;
      if constexpr (R <= 2) {
        // per-row destinations on the scalar unit, then picked per lane
        d = dst(t, 0);
        if constexpr (has_aux(MODE)) ad = adst(t, 0);
        if constexpr (R == 2) {
          d = sub ? dst(t, 1) : d;
          if constexpr (has_aux(MODE)) ad = sub ? adst(t, 1) : ad;
        }
      } else {
        // many rows per wave: each lane computes its own row's destination
        const uint32_t sl = t.own;
        const bool live = lane_live(t);
        d = live ? row_addr(a.cache, sl, a, a.c_pitch, a.c_bstride) : g_sink;
        if constexpr (has_aux(MODE))
          ad = live ? row_addr(a.aux, sl, a, a.a_pitch, a.a_bstride) : g_sink + kSinkHalf;
      }
      out.p0 = d;
      out.p1 = ad;
      store_row<MODE, ROPE, L, C, FAST>(a, li, lane, out);
    }
  };

  int win_cur = win_load(0), win_next = win_load(1);
  // window of iteration j, loading the one after it on entering a window
  auto window = [&](int j) -> int {
    if (j % L == 0 && j > 0) {
      win_cur = win_next;
      win_next = win_load(j / L + 1);
    }
    return win_cur;
  };

  if constexpr (C > 2) {
    // rows of more than two chunks per lane: no prefetch (their registers
    // are needed for the row itself)
    RowBuf<MODE, ROPE, L, C> cur;
    for (int it = 0; it < n_it; ++it) {
      const IterInfo<R> t = prep(it, window(it));
      issue(t, cur);
      compute(t, cur);
      store(t);
    }
  } else {
    // Software pipeline, D iterations ahead, with D register sets (set d
    // holds the iterations j with j % D == d).  gfx9 has a single in-order
    // counter for vector loads and stores, so a wait for a load also waits
    // for every store issued before it.  Each step j therefore computes
    // iteration j (loaded D steps earlier), then issues the loads of
    // iteration j + D and only then the stores of iteration j; the wait
    // before computing j + 1 then leaves the stores of the last D - 1
    // iterations in flight.  Every step issues the same memory operations
    // (skipped tokens re-read a live row of their iteration and store to a
    // sink), so the compiler's wait counts are exact.  (Three or four sets
    // measured slower or no faster: registers are the scarcer resource.)
    constexpr int D = 2;
    RowBuf<MODE, ROPE, L, C> buf[D];
    IterInfo<R> t[D];
    // The first D iterations load every lane's own row before the slots are
    // known (a skipped token's row is read for nothing), so that the row
    // loads do not wait for the slot window: short launches are bound by
    // this chain of memory latencies.
#pragma unroll
    for (int d = 0; d < D; ++d) issue_own(d, buf[d]);
#pragma unroll
    for (int d = 0; d < D; ++d) t[d] = prep(d, window(d));
    // drain once before the loop: otherwise the loop's waits are sized for
    // the first trip, whose loads were issued in an order of the compiler's
    // choosing
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    for (int it = 0; it < n_it; it += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        compute(t[d], buf[d]);
        const IterInfo<R> nt = prep(it + d + D, window(it + d + D));
        issue(nt, buf[d]);
        store(t[d]);
        t[d] = nt;
      }
    }
  }
}

// ------------------------------------------------------------------------
// dispatch
// ------------------------------------------------------------------------
typedef void (*kfn_t)(const KArgs);

template <int MODE, bool NORM, bool ROPE, int FAST, bool XF16 = false>
kfn_t pick_layout_f(int L, int C) {
  if (L == 8) return epilog_kernel<MODE, NORM, ROPE, 8, 1, FAST, XF16>;
  if (L == 16) return epilog_kernel<MODE, NORM, ROPE, 16, 1, FAST, XF16>;
  if (L == 32)
    return C == 1 ? epilog_kernel<MODE, NORM, ROPE, 32, 1, FAST, XF16>
                  : epilog_kernel<MODE, NORM, ROPE, 32, 2, FAST, XF16>;
  switch (C) {
    case 1: return epilog_kernel<MODE, NORM, ROPE, 64, 1, FAST, XF16>;
    case 2: return epilog_kernel<MODE, NORM, ROPE, 64, 2, FAST, XF16>;
    case 4: return epilog_kernel<MODE, NORM, ROPE, 64, 4, FAST, XF16>;
    case 8: return epilog_kernel<MODE, NORM, ROPE, 64, 8, FAST, XF16>;
    default: return epilog_kernel<MODE, NORM, ROPE, 64, 16, FAST, XF16>;
  }
}

// indexer modes: bf16 or fp16 rows
template <int MODE>
kfn_t pick_indexer(int L, int C, int fast, bool xf16) {
  if (xf16)
    return fast ? pick_layout_f<MODE, false, false, 1, true>(L, C)
                : pick_layout_f<MODE, false, false, 0, true>(L, C);
  return fast ? pick_layout_f<MODE, false, false, 1>(L, C)
              : pick_layout_f<MODE, false, false, 0>(L, C);
}

template <int MODE, bool NORM, bool ROPE>
kfn_t pick_layout(int L, int C, int fast) {
  if constexpr (staged_mode(MODE))
    if (fast == 2)
      return C == 1 ? epilog_kernel<MODE, NORM, ROPE, 32, 1, 2>
                    : epilog_kernel<MODE, NORM, ROPE, 32, 2, 2>;
  return fast ? pick_layout_f<MODE, NORM, ROPE, 1>(L, C)
              : pick_layout_f<MODE, NORM, ROPE, 0>(L, C);
}

kfn_t pick(int mode, bool norm, bool rope, bool xf16, int L, int C, int fast) {
  switch (mode) {
    case M_FP8_BF16:
      if (norm)
        return rope ? pick_layout<M_FP8_BF16, true, true>(L, C, fast)
                    : pick_layout<M_FP8_BF16, true, false>(L, C, fast);
      return rope ? pick_layout<M_FP8_BF16, false, true>(L, C, fast)
                  : pick_layout<M_FP8_BF16, false, false>(L, C, fast);
    case M_FP8_E8M0:
      if (norm)
        return rope ? pick_layout<M_FP8_E8M0, true, true>(L, C, fast)
                    : pick_layout<M_FP8_E8M0, true, false>(L, C, fast);
      return rope ? pick_layout<M_FP8_E8M0, false, true>(L, C, fast)
                  : pick_layout<M_FP8_E8M0, false, false>(L, C, fast);
    case M_MXFP4:
      return pick_indexer<M_MXFP4>(L, C, fast, xf16);
    case M_MXFP8:
      return pick_indexer<M_MXFP8>(L, C, fast, xf16);
    case M_FP8_ROW:
      return pick_indexer<M_FP8_ROW>(L, C, fast, xf16);
    case M_FP4_NOPE:
      return norm ? pick_layout<M_FP4_NOPE, true, false>(L, C, fast)
                  : pick_layout<M_FP4_NOPE, false, false>(L, C, fast);
    case M_SPLIT_G:
      return pick_layout<M_SPLIT_G, true, true>(L, C, fast);
    default:
      return pick_layout<M_SPLIT, true, true>(L, C, fast);
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

// Blocks of 256 threads that one CU holds at once for a kernel instance (set
// by its register and LDS use), cached per instance and LDS size.
int blocks_per_cu(kfn_t fn, size_t lds) {
  struct Entry {
    kfn_t fn;
    size_t lds;
    int nb;
  };
  static Entry cache[128];
  static int n = 0;
  static std::mutex mu;
  std::lock_guard<std::mutex> guard(mu);
  for (int i = 0; i < n; ++i)
    if (cache[i].fn == fn && cache[i].lds == lds) return cache[i].nb;
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, reinterpret_cast<const void *>(fn), 256,
                                                   lds) != hipSuccess ||
      nb <= 0)
    nb = 2;
  if (nb > 8) nb = 8;
  if (n < 128) cache[n++] = Entry{fn, lds, nb};
  return nb;
}

}  // namespace kvepi

static_assert(sizeof(kvepi::KArgs) <= KVEPI_KARGS_BYTES && alignof(kvepi::KArgs) <= 8,
              "the kernel arguments must fit kvepi_launch_cfg::args");

kvepi_status kvepi_configure(const kvepi_plan &p, kvepi_launch_cfg *cfg) {
  using namespace kvepi;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return KVEPI_ERR_RUNTIME;
  KArgs a{};
  a.x = p.x;
  a.gamma = p.gamma;
  a.cos = p.cos;
  a.sin = p.sin;
  a.slots = p.slots;
  a.cache = p.cache;
  a.aux = p.aux;
  a.x_stride = p.x_stride;
  a.x_pitch = (uint32_t)(p.x_stride * 2);
  a.c_pitch = p.c_pitch;
  a.c_bstride = p.c_bstride;
  a.a_pitch = p.a_pitch;
  a.a_bstride = p.a_bstride;
  // slot / block_size for slot < 2^31: m = ceil(2^(31+l) / bs), l = ceil(log2 bs)
  int l = 0;
  while ((INT64_C(1) << l) < p.block_size) ++l;
  const int shift = 31 + l;
  const unsigned __int128 num = (unsigned __int128)1 << shift;
  a.bs_magic = (uint64_t)((num + (unsigned __int128)p.block_size - 1) /
                          (unsigned __int128)p.block_size);
  a.bs_shift = shift;
  a.block_size = (int32_t)p.block_size;
  a.bs_log2 = (INT64_C(1) << l) == p.block_size ? l : -1;
  a.T = (int32_t)p.T;
  a.index_mode = p.index_mode;
  a.seq_len = p.index_mode == KVEPI_INDEX_SLOT ? 1 : (int32_t)p.seq_len;
  {
    // row / seq_len for row < 2^31, as for the block size below
    int ls = 0;
    while ((INT64_C(1) << ls) < a.seq_len) ++ls;
    const unsigned __int128 n2 = (unsigned __int128)1 << (31 + ls);
    a.sq_magic = (uint64_t)((n2 + (unsigned __int128)a.seq_len - 1) / (unsigned __int128)a.seq_len);
    a.sq_shift = 31 + ls;
  }
  a.n_chunk_b = (int32_t)((a.seq_len + p.block_size - 1) / p.block_size);
  a.num_slots = (int32_t)p.num_slots;
  a.nseg = (int32_t)p.nope;
  a.nchunk = (int32_t)(p.nope / 8);
  a.concat_col = (int32_t)p.concat_col;
  a.kv_cache_col = (int32_t)p.kv_cache_col;
  a.pad16 = (p.c_align >= 16 && p.concat_col % 16 == 0 &&
             (p.kv_cache_col - p.concat_col) % 16 == 0)
                ? (int32_t)((p.kv_cache_col - p.concat_col) / 16)
                : -1;
  a.c_align = p.c_align;
  a.a_align = p.aux != nullptr ? p.a_align : 16;
  a.eps = p.eps;
  // FP4 nope mode: chunks of 8 values per scale group (2, 4 or 8)
  a.glog = p.mode == KVEPI_MODE_FP4_NOPE ? (p.group_size == 16 ? 1 : p.group_size == 32 ? 2 : 3)
                                         : 0;
  // staged rows: mode 0 stages the whole row, the FP4 nope mode the part
  // after the 64 rope bytes
  a.img_off = p.mode == KVEPI_MODE_FP4_NOPE ? 64 : 0;
  a.img_bytes = (int32_t)(p.kv_cache_col - a.img_off);
  a.rope_half = (int32_t)(p.rope_dim / 2);
  a.rope_pitch = (int32_t)(2 * p.rope_dim);
  a.nseg_f = (float)p.nope;
  a.inv_nseg = (p.nope & (p.nope - 1)) == 0 ? 1.0f / (float)p.nope : 0.0f;

  // layout: L lanes per row (power of two, 8..64), C chunks per lane; rows
  // of 64 chunks (d = 576) go two to a wave
  int L = 8;
  while (L < 64 && L < a.nchunk) L *= 2;
  if (a.nchunk == 64) L = 32;
  int C = 1;
  while (C * L < a.nchunk) C *= 2;

  const int rows_per_wave = 64 / L;
  const int64_t n_groups = (p.T + rows_per_wave - 1) / rows_per_wave;
  // FAST: whole chunks per lane and 16-byte aligned rows (4-byte aligned k
  // rows in the bf16 split mode); stores then need no alignment dispatch
  // 2: mode 0 and FP4 nope rows laid out on 32 lanes (one or two chunks
  // each) also assemble their rows in LDS
  const bool aligned = L * C == a.nchunk && a.c_align >= 16 &&
                       (p.mode != KVEPI_MODE_BF16_SPLIT || a.a_align >= 4);
  const bool stages =
      p.mode == KVEPI_MODE_FP8_BF16SCALE || p.mode == KVEPI_MODE_FP4_NOPE;
  const int fast = !aligned ? 0 : (stages && L == 32) ? 2 : 1;
  // the bf16 split with a rope segment of another length than 64
  const int kmode = p.mode == KVEPI_MODE_BF16_SPLIT && p.rope_dim != 64 ? (int)M_SPLIT_G : p.mode;
  kfn_t fn = pick(kmode, p.norm, p.rope, p.x_fp16, L, C, fast);
  size_t lds = p.norm ? (size_t)L * C * 32 : 0;  // gamma as fp32, 32 KB at most
  if (fast == 2) lds += 128 * 8 + (size_t)4 * (64 / L) * a.img_bytes;  // table, staging

  // persistent waves: exactly as many blocks as the CUs hold at once
  const int cus = device_cus();
  int64_t max_waves = (int64_t)cus * blocks_per_cu(fn, lds) * 4;
  // KVEPI_MAX_WAVES (a multiple of 4, read at every launch) caps the grid:
  // tests use it to run many iterations per wave on small inputs
  if (const char *cap = getenv("KVEPI_MAX_WAVES")) {
    const long v = strtol(cap, nullptr, 10);
    if (v >= 4 && v < max_waves) max_waves = v & ~3L;
  }
  // Two iterations per wave, so that every wave's loads of its second
  // iteration overlap its first: with 2048 to 16384 row groups (up to 8 per
  // SIMD) that measured 7-20 % faster than one iteration per wave.  With no
  // more row groups than SIMDs, one iteration per wave spreads them over
  // more SIMDs and measured 6-15 % faster (launches timed as HIP-graph
  // replays, 128 to 2048 tokens).
  const int64_t simds = (int64_t)cus * 4;
  const int64_t waves = n_groups <= simds ? (n_groups < max_waves ? n_groups : max_waves)
                        : n_groups >= 2 * max_waves ? max_waves : (n_groups + 1) / 2;
  const int64_t blocks = (waves + 3) / 4;
  a.nwaves = (int32_t)(blocks * 4);
  a.n_groups = (int32_t)n_groups;

  *cfg = kvepi_launch_cfg{};
  cfg->fn = reinterpret_cast<const void *>(fn);
  cfg->blocks = (uint32_t)blocks;
  cfg->lds = (uint32_t)lds;
  cfg->device = dev;
  memcpy(cfg->args, &a, sizeof a);
  return KVEPI_OK;
}

kvepi_status kvepi_enqueue(const kvepi_launch_cfg &cfg, void *stream) {
  // the kernel takes its KArgs by value: HIP copies sizeof(KArgs) bytes from
  // the address given for argument 0
  void *args[] = {const_cast<unsigned char *>(cfg.args)};
  hipError_t e = hipLaunchKernel(cfg.fn, dim3(cfg.blocks), dim3(256), args, cfg.lds,
                                 static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVEPI_OK : KVEPI_ERR_RUNTIME;
}

kvepi_status kvepi_current_device(int32_t *device) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return KVEPI_ERR_RUNTIME;
  *device = dev;
  return KVEPI_OK;
}

kvepi_status kvepi_launch(const kvepi_plan &p, void *stream) {
  kvepi_launch_cfg cfg;
  const kvepi_status st = kvepi_configure(p, &cfg);
  return st != KVEPI_OK ? st : kvepi_enqueue(cfg, stream);
}
