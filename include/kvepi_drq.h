/*
 * kvepi_drq.h -- C ABI of the dequant -> RoPE -> static int8 quantisation ->
 * KV cache operator for AMD Instinct MI355X (gfx950), the companion of the
 * fused epilog of kvepi.h (the blog on aclnnDequantRopeQuantKvcache:
 * 计算步骤公式 steps 1-5, 两种 KV Cache 更新模式, 约束说明).
 *
 * For each token row t of x [T, H], H = (nq + 2 nkv) * head_dim:
 *   1. dequantX = x when x is bf16/fp16; for int32 x (the dequant path)
 *      float(x) * weight_scale[h], times act_scale[t] when given, plus
 *      bias[h] when given, in fp32, then rounded to out_dtype;
 *   2. split into nq q heads, nkv k heads, nkv v heads of head_dim values;
 *   3. rotate-half RoPE of every q and k head with the token's cos / sin
 *      [head_dim] (out[j] = a*cos[j] - b*sin[j], out[j+D/2] = b*cos[j+D/2] +
 *      a*sin[j+D/2] for a = in[j], b = in[j+D/2], j < D/2; products and the
 *      sum in fp32, then out_dtype) -> q_out, k_out; v_out = the v heads;
 *   4. static int8 quantisation of k_out and v_out per channel c of
 *      [nkv * head_dim]: rint(v / scale[c] + offset[c]) (offset optional),
 *      half to even, saturated to [-128, 127];
 *   5. the int8 rows written to k_cache / v_cache at the token's row.
 * Two stages as in kvepi.h: kvepi_drq_get_workspace validates and returns 0,
 * kvepi_drq_run validates again and launches on the caller's stream; the
 * conventions of kvepi.h apply (DEVICE pointers only checked for NULL and
 * alignment, caller-owned buffers, asynchronous, errors before any launch,
 * deterministic results).
 */
#ifndef KVEPI_DRQ_H
#define KVEPI_DRQ_H

#include "kvepi.h"

#ifdef __cplusplus
extern "C" {
#endif

/* element types */
#define KVEPI_DT_BF16 0
#define KVEPI_DT_FP16 1
#define KVEPI_DT_INT32 2
#define KVEPI_DT_FP32 3

/* cache modes (the blog's 两种 KV Cache 更新模式) */
#define KVEPI_DRQ_PAGE 0       /* indices [T]: the token's slot in a paged cache
                                  [block_num, block_size, nkv, head_dim]; -1
                                  or a value outside [0, num_slots) skips the
                                  cache write of the token                    */
#define KVEPI_DRQ_CONTIGUOUS 1 /* indices [B], T = B * seq_len: token s of
                                  batch b goes to row indices[b] + s of batch
                                  b's cache [Bc >= B, Sc, nkv, head_dim]
                                  (block b, block_size = Sc); -1, or a row
                                  past Sc, skips the write                    */

typedef struct kvepi_drq_params {
  const void *x;            /* DEVICE [num_tokens, H], 16-byte aligned         */
  int32_t x_dtype;          /* KVEPI_DT_INT32, or out_dtype                    */
  int32_t out_dtype;        /* KVEPI_DT_BF16 / FP16: cos, sin and the outputs  */
  int64_t num_tokens;       /* T >= 0                                          */
  int64_t x_row_stride;     /* elements between rows, >= H, multiple of 8      */
  int32_t nq, nkv;          /* heads (>= 1 each)                                */
  int32_t head_dim;         /* D, multiple of 16; H <= 4096, H % 64 == 0       */
  const void *cos, *sin;    /* DEVICE [T, D] out_dtype, 16-byte aligned         */
  const float *weight_scale;   /* DEVICE [H]: required for int32 x, else NULL  */
  const float *act_scale;      /* DEVICE [T] or NULL (int32 x only)            */
  const void *bias;            /* DEVICE [H] of bias_dtype or NULL (int32 x)   */
  int32_t bias_dtype;          /* KVEPI_DT_FP32 / INT32 / BF16 / FP16          */
  const float *scale_k, *scale_v;   /* DEVICE [nkv * D]                         */
  const float *offset_k, *offset_v; /* DEVICE [nkv * D] or NULL                 */
  const int32_t *indices;   /* DEVICE int32, see the cache modes                */
  int32_t cache_mode;       /* KVEPI_DRQ_PAGE or KVEPI_DRQ_CONTIGUOUS           */
  int64_t seq_len;          /* contiguous mode: tokens per batch               */
  kvepi_cache k_cache;      /* int8, head_dim >= nkv * D; data, head_dim and
                               block_stride multiples of 8 bytes              */
  kvepi_cache v_cache;      /* the same block_num and block_size as k_cache   */
  void *q_out;              /* DEVICE [T, nq * D] out_dtype, 16-byte aligned   */
  void *k_out, *v_out;      /* DEVICE [T, nkv * D] out_dtype, both or neither
                               (the operator's kvOutput)                      */
} kvepi_drq_params;

/* Errors: NULLPTR for a missing required pointer; PARAM for a dtype, cache
 * mode or optional-input combination the operator does not take (约束说明
 * 4 and 5); SHAPE for sizes outside the constraints (约束说明 6: H <= 4096
 * and H % 64 == 0; head_dim % 16 == 0; cache rows shorter than nkv * D;
 * contiguous mode with seq_len not dividing T, more batches than cache
 * blocks, or seq_len above the block size); LAYOUT for alignment. */
KVEPI_API kvepi_status kvepi_drq_get_workspace(const kvepi_drq_params *params,
                                               uint64_t *workspace_bytes);
/* Debug aid: with the environment variable KVEPI_CHECK_SLOTS set (to
 * anything but "0"; read at every call), kvepi_drq_run in page mode copies
 * indices to the host, synchronously on `stream`, and returns
 * KVEPI_ERR_PARAM before any launch if two tokens name the same row (a
 * failed copy returns KVEPI_ERR_RUNTIME); otherwise repeated slots are not
 * detected and their rows are unspecified. */
KVEPI_API kvepi_status kvepi_drq_run(const kvepi_drq_params *params, void *workspace,
                                     uint64_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* KVEPI_DRQ_H */
