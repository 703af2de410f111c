/*
 * kvepi_oracle.h -- plain, slow, single-threaded CPU oracle of the fused
 * KV-cache write epilog.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library includes, links or
 * calls this code; only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header, table or constant with the
 * HIP path.
 *
 * What it computes (sources, cited by page title and section):
 *  - "aclnnKvCompressEpilog", 功能说明 / 计算公式: the last 64 columns of a row
 *    are the rope segment, the first d-64 the nope segment; per-group amax
 *    quantisation of the nope segment, q_i = round(x_i / scale_g) with
 *    scale_g = max|x_g| / FP8_MAX; mode 0 stores the scale as bf16, mode 1 as
 *    an e8m0 power of two rounded up.
 *  - "aclnnKvCompressEpilog", 约束说明: the cache is [blockNum, blockSize, 1,
 *    headDim]; the row byte count kvCacheCol = align(concatCol); slot -1 is
 *    skipped; only the blockNum dimension may be non-contiguous.
 *  - "aclnnKvRmsNormRopeCache", 计算公式 (1) interleaveRope and (2) rmsNorm.
 *  - "indexer_quant_cache", 接口功能 / 约束: MX-FP4 groups of 32 with an e8m0
 *    scale written to a separate cache_scale tensor; rows not hit keep their
 *    values.  The same page's mxfp8 mode (E4M3 codes, groups of 32, e8m0
 *    scale) and fp8 mode (E4M3 codes, the whole row one group, one FLOAT
 *    scale per row in cache_scale).
 *  - "aclnnKvCompressEpilog", 计算公式 scene 3 (quantMode=2) and 约束说明:
 *    the nope segment in groups of quantGroupSize (16, 32 or 64) values,
 *    scale_g = max|x_g| / FP4_MAX (6) stored in 2 bytes, codes
 *    FLOAT4_E2M1(x_i / scale_g); the row is 64 rope bytes, (d-64)/2 code
 *    bytes and 2 bytes per group, padded to 32 bytes.  The rope bytes are
 *    HiFloat8 codes, a format the pages do not define: this mode writes the
 *    rest of the row and leaves them untouched.
 *
 * Arithmetic: IEEE fp32 (the precision the quantiser's division is defined
 * in), evaluated in the order written, compiled with -ffp-contract=off.  The
 * one order the pages leave open, the RMSNorm sum of squares, is a balanced
 * pairwise tree over the zero-padded power-of-two length.
 *
 * bf16 values are passed as their uint16_t bit patterns.
 */
#ifndef KVEPI_ORACLE_H
#define KVEPI_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Output modes (the oracle's own numbering). */
#define KVO_MODE_FP8_BF16SCALE 0 /* group-64 E4M3 codes, bf16 scale        */
#define KVO_MODE_FP8_E8M0 1      /* group-64 E4M3 codes, e8m0 scale        */
#define KVO_MODE_MXFP4 3         /* group-32 E2M1 nibbles, e8m0 scale row  */
#define KVO_MODE_BF16_SPLIT 4    /* RMSNorm -> ckv cache, RoPE -> k cache  */
#define KVO_MODE_MXFP8 5         /* group-32 E4M3 codes, e8m0 scale row    */
#define KVO_MODE_FP8_ROW 6       /* whole-row E4M3 codes, fp32 scale       */
#define KVO_MODE_FP4_NOPE 7      /* quantMode 2's nope half: group-G E2M1  */
                                 /* nibbles, bf16 scales; the 64 rope      */
                                 /* bytes at the row start not written     */

/* ---- number formats ---------------------------------------------------- */
float kvo_bf16_to_f32(uint16_t h);
float kvo_fp16_to_f32(uint16_t h);     /* IEEE binary16, exact           */
uint16_t kvo_f32_to_fp16(float f);     /* round to nearest, ties to even   */
uint16_t kvo_f32_to_bf16(float f);     /* round to nearest, ties to even   */
uint8_t kvo_enc_e4m3(float v);         /* OCP E4M3FN, RNE, saturate to 448 */
uint8_t kvo_enc_e2m1(float v);         /* OCP E2M1 nibble, RNE, sat. to 6  */
int kvo_e8m0_exponent(float amax, float fmax); /* smallest E>=-127 with
                                                  amax <= fmax*2^E         */

void kvo_enc_e4m3_batch(const float *v, uint8_t *out, int64_t n);
void kvo_enc_e2m1_batch(const float *v, uint8_t *out, int64_t n);
void kvo_f32_to_bf16_batch(const float *v, uint16_t *out, int64_t n);
void kvo_e8m0_exponent_batch(const float *amax, float fmax, int32_t *out,
                             int64_t n);

/* ---- per-row steps ----------------------------------------------------- */
/* RMSNorm over n bf16 values: y = bf16((x / sqrt(mean(x^2) + eps)) * gamma) */
void kvo_rmsnorm_row(const uint16_t *x, const uint16_t *gamma, int64_t n,
                     float eps, uint16_t *y);
/* Sum of squares as the balanced pairwise tree (exposed for its pin). */
float kvo_sumsq_tree(const uint16_t *x, int64_t n);
/* Interleaved RoPE on 64 values -> 64 half-split values. */
/* the same for a rope segment of n (even) values */
void kvo_rope_row_n(const uint16_t *x, const uint16_t *cos, const uint16_t *sin, int64_t n,
                    uint16_t *y);
void kvo_rope_row(const uint16_t *x, const uint16_t *cos, const uint16_t *sin,
                  uint16_t *y);

/* Row geometry.  Returns 0 on success, -1 for an unsupported combination. */
int kvo_row_bytes(int mode, int64_t d, int32_t group_size, int64_t *concat_col,
                  int64_t *kv_cache_col, int64_t *scale_col);

/* Quantise one prepared row v[0..d) (bf16 bits: nope segment already
 * normalised if RMSNorm is on, rope segment already rotated if RoPE is on)
 * into out[0..kv_cache_col) (modes 0/1), out[0..d/2) plus scale_out[0..d/32)
 * (MX-FP4), out[0..d) plus scale_out[0..d/32) (MX-FP8) or out[0..d) plus
 * the 4 little-endian bytes of the fp32 scale in scale_out (FP8 row). */
int kvo_quant_row(int mode, const uint16_t *v, int64_t d, int32_t group_size,
                  uint8_t *out, uint8_t *scale_out);
/* The same with x_fp16 != 0 reading v as IEEE binary16 (indexer modes). */
int kvo_quant_row_x(int mode, const uint16_t *v, int64_t d, int32_t group_size, int x_fp16,
                    uint8_t *out, uint8_t *scale_out);

/* ---- whole epilog ------------------------------------------------------ */
/* Cache geometry: [block_num, block_size, 1, head_dim] with head_dim and
 * block_stride counted in elements of elem_bytes bytes. */
typedef struct {
  uint8_t *data;
  int64_t block_num, block_size, head_dim, block_stride;
} kvo_cache;

/* Runs the epilog for tokens t = 0..T-1 in order.  gamma (length d-64) and
 * cos/sin ([T,64]) may be NULL.  aux is the cache_scale tensor (MX-FP4,
 * MX-FP8: bytes; FP8 row: fp32 elements) or the k cache (BF16 split).
 * Returns 0, or -1 on an argument it rejects. */
int kvo_epilog(int mode, int64_t T, int64_t d, const uint16_t *x,
               int64_t x_row_stride, const uint16_t *gamma,
               const uint16_t *cos, const uint16_t *sin, float eps,
               const int32_t *slot_mapping, int32_t group_size,
               const kvo_cache *cache, const kvo_cache *aux);

/* How a token finds its cache row (see kvo_token_slot). */
#define KVO_INDEX_SLOT 0        /* index[T]: one slot per token              */
#define KVO_INDEX_BATCH 1       /* index[B,S]: row within the batch's rows   */
#define KVO_INDEX_BLOCK 2       /* index[B,ceil(S/bs)]: one block per chunk  */
#define KVO_INDEX_BATCH_START 3 /* index[B]: first row of the batch's tokens */
int64_t kvo_token_slot(int index_mode, const int32_t *index, int64_t t, int64_t seq_len,
                       int64_t block_num, int64_t block_size);

/* kvo_epilog with fp16 rows (x_fp16, indexer modes only), the index modes
 * above (T must be a multiple of seq_len outside the SLOT mode) and the
 * rope segment length (64; any even value with d - rope_dim a multiple of
 * 8 in the bf16 split mode, whose cos / sin are then [T, rope_dim]). */
int kvo_epilog_ex(int mode, int64_t T, int64_t d, const uint16_t *x, int64_t x_row_stride,
                  int x_fp16, const uint16_t *gamma, const uint16_t *cos, const uint16_t *sin,
                  float eps, const int32_t *index, int index_mode, int64_t seq_len,
                  int rope_dim, int32_t group_size, const kvo_cache *cache,
                  const kvo_cache *aux);

/* ---- dequant -> RoPE -> int8 KV cache ----------------------------------- */
#define KVO_DT_BF16 0
#define KVO_DT_FP16 1
#define KVO_DT_INT32 2
#define KVO_DT_FP32 3
int8_t kvo_quant_int8(float v, float scale, const float *offset);
/* x [T, (nq + 2 nkv) * D] (int32, or bf16 / fp16 equal to out_dtype), cos /
 * sin [T, D] in out_dtype; weight_scale [H] (int32 x only, required),
 * act_scale [T], bias [H] of bias_dtype (int32 x only, optional);
 * scale_k / scale_v / offset_k / offset_v [nkv * D]; index: one slot per
 * token (KVO_INDEX_SLOT, the page mode) or one start row per batch
 * (KVO_INDEX_BATCH_START, the contiguous mode); caches int8 with head_dim
 * nkv * D; q_out [T, nq * D], k_out / v_out [T, nkv * D] (may be NULL) in
 * out_dtype. */
int kvo_drq(int64_t T, int nq, int nkv, int D, const void *x, int x_dtype, int64_t x_row_stride,
            const uint16_t *cos, const uint16_t *sin, int out_dtype, const float *weight_scale,
            const float *act_scale, const void *bias, int bias_dtype, const float *scale_k,
            const float *scale_v, const float *offset_k, const float *offset_v,
            const int32_t *index, int index_mode, int64_t seq_len, const kvo_cache *k_cache,
            const kvo_cache *v_cache, uint16_t *q_out, uint16_t *k_out, uint16_t *v_out);

#ifdef __cplusplus
}
#endif
#endif
