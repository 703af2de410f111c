/*
 * kvepi.h -- C ABI of the fused KV-cache write epilog for AMD Instinct MI355X
 * (gfx950).
 *
 * For each token row t of a bf16 activation x[T, d] whose slot_mapping[t] is
 * a valid slot, the library writes one packed row into a paged cache
 * [blockNum, blockSize, 1, headDim] in place:
 *
 *   1. optional RMSNorm over the nope segment x[t, 0:d-64]
 *        ("aclnnKvRmsNormRopeCache", 计算公式 (2) rmsNorm),
 *   2. optional interleaved RoPE over the rope segment x[t, d-64:d], giving a
 *      half-split result ("aclnnKvRmsNormRopeCache", 计算公式 (1)),
 *   3. per-group amax dynamic quantisation of the nope segment
 *        ("aclnnKvCompressEpilog", 计算公式 scenes 1 and 2) or of the whole
 *        row in MX-FP4 ("indexer_quant_cache", 接口功能),
 *   4. the scatter of the packed row to slot slot_mapping[t]; tokens whose
 *      slot is -1 are skipped and every byte outside the written rows keeps
 *      its value ("aclnnKvCompressEpilog", 约束说明; "indexer_quant_cache",
 *      语义说明).
 *
 * The call is split in two stages, as on the pages: kvepi_get_workspace
 * validates the arguments and returns the workspace size, kvepi_run validates
 * again and launches asynchronously on the caller's HIP stream
 * ("aclnnKvCompressEpilog", the two-stage interface description).
 *
 * Conventions shared by every entry point
 *  - bf16 data is passed as 16-bit little-endian bit patterns.
 *  - Pointers named x, gamma, cos, sin, slot_mapping and kvepi_cache.data are
 *    DEVICE pointers; they are checked for NULL and alignment only, never
 *    dereferenced on the host.  Struct and out-parameter pointers are HOST
 *    pointers.
 *  - The caller owns every buffer, the workspace and the stream.  The library
 *    allocates nothing and keeps no pointer after a call returns.
 *  - kvepi_run is asynchronous: buffers must stay alive and unmodified until
 *    the stream has passed the launched kernel.  The library never
 *    synchronises the stream (except under the KVEPI_CHECK_SLOTS debug check
 *    described at kvepi_run).
 *  - Every check runs before any launch, so a call that returns an error
 *    writes nothing.
 *  - Results are deterministic: the same inputs give the same bytes
 *    ("aclnnKvCompressEpilog", 约束说明: deterministic by default).
 */
#ifndef KVEPI_H
#define KVEPI_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVEPI_VERSION 140 /* 1.4.0: prepared calls (kvepi_prepare_ex) */

#if defined(__GNUC__) || defined(__clang__)
#define KVEPI_API __attribute__((visibility("default")))
#else
#define KVEPI_API
#endif

typedef enum kvepi_status {
  KVEPI_OK = 0,
  KVEPI_ERR_NULLPTR = 1,     /* a required pointer is NULL                  */
  KVEPI_ERR_SHAPE = 2,       /* a size violates the operation's constraints */
  KVEPI_ERR_LAYOUT = 3,      /* strides / alignment / cache layout invalid  */
  KVEPI_ERR_PARAM = 4,       /* group size, eps or optional-input mismatch  */
  KVEPI_ERR_UNSUPPORTED = 5, /* quant mode or combination not implemented   */
  KVEPI_ERR_WORKSPACE = 6,   /* workspace smaller than kvepi_get_workspace  */
  KVEPI_ERR_RUNTIME = 7      /* the HIP runtime refused the launch          */
} kvepi_status;

/* quant_mode values.
 *  0  FP8 E4M3 codes per group of 64 nope values, scale = amax/448 stored as
 *     bf16 ("aclnnKvCompressEpilog" 计算公式, quantMode=0).
 *     Row: [d-64 codes | 64 rope bf16 | ceil((d-64)/64) bf16 scales | zero pad
 *     to a multiple of 32 bytes].
 *  1  as 0, scale stored as one e8m0 byte, the power of two 2^E with E the
 *     smallest integer such that amax <= 448 * 2^E (quantMode=1).  Row is not
 *     padded.
 *  2  quantMode=2 of the page (HiFloat8 rope + FP4 nope): the HiFloat8
 *     encoding is not defined there -> KVEPI_ERR_UNSUPPORTED; its nope half
 *     is mode 7.
 *  3  MX-FP4: E2M1 codes of the whole row, two per byte (element 2j in the
 *     low nibble), one e8m0 scale (amax <= 6 * 2^E) per group of 32 written
 *     to cache_aux ("indexer_quant_cache", mxfp4 mode).
 *  4  bf16 split: RMSNorm output -> cache (ckv, headDim >= d-64 bf16),
 *     RoPE output -> cache_aux (k, headDim >= 64 bf16)
 *     ("aclnnKvRmsNormRopeCache", 接口功能).
 *  5  MX-FP8: E4M3 codes of the whole row, one byte each, one e8m0 scale
 *     (amax <= 448 * 2^E) per group of 32 written to cache_aux (uint8)
 *     ("indexer_quant_cache", mxfp8 mode).
 *  6  FP8 per row: the whole row is one group; E4M3 codes of x / s with
 *     s = amax / 448 in fp32 (a zero row: s = 0, all codes 0), s written as
 *     one little-endian fp32 value to cache_aux, whose elements are 4-byte
 *     floats ("indexer_quant_cache", fp8 mode: cache_scale is FLOAT).
 *  7  quantMode=2's FP4 nope segment ("aclnnKvCompressEpilog" 计算公式
 *     scene 3, 约束说明): the d-64 nope values in groups of group_size (16,
 *     32 or 64), scale = amax/6 stored as bf16, E2M1 codes of x / scale (the
 *     stored scale) two per byte (element 2j in the low nibble).
 *     Row: [64 rope bytes, NOT written | (d-64)/2 code bytes |
 *     (d-64)/group_size bf16 scales | zero pad to a multiple of 32 bytes]:
 *     the rope segment's HiFloat8 codes are left untouched.  Takes gamma
 *     (RMSNorm over the nope values first), not cos/sin; bf16 x only.
 * Modes 3, 5 and 6 are the indexer modes: they take neither gamma nor
 * cos/sin and need cache_aux.
 * NaN: the RMSNorm of an all-zero row with eps = 0 is 0/0 = NaN; NaN values
 * are left out of a group's amax (a group of NaNs gets scale 0 and codes 0),
 * and a NaN quotient is encoded as 0x7F (E4M3) or 0x7 (E2M1).  NaN or
 * infinite inputs x are outside the contract.
 */
#define KVEPI_MODE_FP8_BF16SCALE 0
#define KVEPI_MODE_FP8_E8M0 1
#define KVEPI_MODE_HIF8_FP4 2
#define KVEPI_MODE_MXFP4 3
#define KVEPI_MODE_BF16_SPLIT 4
#define KVEPI_MODE_MXFP8 5
#define KVEPI_MODE_FP8_ROW 6
#define KVEPI_MODE_FP4_NOPE 7

/* A paged cache [block_num, block_size, 1, head_dim] ("aclnnKvCompressEpilog",
 * 约束说明: four dimensions, dimension -2 fixed at 1, only the block
 * dimension may be non-contiguous; "indexer_quant_cache" 约束: blocks may be
 * laid out loosely but are contiguous inside).
 *  data          DEVICE pointer to element [0,0,0,0]; any byte alignment.
 *  head_dim      elements per row (uint8 caches: bytes; bf16 caches for mode
 *                4: 2-byte elements; the mode-6 scale cache: 4-byte floats).
 *                data must be aligned to the element size.
 *  block_stride  elements between consecutive blocks, >= block_size*head_dim.
 * Slot s lives at data + ((s / block_size) * block_stride +
 * (s % block_size) * head_dim) * element_size.  num_slots = block_num *
 * block_size must be <= 2^31 - 1. */
typedef struct kvepi_cache {
  void *data;
  int64_t block_num;
  int64_t block_size;
  int64_t head_dim;
  int64_t block_stride;
} kvepi_cache;

/* Row geometry of a mode ("aclnnKvCompressEpilog", 约束说明, headDim rule:
 * concatCol = (d-64) + 128 + ceil((d-64)/64) * scaleBytes with scaleBytes 2
 * for mode 0 and 1 for mode 1; kvCacheCol = concatCol for mode 1 and
 * concatCol rounded up to 32 bytes for mode 0; e.g. d=256 in mode 1 gives
 * 323.  "indexer_quant_cache", 约束: MX-FP4 codes take ceil(d/2) bytes and
 * scaleCol = ceil(d/32), e.g. d=128 gives 4; MX-FP8 codes take d bytes with
 * the same scaleCol; the per-row FP8 mode takes d bytes and scaleCol = 1;
 * "aclnnKvCompressEpilog", 约束说明, quantMode=2: concatCol = 64 + (d-64)/2 +
 * ((d-64)/G) * 2, padded to 32 bytes, e.g. d=576, G=32 gives 352.)
 *   concat_col    bytes of data per row (mode 4: ckv elements per row)
 *   kv_cache_col  bytes written per row, the minimum headDim (mode 4: d-64)
 *   scale_col     scale entries per row (modes 3, 5, 6: the minimum
 *                 cache_aux headDim; mode 4: 64, the k-cache elements per row;
 *                 mode 7: the bf16 scales in the row)
 * Any out-pointer may be NULL.  Errors: KVEPI_ERR_UNSUPPORTED for an unknown
 * mode or mode 2, KVEPI_ERR_SHAPE for d outside the mode's range
 * (modes 0/1/4/7: d % 64 == 0 and 64 < d <= 8192; modes 3/5/6: d % 32 == 0
 * and 32 <= d <= 8192), KVEPI_ERR_PARAM for a group size other than 64
 * (modes 0/1), 32 (modes 3/5), 0 or d (mode 6) or 16/32/64 (mode 7). */
KVEPI_API kvepi_status kvepi_row_bytes(int32_t quant_mode, int64_t d, int32_t group_size,
                             int64_t *concat_col, int64_t *kv_cache_col,
                             int64_t *scale_col);

/* Stage one: validate and report the workspace size (always 0 in this
 * implementation; NULL workspaces are accepted).
 *
 *  x             DEVICE, bf16 [num_tokens, d], rows x_row_stride elements
 *                apart; 16-byte aligned base, x_row_stride % 8 == 0 and
 *                d <= x_row_stride <= 2^27.  Leading dimensions of the caller's
 *                tensor are flattened into num_tokens
 *                ("aclnnKvCompressEpilog", 约束说明, slotMapping shape rule).
 *  gamma         DEVICE, bf16 [d-64], 16-byte aligned, or NULL for no
 *                RMSNorm (required in mode 4, rejected in modes 3, 5, 6).
 *  cos, sin      DEVICE, bf16 [num_tokens, 64] contiguous, 16-byte aligned,
 *                both or neither; NULL for no RoPE (the rope columns are then
 *                copied unchanged).  Required in mode 4, rejected in modes
 *                3, 5, 6 (KVEPI_ERR_UNSUPPORTED) and 7 (KVEPI_ERR_PARAM: the
 *                rope bytes are not written).
 *  slot_mapping  DEVICE, int32 [num_tokens], 4-byte aligned.  -1 skips the
 *                token; any value outside [0, num_slots) is skipped too.
 *                Valid values must be distinct; with duplicates the result of
 *                the repeated rows is unspecified ("aclnnKvCompressEpilog",
 *                约束说明).
 *  cache         HOST struct describing the main cache (uint8; bf16 in mode
 *                4).  headDim >= kv_cache_col.
 *  cache_aux     HOST struct, NULL except in modes 3 and 5 (cache_scale,
 *                uint8, headDim >= scale_col), mode 6 (cache_scale, fp32,
 *                headDim >= 1) and mode 4 (k cache, bf16, headDim >= 64);
 *                same block_num and block_size as cache.
 *  quant_mode    KVEPI_MODE_*.
 *  group_size    64 (modes 0, 1), 32 (modes 3, 5), 0 or d (mode 6), 16, 32
 *                or 64 (mode 7), ignored in mode 4.
 *  eps           RMSNorm epsilon, finite and >= 0 (used only with gamma).
 *  workspace_bytes  HOST out-parameter.
 * num_tokens == 0 is valid and makes kvepi_run a no-op. */
KVEPI_API kvepi_status kvepi_get_workspace(const void *x, int64_t num_tokens, int64_t d,
                                 int64_t x_row_stride, const void *gamma,
                                 const void *cos, const void *sin,
                                 const int32_t *slot_mapping,
                                 const kvepi_cache *cache,
                                 const kvepi_cache *cache_aux,
                                 int32_t quant_mode, int32_t group_size,
                                 float eps, uint64_t *workspace_bytes);

/* Stage two: validate as kvepi_get_workspace, then enqueue the epilog on
 * `stream` (a hipStream_t; NULL = the null stream of the current device).
 * The current HIP device must be the one holding the buffers.  Returns
 * KVEPI_ERR_WORKSPACE if workspace_bytes is below the stage-one size and
 * KVEPI_ERR_RUNTIME if the launch is refused (for example on a device that
 * is not gfx950).
 * The launch uses one persistent workgroup per resident slot of the device.
 * The environment variable KVEPI_MAX_WAVES (a multiple of 4, read at every
 * call) caps the number of wavefronts; it exists for tests of the kernel's
 * multi-iteration paths and never changes the result.
 * Debug aid: with the environment variable KVEPI_CHECK_SLOTS set (to anything
 * but "0"; read at every call), kvepi_run and kvepi_run_ex copy slot_mapping
 * to the host, synchronously on `stream`, and return KVEPI_ERR_PARAM before
 * any launch if two tokens name the same row (index mode KVEPI_INDEX_SLOT
 * only; a failed copy returns KVEPI_ERR_RUNTIME).  Repeated slots are
 * otherwise not detected: their rows are unspecified. */
KVEPI_API kvepi_status kvepi_run(const void *x, int64_t num_tokens, int64_t d,
                       int64_t x_row_stride, const void *gamma,
                       const void *cos, const void *sin,
                       const int32_t *slot_mapping, const kvepi_cache *cache,
                       const kvepi_cache *cache_aux, int32_t quant_mode,
                       int32_t group_size, float eps, void *workspace,
                       uint64_t workspace_bytes, void *stream);

/* ---- options: fp16 rows and index modes (version 1.1) -------------------
 *
 * The _ex entry points take the arguments of kvepi_get_workspace / kvepi_run
 * plus an options struct (HOST pointer; NULL = every field 0, which is
 * exactly the behaviour of the entry points above).
 *
 *  x_dtype     KVEPI_X_BF16, or KVEPI_X_FP16: x holds IEEE binary16 values
 *              ("indexer_quant_cache" 接口功能: float16 or bfloat16 x); only
 *              in the indexer modes 3, 5, 6, otherwise KVEPI_ERR_UNSUPPORTED.
 *  index_mode  how the int32 array passed as slot_mapping places token t
 *              (tokens are batch-major, t = b * seq_len + s, B = T / seq_len):
 *    KVEPI_INDEX_SLOT        [T]: the token's slot, as above.
 *    KVEPI_INDEX_BATCH       [B, seq_len]: row index[b, s] of batch b's rows,
 *                            which are block b of the cache (block_size rows:
 *                            the cache is [Bcache, Scache, 1, headDim] with
 *                            Bcache = block_num >= B, Scache = block_size);
 *                            values in [-1, Scache), repeats across batches
 *                            allowed ("aclnnKvRmsNormRopeCache", index
 *                            constraints, Norm mode).
 *    KVEPI_INDEX_BLOCK       [B, ceil(seq_len / block_size)]: entry c names
 *                            the block (value / block_size) taking tokens
 *                            c*block_size .. of batch b, token s at row
 *                            s % block_size of it; the blocks named must be
 *                            distinct ("aclnnKvRmsNormRopeCache", index
 *                            constraints, PA_BLK modes).
 *    KVEPI_INDEX_BATCH_START [B]: token s of batch b goes to row index[b] + s
 *                            of batch b's rows (block b); needs
 *                            seq_len <= block_size (the blog on
 *                            aclnnDequantRopeQuantKvcache, cache modes,
 *                            contiguous mode).
 *              -1, and any value that would place a token outside the cache
 *              (or outside its batch's rows), skips the token(s).
 *  seq_len     tokens per batch for the index modes other than SLOT: >= 1,
 *              dividing num_tokens; B must not exceed block_num in the
 *              BATCH and BATCH_START modes (KVEPI_ERR_SHAPE otherwise).
 *  rope_dim    length Dk of the rope segment, 0 meaning 64.  Modes 0 and 1
 *              fix it at 64 ("aclnnKvCompressEpilog", 接口功能: the last 64
 *              columns; anything else is KVEPI_ERR_PARAM).  The bf16 split
 *              mode 4 takes any even Dk in [2, 128] with Dv = d - Dk a
 *              multiple of 8 and at least 8 ("aclnnKvRmsNormRopeCache",
 *              shape notes: Dk + Dv = D, Dk even; KVEPI_ERR_SHAPE
 *              otherwise): RMSNorm over Dv (gamma [Dv], the ckv cache rows
 *              Dv elements), RoPE over Dk (cos / sin [T, Dk], the k cache
 *              rows Dk elements).  x_row_stride stays a multiple of 8, so
 *              a d that is not (Dk not a multiple of 8) needs padded rows.
 */
#define KVEPI_X_BF16 0
#define KVEPI_X_FP16 1
#define KVEPI_INDEX_SLOT 0
#define KVEPI_INDEX_BATCH 1
#define KVEPI_INDEX_BLOCK 2
#define KVEPI_INDEX_BATCH_START 3

typedef struct kvepi_options {
  int32_t x_dtype;
  int32_t index_mode;
  int64_t seq_len;
  int32_t rope_dim;
  int32_t reserved; /* must be 0 */
} kvepi_options;

KVEPI_API kvepi_status kvepi_get_workspace_ex(const void *x, int64_t num_tokens, int64_t d,
                                    int64_t x_row_stride, const void *gamma,
                                    const void *cos, const void *sin,
                                    const int32_t *slot_mapping,
                                    const kvepi_cache *cache,
                                    const kvepi_cache *cache_aux,
                                    int32_t quant_mode, int32_t group_size,
                                    float eps, const kvepi_options *options,
                                    uint64_t *workspace_bytes);

KVEPI_API kvepi_status kvepi_run_ex(const void *x, int64_t num_tokens, int64_t d,
                          int64_t x_row_stride, const void *gamma,
                          const void *cos, const void *sin,
                          const int32_t *slot_mapping, const kvepi_cache *cache,
                          const kvepi_cache *cache_aux, int32_t quant_mode,
                          int32_t group_size, float eps, const kvepi_options *options,
                          void *workspace, uint64_t workspace_bytes, void *stream);

/* ---- prepared calls (version 1.4) ----------------------------------------
 *
 * For callers that launch the same call again and again over fixed buffers
 * (a serving loop that refills its x and slot_mapping buffers every step):
 * kvepi_prepare_ex does the work of a kvepi_run_ex call that does not depend
 * on the buffers' contents once -- the validation, the choice of kernel and
 * its grid on the current device -- and stores it in a caller-owned
 * kvepi_prepared; kvepi_run_prepared then only checks the device and
 * enqueues the kernel.  A run of a prepared call writes exactly what
 * kvepi_run_ex with the same arguments writes for the buffers' contents at
 * the time the kernel executes.
 *
 *  kvepi_prepare_ex  takes the arguments of kvepi_get_workspace_ex (the
 *        workspace size is 0 for every call, so there is no out-parameter)
 *        and a HOST pointer to the kvepi_prepared to fill.  It returns what
 *        kvepi_get_workspace_ex returns for the same arguments; then, for
 *        num_tokens > 0, it reads the current HIP device (KVEPI_ERR_RUNTIME
 *        if that fails) and the KVEPI_MAX_WAVES cap described at kvepi_run.
 *        It launches nothing and never synchronises.  On any error status
 *        *prepared is marked invalid.
 *  kvepi_run_prepared  enqueues a prepared call on `stream` (as kvepi_run).
 *        KVEPI_ERR_NULLPTR for a NULL prepared, KVEPI_ERR_PARAM for a struct
 *        whose header does not mark it as filled by a kvepi_prepare_ex that
 *        returned KVEPI_OK (a zeroed or uninitialised struct, or one whose
 *        preparation failed), or when the current HIP device is not the one
 *        that was current at preparation; only that header is checked, so
 *        running a struct whose other bytes changed after preparation is
 *        undefined;
 *        KVEPI_ERR_RUNTIME if the launch is refused.  A prepared call of 0
 *        tokens is a no-op.  The KVEPI_CHECK_SLOTS debug check is applied at
 *        every run, as in kvepi_run.
 *
 * Ownership.  The kvepi_prepared belongs to the caller; it holds the device
 * pointers it was prepared with and nothing else (no allocation, no pointer
 * into itself): it may be copied bytewise, used from several threads at
 * once, and dropped without any call.  It is meaningful only in the process
 * that prepared it, while this library stays loaded (it names the library's
 * kernel by address).  Those buffers must stay allocated,
 * at the same addresses, for as long as the prepared call is run; their
 * contents may change between runs (the stream orders the kernel after the
 * writes enqueued before it, as for any launch).
 */
#define KVEPI_PREPARED_BYTES 1024

typedef struct kvepi_prepared {
  uint64_t opaque[KVEPI_PREPARED_BYTES / 8];
} kvepi_prepared;

KVEPI_API kvepi_status kvepi_prepare_ex(const void *x, int64_t num_tokens, int64_t d,
                              int64_t x_row_stride, const void *gamma,
                              const void *cos, const void *sin,
                              const int32_t *slot_mapping, const kvepi_cache *cache,
                              const kvepi_cache *cache_aux, int32_t quant_mode,
                              int32_t group_size, float eps, const kvepi_options *options,
                              kvepi_prepared *prepared);

KVEPI_API kvepi_status kvepi_run_prepared(const kvepi_prepared *prepared, void *stream);

/* Static text for a status code (never NULL). */
KVEPI_API const char *kvepi_status_str(kvepi_status status);

/* KVEPI_VERSION of the built library. */
KVEPI_API int32_t kvepi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* KVEPI_H */
