// kvepi_host.cpp -- argument validation, row geometry, the two-stage C ABI
// of the fused KV-cache write epilog and its prepared calls.  Pure host
// code: the GPU is reached only through the launcher and the device query
// of kvepi_kernels.hip and the optional duplicate-slot check of
// kvepi_debug.cpp, each after every check has passed, so every check can run
// (and be tested) without a GPU.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "kvepi.h"
#include "kvepi_plan.h"

namespace {

bool aligned(const void *p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

// Largest power of two <= 16 dividing v (v == 0 counts as 16-aligned).
int32_t pow2_align(uint64_t v) {
  int32_t a = 16;
  while (a > 1 && (v & (uint64_t)(a - 1)) != 0) a >>= 1;
  return a;
}

int32_t min_align(int32_t a, int32_t b) { return a < b ? a : b; }

// What a kvepi_prepared holds: the validated plan and its launch.
constexpr uint64_t PREPARED_MAGIC = 0x3172706970657624ull;
struct prepared_state {
  uint64_t magic;        // PREPARED_MAGIC once kvepi_prepare_ex returned KVEPI_OK
  uint64_t state_bytes;  // sizeof(prepared_state) of the library that wrote it
  kvepi_plan plan;
  kvepi_launch_cfg cfg;  // meaningful for plan.T > 0
};
static_assert(sizeof(prepared_state) <= sizeof(kvepi_prepared),
              "kvepi_prepared must hold a prepared_state");
static_assert(alignof(prepared_state) <= alignof(kvepi_prepared),
              "kvepi_prepared must be aligned for a prepared_state");

// Row geometry ("aclnnKvCompressEpilog" 约束说明 headDim rule;
// "indexer_quant_cache" 约束 headDim/scaleCol rule).
kvepi_status row_geometry(int32_t mode, int64_t d, int32_t group_size,
                          int64_t *cc, int64_t *kc, int64_t *sc) {
  switch (mode) {
    case KVEPI_MODE_FP8_BF16SCALE:
    case KVEPI_MODE_FP8_E8M0: {
      if (d % 64 != 0 || d <= 64 || d > 8192) return KVEPI_ERR_SHAPE;
      if (group_size != 64) return KVEPI_ERR_PARAM;
      const int64_t nope = d - 64;
      const int64_t groups = (nope + 63) / 64;
      const int64_t scale_bytes = mode == KVEPI_MODE_FP8_BF16SCALE ? 2 : 1;
      *cc = nope + 128 + groups * scale_bytes;
      *kc = mode == KVEPI_MODE_FP8_E8M0 ? *cc : (*cc + 31) / 32 * 32;
      *sc = groups;
      return KVEPI_OK;
    }
    case KVEPI_MODE_MXFP4:
      if (d % 32 != 0 || d < 32 || d > 8192) return KVEPI_ERR_SHAPE;
      if (group_size != 32) return KVEPI_ERR_PARAM;
      *cc = (d + 1) / 2;
      *kc = *cc;
      *sc = (d + 31) / 32;
      return KVEPI_OK;
    case KVEPI_MODE_MXFP8:
      if (d % 32 != 0 || d < 32 || d > 8192) return KVEPI_ERR_SHAPE;
      if (group_size != 32) return KVEPI_ERR_PARAM;
      *cc = d;
      *kc = d;
      *sc = d / 32;
      return KVEPI_OK;
    case KVEPI_MODE_FP8_ROW:
      // the whole row is one group: group_size 0 or d
      if (d % 32 != 0 || d < 32 || d > 8192) return KVEPI_ERR_SHAPE;
      if (group_size != 0 && group_size != d) return KVEPI_ERR_PARAM;
      *cc = d;
      *kc = d;
      *sc = 1;
      return KVEPI_OK;
    case KVEPI_MODE_FP4_NOPE: {
      // quantMode=2: concatCol = 64 + (d-64)/2 + ((d-64)/G)*2, padded to 32
      // bytes; G in {16, 32, 64} dividing d-64
      if (d % 64 != 0 || d <= 64 || d > 8192) return KVEPI_ERR_SHAPE;
      if (group_size != 16 && group_size != 32 && group_size != 64) return KVEPI_ERR_PARAM;
      if ((d - 64) % group_size != 0) return KVEPI_ERR_SHAPE;
      *cc = 64 + (d - 64) / 2 + ((d - 64) / group_size) * 2;
      *kc = (*cc + 31) / 32 * 32;
      *sc = (d - 64) / group_size;
      return KVEPI_OK;
    }
    case KVEPI_MODE_BF16_SPLIT:
      if (d % 64 != 0 || d <= 64 || d > 8192) return KVEPI_ERR_SHAPE;
      *cc = d - 64;
      *kc = d - 64;
      *sc = 64;
      return KVEPI_OK;
    default:
      return KVEPI_ERR_UNSUPPORTED;
  }
}

// Checks one paged cache and returns its byte geometry.
kvepi_status check_cache(const kvepi_cache *c, int64_t elem, int64_t min_cols,
                         int64_t *pitch, int64_t *bstride, int32_t *align) {
  if (c == nullptr || c->data == nullptr) return KVEPI_ERR_NULLPTR;
  if (c->block_num <= 0 || c->block_size <= 0 || c->head_dim <= 0)
    return KVEPI_ERR_SHAPE;
  if (c->block_num > INT32_MAX || c->block_size > INT32_MAX ||
      c->block_num * c->block_size > INT32_MAX)
    return KVEPI_ERR_SHAPE;
  if (c->head_dim < min_cols) return KVEPI_ERR_SHAPE;
  if (c->head_dim > (INT64_C(1) << 40) / c->block_size) return KVEPI_ERR_SHAPE;
  if (c->block_stride < c->block_size * c->head_dim) return KVEPI_ERR_LAYOUT;
  if (c->block_stride > (INT64_C(1) << 46) / c->block_num) return KVEPI_ERR_SHAPE;
  if (!aligned(c->data, (uintptr_t)elem)) return KVEPI_ERR_LAYOUT;
  *pitch = c->head_dim * elem;
  *bstride = c->block_stride * elem;
  *align = min_align(pow2_align(reinterpret_cast<uintptr_t>(c->data)),
                     min_align(pow2_align((uint64_t)*pitch),
                               pow2_align((uint64_t)*bstride)));
  return KVEPI_OK;
}

}  // namespace

kvepi_status kvepi_validate(const void *x, int64_t num_tokens, int64_t d,
                            int64_t x_row_stride, const void *gamma,
                            const void *cos, const void *sin,
                            const int32_t *slot_mapping,
                            const kvepi_cache *cache,
                            const kvepi_cache *cache_aux, int32_t quant_mode,
                            int32_t group_size, float eps, const kvepi_options *opt,
                            kvepi_plan *p) {
  if (quant_mode == KVEPI_MODE_HIF8_FP4) return KVEPI_ERR_UNSUPPORTED;
  const kvepi_options o = opt != nullptr ? *opt : kvepi_options{0, 0, 0, 0, 0};
  if (o.x_dtype != KVEPI_X_BF16 && o.x_dtype != KVEPI_X_FP16) return KVEPI_ERR_PARAM;
  if (o.index_mode < KVEPI_INDEX_SLOT || o.index_mode > KVEPI_INDEX_BATCH_START)
    return KVEPI_ERR_PARAM;
  if (o.reserved != 0) return KVEPI_ERR_PARAM;
  const int32_t rope_dim = o.rope_dim == 0 ? 64 : o.rope_dim;
  int64_t cc = 0, kc = 0, sc = 0;
  kvepi_status st;
  if (quant_mode == KVEPI_MODE_BF16_SPLIT && rope_dim != 64) {
    // "aclnnKvRmsNormRopeCache", shape notes: Dk + Dv = D, Dk even
    if (rope_dim < 2 || rope_dim % 2 != 0 || rope_dim > 128) return KVEPI_ERR_PARAM;
    const int64_t dv = d - rope_dim;
    if (dv < 8 || dv % 8 != 0 || d > 8192) return KVEPI_ERR_SHAPE;
    cc = kc = dv;
    sc = rope_dim;
  } else {
    if (rope_dim != 64) return KVEPI_ERR_PARAM;
    st = row_geometry(quant_mode, d, group_size, &cc, &kc, &sc);
    if (st != KVEPI_OK) return st;
  }

  if (num_tokens < 0 || num_tokens > INT32_MAX) return KVEPI_ERR_SHAPE;
  if (num_tokens > 0 && (x == nullptr || slot_mapping == nullptr))
    return KVEPI_ERR_NULLPTR;
  // row offsets of x are kept in 32 bits on the device
  if (x_row_stride < d || x_row_stride % 8 != 0 || x_row_stride > (INT64_C(1) << 27))
    return KVEPI_ERR_LAYOUT;
  if (x != nullptr && !aligned(x, 16)) return KVEPI_ERR_LAYOUT;
  if (slot_mapping != nullptr && !aligned(slot_mapping, 4))
    return KVEPI_ERR_LAYOUT;

  const bool has_norm = gamma != nullptr;
  const bool has_rope = cos != nullptr || sin != nullptr;
  if (has_rope && (cos == nullptr || sin == nullptr)) return KVEPI_ERR_PARAM;
  const bool indexer = quant_mode == KVEPI_MODE_MXFP4 || quant_mode == KVEPI_MODE_MXFP8 ||
                       quant_mode == KVEPI_MODE_FP8_ROW;
  if (indexer && (has_norm || has_rope)) return KVEPI_ERR_UNSUPPORTED;
  if (o.x_dtype == KVEPI_X_FP16 && !indexer) return KVEPI_ERR_UNSUPPORTED;
  // batch-major tokens for the index modes other than SLOT
  if (o.index_mode != KVEPI_INDEX_SLOT &&
      (o.seq_len < 1 || o.seq_len > INT32_MAX || num_tokens % o.seq_len != 0))
    return KVEPI_ERR_SHAPE;
  if (quant_mode == KVEPI_MODE_BF16_SPLIT && (!has_norm || !has_rope))
    return KVEPI_ERR_PARAM;
  // the FP4 nope mode leaves the rope bytes of its rows untouched: no RoPE
  if (quant_mode == KVEPI_MODE_FP4_NOPE && has_rope) return KVEPI_ERR_PARAM;
  if (has_norm && (!isfinite(eps) || eps < 0.0f)) return KVEPI_ERR_PARAM;
  if (has_norm && !aligned(gamma, 16)) return KVEPI_ERR_LAYOUT;
  if (has_rope && (!aligned(cos, 16) || !aligned(sin, 16)))
    return KVEPI_ERR_LAYOUT;

  const bool needs_aux = indexer || quant_mode == KVEPI_MODE_BF16_SPLIT;
  if (needs_aux && cache_aux == nullptr) return KVEPI_ERR_NULLPTR;
  if (!needs_aux && cache_aux != nullptr) return KVEPI_ERR_PARAM;

  // element sizes: bf16 caches in the split mode, fp32 scales in the
  // per-row FP8 mode, bytes otherwise
  const int64_t elem = quant_mode == KVEPI_MODE_BF16_SPLIT ? 2 : 1;
  const int64_t aux_elem = quant_mode == KVEPI_MODE_FP8_ROW ? 4 : elem;
  kvepi_plan q{};
  st = check_cache(cache, elem, kc, &q.c_pitch, &q.c_bstride, &q.c_align);
  if (st != KVEPI_OK) return st;
  if (needs_aux) {
    st = check_cache(cache_aux, aux_elem, sc, &q.a_pitch, &q.a_bstride, &q.a_align);
    if (st != KVEPI_OK) return st;
    if (cache_aux->block_num != cache->block_num ||
        cache_aux->block_size != cache->block_size)
      return KVEPI_ERR_SHAPE;
  }
  if (o.index_mode == KVEPI_INDEX_BATCH || o.index_mode == KVEPI_INDEX_BATCH_START) {
    // batch b owns block b: Bcache >= B
    if (num_tokens / o.seq_len > cache->block_num) return KVEPI_ERR_SHAPE;
    if (o.index_mode == KVEPI_INDEX_BATCH_START && o.seq_len > cache->block_size)
      return KVEPI_ERR_SHAPE;
  }

  if (p != nullptr) {
    q.mode = quant_mode;
    q.norm = has_norm;
    q.rope = has_rope;
    q.x_fp16 = o.x_dtype == KVEPI_X_FP16;
    q.index_mode = o.index_mode;
    q.seq_len = o.index_mode == KVEPI_INDEX_SLOT ? 0 : o.seq_len;
    q.T = num_tokens;
    q.d = d;
    q.nope = indexer ? d : d - rope_dim;
    q.rope_dim = rope_dim;
    q.x_stride = x_row_stride;
    q.x = static_cast<const uint16_t *>(x);
    q.gamma = static_cast<const uint16_t *>(gamma);
    q.cos = static_cast<const uint16_t *>(cos);
    q.sin = static_cast<const uint16_t *>(sin);
    q.slots = slot_mapping;
    q.cache = static_cast<uint8_t *>(cache->data);
    q.aux = needs_aux ? static_cast<uint8_t *>(cache_aux->data) : nullptr;
    q.block_size = cache->block_size;
    q.num_slots = cache->block_num * cache->block_size;
    q.concat_col = cc;
    q.kv_cache_col = kc;
    q.scale_col = sc;
    q.group_size = group_size;
    q.eps = eps;
    *p = q;
  }
  return KVEPI_OK;
}

extern "C" {

kvepi_status kvepi_row_bytes(int32_t quant_mode, int64_t d, int32_t group_size,
                             int64_t *concat_col, int64_t *kv_cache_col,
                             int64_t *scale_col) {
  if (quant_mode == KVEPI_MODE_HIF8_FP4) return KVEPI_ERR_UNSUPPORTED;
  int64_t cc = 0, kc = 0, sc = 0;
  kvepi_status st = row_geometry(quant_mode, d, group_size, &cc, &kc, &sc);
  if (st != KVEPI_OK) return st;
  if (concat_col) *concat_col = cc;
  if (kv_cache_col) *kv_cache_col = kc;
  if (scale_col) *scale_col = sc;
  return KVEPI_OK;
}

kvepi_status kvepi_get_workspace_ex(const void *x, int64_t num_tokens, int64_t d,
                                    int64_t x_row_stride, const void *gamma,
                                    const void *cos, const void *sin,
                                    const int32_t *slot_mapping,
                                    const kvepi_cache *cache,
                                    const kvepi_cache *cache_aux,
                                    int32_t quant_mode, int32_t group_size,
                                    float eps, const kvepi_options *options,
                                    uint64_t *workspace_bytes) {
  if (workspace_bytes == nullptr) return KVEPI_ERR_NULLPTR;
  kvepi_status st =
      kvepi_validate(x, num_tokens, d, x_row_stride, gamma, cos, sin,
                     slot_mapping, cache, cache_aux, quant_mode, group_size,
                     eps, options, nullptr);
  if (st != KVEPI_OK) return st;
  *workspace_bytes = 0;
  return KVEPI_OK;
}

kvepi_status kvepi_run_ex(const void *x, int64_t num_tokens, int64_t d,
                          int64_t x_row_stride, const void *gamma,
                          const void *cos, const void *sin,
                          const int32_t *slot_mapping, const kvepi_cache *cache,
                          const kvepi_cache *cache_aux, int32_t quant_mode,
                          int32_t group_size, float eps, const kvepi_options *options,
                          void *workspace, uint64_t workspace_bytes, void *stream) {
  (void)workspace;
  (void)workspace_bytes;  // the epilog needs no workspace (size 0)
  kvepi_plan plan;
  kvepi_status st =
      kvepi_validate(x, num_tokens, d, x_row_stride, gamma, cos, sin,
                     slot_mapping, cache, cache_aux, quant_mode, group_size,
                     eps, options, &plan);
  if (st != KVEPI_OK) return st;
  if (plan.T == 0) return KVEPI_OK;
  st = kvepi_debug_check_slots(plan, slot_mapping, stream);
  if (st != KVEPI_OK) return st;
  return kvepi_launch(plan, stream);
}

kvepi_status kvepi_prepare_ex(const void *x, int64_t num_tokens, int64_t d,
                              int64_t x_row_stride, const void *gamma,
                              const void *cos, const void *sin,
                              const int32_t *slot_mapping, const kvepi_cache *cache,
                              const kvepi_cache *cache_aux, int32_t quant_mode,
                              int32_t group_size, float eps, const kvepi_options *options,
                              kvepi_prepared *prepared) {
  if (prepared == nullptr) return KVEPI_ERR_NULLPTR;
  memset(prepared, 0, sizeof *prepared);  // invalid unless every step succeeds
  prepared_state ps;
  memset(&ps, 0, sizeof ps);
  kvepi_status st =
      kvepi_validate(x, num_tokens, d, x_row_stride, gamma, cos, sin,
                     slot_mapping, cache, cache_aux, quant_mode, group_size,
                     eps, options, &ps.plan);
  if (st != KVEPI_OK) return st;
  if (ps.plan.T > 0) {
    st = kvepi_configure(ps.plan, &ps.cfg);
    if (st != KVEPI_OK) return st;
  }
  ps.magic = PREPARED_MAGIC;
  ps.state_bytes = sizeof ps;
  memcpy(prepared, &ps, sizeof ps);
  return KVEPI_OK;
}

kvepi_status kvepi_run_prepared(const kvepi_prepared *prepared, void *stream) {
  if (prepared == nullptr) return KVEPI_ERR_NULLPTR;
  prepared_state ps;
  memcpy(&ps, prepared, sizeof ps);
  if (ps.magic != PREPARED_MAGIC || ps.state_bytes != sizeof ps) return KVEPI_ERR_PARAM;
  if (ps.plan.T == 0) return KVEPI_OK;
  int32_t dev = -1;
  kvepi_status st = kvepi_current_device(&dev);
  if (st != KVEPI_OK) return st;
  if (dev != ps.cfg.device) return KVEPI_ERR_PARAM;
  st = kvepi_debug_check_slots(ps.plan, ps.plan.slots, stream);
  if (st != KVEPI_OK) return st;
  return kvepi_enqueue(ps.cfg, stream);
}

kvepi_status kvepi_get_workspace(const void *x, int64_t num_tokens, int64_t d,
                                 int64_t x_row_stride, const void *gamma,
                                 const void *cos, const void *sin,
                                 const int32_t *slot_mapping,
                                 const kvepi_cache *cache,
                                 const kvepi_cache *cache_aux,
                                 int32_t quant_mode, int32_t group_size,
                                 float eps, uint64_t *workspace_bytes) {
  return kvepi_get_workspace_ex(x, num_tokens, d, x_row_stride, gamma, cos, sin, slot_mapping,
                                cache, cache_aux, quant_mode, group_size, eps, nullptr,
                                workspace_bytes);
}

kvepi_status kvepi_run(const void *x, int64_t num_tokens, int64_t d,
                       int64_t x_row_stride, const void *gamma,
                       const void *cos, const void *sin,
                       const int32_t *slot_mapping, const kvepi_cache *cache,
                       const kvepi_cache *cache_aux, int32_t quant_mode,
                       int32_t group_size, float eps, void *workspace,
                       uint64_t workspace_bytes, void *stream) {
  return kvepi_run_ex(x, num_tokens, d, x_row_stride, gamma, cos, sin, slot_mapping, cache,
                      cache_aux, quant_mode, group_size, eps, nullptr, workspace,
                      workspace_bytes, stream);
}

const char *kvepi_status_str(kvepi_status s) {
  switch (s) {
    case KVEPI_OK: return "KVEPI_OK";
    case KVEPI_ERR_NULLPTR: return "KVEPI_ERR_NULLPTR: a required pointer is NULL";
    case KVEPI_ERR_SHAPE: return "KVEPI_ERR_SHAPE: a size violates the operation's constraints";
    case KVEPI_ERR_LAYOUT: return "KVEPI_ERR_LAYOUT: invalid stride, alignment or cache layout";
    case KVEPI_ERR_PARAM: return "KVEPI_ERR_PARAM: invalid group size, eps or optional-input combination";
    case KVEPI_ERR_UNSUPPORTED: return "KVEPI_ERR_UNSUPPORTED: quant mode or combination not implemented";
    case KVEPI_ERR_WORKSPACE: return "KVEPI_ERR_WORKSPACE: workspace too small";
    case KVEPI_ERR_RUNTIME: return "KVEPI_ERR_RUNTIME: the HIP runtime refused the launch";
  }
  return "KVEPI_ERR_UNKNOWN";
}

int32_t kvepi_version(void) { return KVEPI_VERSION; }

}  // extern "C"
