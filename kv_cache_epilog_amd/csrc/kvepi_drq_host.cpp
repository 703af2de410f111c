// kvepi_drq_host.cpp -- argument validation and the two-stage C ABI of the
// dequant -> RoPE -> static int8 quantisation -> KV cache operator (the blog
// on aclnnDequantRopeQuantKvcache: 约束说明 and the parameter semantics).
// Pure host code: nothing here touches the GPU.
#include <stdint.h>

#include "kvepi_drq.h"
#include "kvepi_drq_plan.h"

namespace {

bool aligned(const void *p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

bool is16(int32_t dt) { return dt == KVEPI_DT_BF16 || dt == KVEPI_DT_FP16; }

kvepi_status check_cache(const kvepi_cache &c, int64_t row) {
  if (c.data == nullptr) return KVEPI_ERR_NULLPTR;
  if (c.block_num <= 0 || c.block_size <= 0 || c.head_dim <= 0) return KVEPI_ERR_SHAPE;
  if (c.block_num > INT32_MAX || c.block_size > INT32_MAX ||
      c.block_num * c.block_size > INT32_MAX)
    return KVEPI_ERR_SHAPE;
  if (c.head_dim < row) return KVEPI_ERR_SHAPE;
  if (c.head_dim > (INT64_C(1) << 40) / c.block_size) return KVEPI_ERR_SHAPE;
  if (c.block_stride < c.block_size * c.head_dim) return KVEPI_ERR_LAYOUT;
  if (c.block_stride > (INT64_C(1) << 46) / c.block_num) return KVEPI_ERR_SHAPE;
  // the codes of 8 channels leave as one 8-byte store
  if (!aligned(c.data, 8) || c.head_dim % 8 != 0 || c.block_stride % 8 != 0)
    return KVEPI_ERR_LAYOUT;
  return KVEPI_OK;
}

}  // namespace

kvepi_status kvepi_drq_validate(const kvepi_drq_params *pp, kvepi_drq_plan *plan) {
  if (pp == nullptr) return KVEPI_ERR_NULLPTR;
  const kvepi_drq_params &p = *pp;
  // dtypes (约束说明 4, 5)
  if (!is16(p.out_dtype)) return KVEPI_ERR_PARAM;
  const bool dequant = p.x_dtype == KVEPI_DT_INT32;
  if (!dequant && p.x_dtype != p.out_dtype) return KVEPI_ERR_PARAM;
  if (dequant && p.weight_scale == nullptr) return KVEPI_ERR_NULLPTR;
  if (!dequant && (p.weight_scale || p.act_scale || p.bias)) return KVEPI_ERR_PARAM;
  if (p.bias && !(p.bias_dtype == KVEPI_DT_FP32 || p.bias_dtype == KVEPI_DT_INT32 ||
                  is16(p.bias_dtype)))
    return KVEPI_ERR_PARAM;
  // shapes (约束说明 6; the head dim of 16-value units)
  if (p.nq < 1 || p.nkv < 1 || p.head_dim < 16 || p.head_dim % 16 != 0) return KVEPI_ERR_SHAPE;
  const int64_t H = (int64_t)(p.nq + 2 * (int64_t)p.nkv) * p.head_dim;
  if (H > 4096 || H % 64 != 0) return KVEPI_ERR_SHAPE;
  if (p.num_tokens < 0 || p.num_tokens > INT32_MAX) return KVEPI_ERR_SHAPE;
  if (p.num_tokens * (H / 8) > INT32_MAX) return KVEPI_ERR_SHAPE;
  if (p.x_row_stride < H || p.x_row_stride % 8 != 0 || p.x_row_stride > (INT64_C(1) << 28))
    return KVEPI_ERR_LAYOUT;
  // required pointers
  const bool any = p.num_tokens > 0;
  if (any && (p.x == nullptr || p.cos == nullptr || p.sin == nullptr || p.indices == nullptr ||
              p.q_out == nullptr))
    return KVEPI_ERR_NULLPTR;
  if (p.scale_k == nullptr || p.scale_v == nullptr) return KVEPI_ERR_NULLPTR;
  if ((p.k_out == nullptr) != (p.v_out == nullptr)) return KVEPI_ERR_PARAM;
  // alignment: every 8-value piece is one or two 16-byte loads / stores
  const void *a16[] = {p.x, p.cos, p.sin, p.weight_scale, p.bias, p.scale_k, p.scale_v,
                       p.offset_k, p.offset_v, p.q_out, p.k_out, p.v_out};
  for (const void *q : a16)
    if (q != nullptr && !aligned(q, 16)) return KVEPI_ERR_LAYOUT;
  if (p.act_scale && !aligned(p.act_scale, 4)) return KVEPI_ERR_LAYOUT;
  if (p.indices && !aligned(p.indices, 4)) return KVEPI_ERR_LAYOUT;
  // caches
  const int64_t row = (int64_t)p.nkv * p.head_dim;
  kvepi_status st = check_cache(p.k_cache, row);
  if (st != KVEPI_OK) return st;
  st = check_cache(p.v_cache, row);
  if (st != KVEPI_OK) return st;
  if (p.k_cache.block_num != p.v_cache.block_num ||
      p.k_cache.block_size != p.v_cache.block_size)
    return KVEPI_ERR_SHAPE;
  // cache mode
  if (p.cache_mode == KVEPI_DRQ_CONTIGUOUS) {
    if (p.seq_len < 1 || p.seq_len > INT32_MAX || p.num_tokens % p.seq_len != 0)
      return KVEPI_ERR_SHAPE;
    if (p.num_tokens / p.seq_len > p.k_cache.block_num || p.seq_len > p.k_cache.block_size)
      return KVEPI_ERR_SHAPE;
  } else if (p.cache_mode != KVEPI_DRQ_PAGE) {
    return KVEPI_ERR_PARAM;
  }
  if (plan) {
    plan->p = p;
    plan->H = H;
    plan->units = p.num_tokens * (H / 16);
    plan->k_pitch = p.k_cache.head_dim;
    plan->k_bstride = p.k_cache.block_stride;
    plan->v_pitch = p.v_cache.head_dim;
    plan->v_bstride = p.v_cache.block_stride;
  }
  return KVEPI_OK;
}

extern "C" {

kvepi_status kvepi_drq_get_workspace(const kvepi_drq_params *params, uint64_t *workspace_bytes) {
  if (workspace_bytes == nullptr) return KVEPI_ERR_NULLPTR;
  const kvepi_status st = kvepi_drq_validate(params, nullptr);
  if (st != KVEPI_OK) return st;
  *workspace_bytes = 0;
  return KVEPI_OK;
}

kvepi_status kvepi_drq_run(const kvepi_drq_params *params, void *workspace,
                           uint64_t workspace_bytes, void *stream) {
  (void)workspace;
  (void)workspace_bytes;  // no workspace (size 0)
  kvepi_drq_plan plan;
  const kvepi_status st = kvepi_drq_validate(params, &plan);
  if (st != KVEPI_OK) return st;
  if (plan.units == 0) return KVEPI_OK;
  const kvepi_status cs = kvepi_drq_debug_check_slots(plan, stream);
  if (cs != KVEPI_OK) return cs;
  return kvepi_drq_launch(plan, stream);
}

}  // extern "C"
