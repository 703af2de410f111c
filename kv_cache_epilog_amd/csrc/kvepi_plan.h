// kvepi_plan.h -- internal description of one validated epilog call, passed
// from the host validation (kvepi_host.cpp) to the launcher
// (kvepi_kernels.hip).  Not part of the public ABI.
#pragma once

#include <stdint.h>

#include "kvepi.h"

struct kvepi_plan {
  int32_t mode;  // KVEPI_MODE_*
  bool norm;     // gamma given
  bool rope;     // cos/sin given
  bool x_fp16;   // x holds fp16 values (indexer modes)
  int32_t index_mode;  // KVEPI_INDEX_*
  int64_t seq_len;     // tokens per batch (index modes other than SLOT)
  int32_t rope_dim;    // rope segment length (64 except in the bf16 split mode)
  int64_t T, d, nope, x_stride;
  const uint16_t *x, *gamma, *cos, *sin;
  const int32_t *slots;
  // main cache (codes / ckv): byte geometry
  uint8_t *cache;
  int64_t c_pitch, c_bstride;
  int32_t c_align;  // largest power of two <= 16 dividing every row start
  // aux cache (cache_scale / k cache)
  uint8_t *aux;
  int64_t a_pitch, a_bstride;
  int32_t a_align;
  int64_t block_size, num_slots;
  int64_t concat_col, kv_cache_col, scale_col;
  int32_t group_size;  // values per scale group
  float eps;
};

// Host-side validation shared by both stages; fills *plan on success.
kvepi_status kvepi_validate(const void *x, int64_t num_tokens, int64_t d,
                            int64_t x_row_stride, const void *gamma,
                            const void *cos, const void *sin,
                            const int32_t *slot_mapping,
                            const kvepi_cache *cache,
                            const kvepi_cache *cache_aux, int32_t quant_mode,
                            int32_t group_size, float eps, const kvepi_options *options,
                            kvepi_plan *plan);

// Enqueue the kernel for a validated plan (T > 0).
kvepi_status kvepi_launch(const kvepi_plan &plan, void *stream);
// The optional duplicate-slot check (KVEPI_CHECK_SLOTS; kvepi_debug.cpp):
// KVEPI_OK unless it is enabled and two tokens name the same row.
kvepi_status kvepi_debug_check_slots(const kvepi_plan &plan, const int32_t *slot_mapping,
                                     void *stream);
