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

// A launch worked out from a validated plan on the current device: the
// kernel instance, its grid and LDS bytes, and the kernel's argument block
// as plain bytes (so that host-only files need no device types).  It holds
// no pointer into itself and may be copied bytewise.
#define KVEPI_KARGS_BYTES 256
struct kvepi_launch_cfg {
  const void *fn;
  uint32_t blocks;
  uint32_t lds;
  int32_t device;  // the HIP device current when the launch was worked out
  int32_t reserved;
  alignas(8) unsigned char args[KVEPI_KARGS_BYTES];
};

// Works out the launch of a validated plan (T > 0) on the current device.
kvepi_status kvepi_configure(const kvepi_plan &plan, kvepi_launch_cfg *cfg);
// Enqueues a launch worked out by kvepi_configure.
kvepi_status kvepi_enqueue(const kvepi_launch_cfg &cfg, void *stream);
// Both of the above: enqueue the kernel for a validated plan (T > 0).
kvepi_status kvepi_launch(const kvepi_plan &plan, void *stream);
// The current HIP device (KVEPI_ERR_RUNTIME if it cannot be read).
kvepi_status kvepi_current_device(int32_t *device);
// The optional duplicate-slot check (KVEPI_CHECK_SLOTS; kvepi_debug.cpp):
// KVEPI_OK unless it is enabled and two tokens name the same row.
kvepi_status kvepi_debug_check_slots(const kvepi_plan &plan, const int32_t *slot_mapping,
                                     void *stream);
