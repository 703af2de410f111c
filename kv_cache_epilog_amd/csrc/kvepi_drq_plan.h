// kvepi_drq_plan.h -- internal description of one validated dequant -> RoPE
// -> int8 KV cache call, passed from the host validation
// (kvepi_drq_host.cpp) to the launcher (kvepi_drq.hip).  Not public ABI.
#pragma once

#include <stdint.h>

#include "kvepi_drq.h"

struct kvepi_drq_plan {
  kvepi_drq_params p;       // the caller's parameters (validated)
  int64_t H;                // (nq + 2 nkv) * head_dim
  int64_t units;            // threads: T * H / 16
  int64_t k_pitch, k_bstride, v_pitch, v_bstride;  // bytes
};

kvepi_status kvepi_drq_validate(const kvepi_drq_params *p, kvepi_drq_plan *plan);
kvepi_status kvepi_drq_launch(const kvepi_drq_plan &plan, void *stream);
// The optional duplicate-slot check of page mode (KVEPI_CHECK_SLOTS;
// kvepi_debug.cpp): KVEPI_OK unless it is enabled and two tokens name the
// same row.
kvepi_status kvepi_drq_debug_check_slots(const kvepi_drq_plan &plan, void *stream);
