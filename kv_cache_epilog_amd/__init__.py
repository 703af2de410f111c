"""MI355X-native fused KV-cache write epilog (gfx950 HIP kernels behind a C ABI).

See include/kvepi.h for the contract.  This package holds the HIP sources
(csrc/), the in-tree build (build.py) and the ctypes binding (binding.py)."""
from .binding import (KVEPI_MODE_BF16_SPLIT, KVEPI_MODE_FP8_BF16SCALE, KVEPI_MODE_FP8_E8M0,
                      KVEPI_MODE_FP4_NOPE, KVEPI_MODE_FP8_ROW, KVEPI_MODE_HIF8_FP4, KVEPI_MODE_MXFP4,
                      KVEPI_MODE_MXFP8, KVEPI_INDEX_BATCH, KVEPI_INDEX_BATCH_START,
                      KVEPI_INDEX_BLOCK, KVEPI_INDEX_SLOT, KVEPI_X_BF16, KVEPI_X_FP16,
                      KVEPI_DRQ_CONTIGUOUS, KVEPI_DRQ_PAGE, KVEPI_DT_BF16, KVEPI_DT_FP16,
                      KVEPI_DT_FP32, KVEPI_DT_INT32, drq_params, kvepi_drq_get_workspace,
                      kvepi_drq_params, kvepi_drq_run, KvepiError, cache_desc, kvepi_options,
                      kvepi_cache, kvepi_get_workspace, kvepi_row_bytes, kvepi_run,
                      KvepiPrepared, kvepi_prepare, kvepi_prepared, kvepi_run_prepared,
                      kvepi_status_str, kvepi_version, lib)

__all__ = ["KVEPI_MODE_BF16_SPLIT", "KVEPI_MODE_FP8_BF16SCALE", "KVEPI_MODE_FP8_E8M0",
           "KVEPI_MODE_FP4_NOPE", "KVEPI_MODE_FP8_ROW", "KVEPI_MODE_HIF8_FP4", "KVEPI_MODE_MXFP4", "KVEPI_MODE_MXFP8",
           "KVEPI_INDEX_BATCH", "KVEPI_INDEX_BATCH_START", "KVEPI_INDEX_BLOCK", "KVEPI_INDEX_SLOT",
           "KVEPI_X_BF16", "KVEPI_X_FP16", "kvepi_options", "KVEPI_DRQ_CONTIGUOUS",
           "KVEPI_DRQ_PAGE", "KVEPI_DT_BF16", "KVEPI_DT_FP16", "KVEPI_DT_FP32", "KVEPI_DT_INT32",
           "drq_params", "kvepi_drq_get_workspace", "kvepi_drq_params", "kvepi_drq_run",
           "KvepiError", "cache_desc", "kvepi_cache", "kvepi_get_workspace", "kvepi_row_bytes",
           "kvepi_run", "KvepiPrepared", "kvepi_prepare", "kvepi_prepared",
           "kvepi_run_prepared", "kvepi_status_str", "kvepi_version", "lib"]
