// kvepi_debug.cpp -- the optional duplicate-slot check of kvepi_run and
// kvepi_drq_run.
//
// Valid slot values must be distinct: the pages leave the rows of repeated
// slots unspecified ("aclnnKvCompressEpilog", 约束说明).  With the environment
// variable KVEPI_CHECK_SLOTS set (to anything but "0"; read at every call),
// the run calls copy the per-token slots to the host, synchronously on the
// caller's stream, and reject the call with KVEPI_ERR_PARAM before any launch
// if two tokens name the same row.  Only the modes with one slot per token
// are checked: the epilog's slot index mode and the operator's page mode (the
// other modes derive rows from batch indices).  It is a debugging aid: it
// synchronises the stream, so it is off by default.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include <algorithm>
#include <vector>

#include "kvepi.h"
#include "kvepi_drq.h"
#include "kvepi_drq_plan.h"
#include "kvepi_plan.h"

namespace {

bool enabled() {
  const char *e = getenv("KVEPI_CHECK_SLOTS");
  return e != nullptr && e[0] != '\0' && !(e[0] == '0' && e[1] == '\0');
}

// KVEPI_ERR_PARAM if two of the n device int32 values in [0, limit) are equal
kvepi_status check_unique(const int32_t *slots, int64_t n, int64_t limit, void *stream) {
  std::vector<int32_t> s(static_cast<size_t>(n));
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(s.data(), slots, s.size() * sizeof(int32_t), hipMemcpyDeviceToHost, st) !=
      hipSuccess)
    return KVEPI_ERR_RUNTIME;
  if (hipStreamSynchronize(st) != hipSuccess) return KVEPI_ERR_RUNTIME;
  std::vector<int32_t> v;
  v.reserve(s.size());
  for (const int32_t x : s)
    if (x >= 0 && x < limit) v.push_back(x);
  std::sort(v.begin(), v.end());
  for (size_t i = 1; i < v.size(); ++i)
    if (v[i] == v[i - 1]) return KVEPI_ERR_PARAM;
  return KVEPI_OK;
}

}  // namespace

kvepi_status kvepi_debug_check_slots(const kvepi_plan &p, const int32_t *slot_mapping,
                                     void *stream) {
  if (!enabled() || p.index_mode != KVEPI_INDEX_SLOT || p.T == 0) return KVEPI_OK;
  return check_unique(slot_mapping, p.T, p.num_slots, stream);
}

kvepi_status kvepi_drq_debug_check_slots(const kvepi_drq_plan &pl, void *stream) {
  const kvepi_drq_params &p = pl.p;
  if (!enabled() || p.cache_mode != KVEPI_DRQ_PAGE || p.num_tokens == 0) return KVEPI_OK;
  return check_unique(p.indices, p.num_tokens, p.k_cache.block_num * p.k_cache.block_size,
                      stream);
}
