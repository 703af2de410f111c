// kvepi_debug.cpp -- the optional duplicate-slot check of kvepi_run.
//
// Valid slot values must be distinct: the pages leave the rows of repeated
// slots unspecified ("aclnnKvCompressEpilog", 约束说明).  With the environment
// variable KVEPI_CHECK_SLOTS set (to anything but "0"; read at every call),
// kvepi_run copies slot_mapping to the host, synchronously on the caller's
// stream, and rejects the call with KVEPI_ERR_PARAM before any launch if two
// tokens name the same row.  Only the slot index mode is checked (the other
// index modes derive rows from batch indices, not from one value per token).
// It is a debugging aid: it synchronises the stream, so it is off by default.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include <algorithm>
#include <vector>

#include "kvepi.h"
#include "kvepi_plan.h"

kvepi_status kvepi_debug_check_slots(const kvepi_plan &p, const int32_t *slot_mapping,
                                     void *stream) {
  const char *e = getenv("KVEPI_CHECK_SLOTS");
  if (e == nullptr || e[0] == '\0' || (e[0] == '0' && e[1] == '\0')) return KVEPI_OK;
  if (p.index_mode != KVEPI_INDEX_SLOT || p.T == 0) return KVEPI_OK;
  std::vector<int32_t> s(static_cast<size_t>(p.T));
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(s.data(), slot_mapping, s.size() * sizeof(int32_t), hipMemcpyDeviceToHost,
                     st) != hipSuccess)
    return KVEPI_ERR_RUNTIME;
  if (hipStreamSynchronize(st) != hipSuccess) return KVEPI_ERR_RUNTIME;
  std::vector<int32_t> v;
  v.reserve(s.size());
  for (const int32_t x : s)
    if (x >= 0 && x < p.num_slots) v.push_back(x);
  std::sort(v.begin(), v.end());
  for (size_t i = 1; i < v.size(); ++i)
    if (v[i] == v[i - 1]) return KVEPI_ERR_PARAM;
  return KVEPI_OK;
}
