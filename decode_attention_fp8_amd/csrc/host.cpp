// Host-only helpers of libpkv: status strings, version, split planning.
#include <stdint.h>

#include <algorithm>

#include "pkv.h"

extern "C" const char* pkv_strerror(int32_t status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_EINVAL: return "invalid argument";
    case PKV_EUNSUPPORTED: return "unsupported shape";
    case PKV_EHIP: return "HIP launch or runtime error";
    default: return "unknown status";
  }
}

extern "C" int32_t pkv_version(void) { return 100; }  // 0.1.0

// Enough (request, kv head, split) units to give every compute unit several
// single-wave workgroups (256 CUs x 8 resident waves, about 8 units each),
// but splits of 128..512 tokens: shorter ones spend more on partial rows
// (one per query head per split) and on per-unit set-up than they gain in
// balance; longer ones leave the last units of long requests running alone.
extern "C" int32_t pkv_suggest_split(int32_t batch, int32_t max_seq_len, int32_t num_kv_heads,
                                     int32_t page_size) {
  if (batch < 1 || max_seq_len < 1 || num_kv_heads < 1 ||
      (page_size != 16 && page_size != 32 && page_size != 64))
    return PKV_EINVAL;
  constexpr int64_t kTargetUnits = 16384;
  const int64_t work = static_cast<int64_t>(batch) * num_kv_heads * max_seq_len;
  int64_t s = 128;
  while (s < 512 && work / s > kTargetUnits) s *= 2;
  s = std::max<int64_t>(s, page_size);
  const int64_t whole = (static_cast<int64_t>(max_seq_len) + page_size - 1) / page_size * page_size;
  s = std::min<int64_t>(s, whole);
  return static_cast<int32_t>(s);
}
