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

// Split planning: a longer split writes fewer partial rows (one per query
// head and split, read again by the merge) and repeats the per-unit set-up
// less often; a shorter one gives more units to spread over 256 compute
// units. Measured on MI355X: see the grouped-query branch below; the wide
// latent kernel keeps gaining up to 4096-token splits at batch 64.
extern "C" int32_t pkv_suggest_split(const pkv_cache* cache, int32_t num_q_heads, int32_t batch,
                                     int64_t total_tokens, int32_t max_seq_len) {
  if (!cache || batch < 1 || max_seq_len < 1 || num_q_heads < 1 || cache->num_kv_heads < 1 ||
      num_q_heads % cache->num_kv_heads || total_tokens < 0 ||
      (cache->page_size != 16 && cache->page_size != 32 && cache->page_size != 64))
    return PKV_EINVAL;
  const int64_t P = cache->page_size;
  const int64_t total = total_tokens > 0 ? total_tokens : static_cast<int64_t>(batch) * max_seq_len;
  const int64_t whole = (static_cast<int64_t>(max_seq_len) + P - 1) / P * P;
  // work units of split s: one per (request, split) and head block
  auto units = [&](int64_t s, int64_t blocks) { return blocks * (total / s + batch / 2 + 1); };
  const bool latent = cache->v_pool == nullptr;
  const int G = num_q_heads / cache->num_kv_heads;
  int64_t s;
  if (latent && cache->head_dim_k == 576 && cache->head_dim_v == 512 &&
      cache->num_kv_heads == 1 && P == 64 && num_q_heads % 128 == 0) {
    // wide latent kernel (e4m3 or bf16): every compute unit takes an equal
    // share of the batch's pages, cut at split boundaries, so the split
    // only sets how finely the shares can be cut: about a sixteenth of a
    // share (a power of two of pages, 1 .. 64), which keeps the cuts within
    // a few percent of equal while the partial rows stay few (batch-64
    // latent workload, flushed, three runs each: decode 0.192 ms at 128
    // tokens against 0.201 at 256, an eighth of a share)
    const int64_t share = std::max<int64_t>(1, total / P / (256 / (num_q_heads / 128)));
    int64_t pages = 1;
    while (pages * 2 <= share / 16 && pages < 64) pages *= 2;
    s = pages * P;
  } else if (!latent && cache->head_dim_k == 128 && cache->head_dim_v == 128 && G <= 16) {
    // MFMA grouped-query kernel (e4m3 or bf16): single-wave units; splits of
    // 128 .. 2048 tokens (128 pages at most, the two-launch step's limit),
    // the longest giving 1100 units or more, enough waves to keep HBM busy:
    // long units pay their start and their partials less often. Measured
    // on the concurrency sweep (flushed step, e4m3): batch 16 0.111 ms at
    // 2048 against 0.119 at 512, batch 32 0.215 at 2048 against 0.221 at
    // 1024, batch 8 0.065 at 1024 and 0.063 at 512 against 0.067 at 256,
    // batch 1 best at 128 (0.0192, against 0.0199 at 64 and 0.0202 at 256).
    // Splits of 128 tokens are kept for launches that 256-token ones would
    // leave with fewer than 1024 units (four per CU): at 32 KB a unit's start
    // and its partial row cost more than the extra waves gain (batch 8 x
    // 4096: 0.0253 ms per step at 256, 1064 units, against 0.0279 at 128).
    s = std::min<int64_t>(2048, 128 * P);
    while (s > 128 && units(s, cache->num_kv_heads) < 1100) s /= 2;
    if (s == 128 && 128 * P >= 256 && units(256, cache->num_kv_heads) >= 1024) s = 256;
  } else {
    constexpr int64_t kTargetUnits = 16384;
    const int64_t work = static_cast<int64_t>(batch) * cache->num_kv_heads * max_seq_len;
    s = 128;
    while (s < 512 && work / s > kTargetUnits) s *= 2;
  }
  s = std::max<int64_t>(s, P);
  s = std::min<int64_t>(s, whole);
  return static_cast<int32_t>(s);
}
