// pkv_verify: the integrity check as a separate batch pass.
//
// "Smaller, faster, safer", section "Protecting a shared KV cache": each
// physical page carries a tag that changes on reallocation, the server
// records the pages and tags each request expects, the mapping is checked
// before decode reads the cache, and a request with any mismatch is aborted.
// The pages keep the check out of the attention kernel (fusing it would race
// between thread groups), so it is its own launch whose flags the decode
// reads later in stream order.
//
// One wave per request: lanes stride over the request's block-table entries
// (coalesced 4-byte reads of the table and of the recorded tags, one random
// 4-byte tag read each), then a wave-wide OR.
#include "common.h"

namespace {

__global__ void __launch_bounds__(256) verify_kernel(const uint32_t* __restrict__ page_tags,
                                                     int32_t num_pages, int32_t page_size,
                                                     const int32_t* __restrict__ block_table,
                                                     const uint32_t* __restrict__ expected,
                                                     const int32_t* __restrict__ seq_lens,
                                                     int32_t batch, int32_t max_pages,
                                                     uint8_t* __restrict__ abort_out) {
  const int b = blockIdx.x * (blockDim.x / pkv::kWave) + threadIdx.x / pkv::kWave;
  const int lane = threadIdx.x % pkv::kWave;
  if (b >= batch) return;
  const int32_t L = seq_lens[b];
  const int64_t need = L > 0 ? (static_cast<int64_t>(L) + page_size - 1) / page_size : 0;
  bool bad = need > max_pages;
  const int64_t n = bad ? max_pages : need;
  const int32_t* row = block_table + static_cast<int64_t>(b) * max_pages;
  const uint32_t* exp = expected + static_cast<int64_t>(b) * max_pages;
  for (int64_t j = lane; j < n && !bad; j += pkv::kWave) {
    const int32_t pid = row[j];
    bad = pid < 0 || pid >= num_pages || page_tags[pid] != exp[j];
  }
  const bool any = __any(bad);
  if (lane == 0) abort_out[b] = any ? 1 : 0;
}

}  // namespace

extern "C" int pkv_verify(const pkv_cache* cache, const int32_t* block_table,
                          const uint32_t* expected_tags, const int32_t* seq_lens, int32_t batch,
                          int32_t max_pages, uint8_t* abort_out, hipStream_t stream) {
  if (!cache || !cache->page_tags || cache->num_pages < 1 ||
      !pkv::valid_page_size(cache->page_size))
    return PKV_EINVAL;
  if (!block_table || !expected_tags || !seq_lens || !abort_out || batch < 0 || max_pages < 1)
    return PKV_EINVAL;
  if (batch == 0) return PKV_OK;
  constexpr int kWavesPerBlock = 4;
  const int blocks = static_cast<int>(pkv::cdiv(batch, kWavesPerBlock));
  verify_kernel<<<blocks, kWavesPerBlock * pkv::kWave, 0, stream>>>(
      cache->page_tags, cache->num_pages, cache->page_size, block_table, expected_tags, seq_lens,
      batch, max_pages, abort_out);
  return pkv::launch_status();
}
