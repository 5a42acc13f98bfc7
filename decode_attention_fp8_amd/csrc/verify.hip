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
// One 256-thread workgroup per request. Each thread takes entries
// j = j0 + 256u + tid for u < 8 of every 2048-entry round: first all eight
// block-table entries and recorded tags (coalesced, independent), then all
// eight pool tags (random 4-byte reads, independent), so a round costs two
// memory latencies whatever the request length. The workgroup ORs the
// verdicts and one thread writes the flag; no atomics, no pre-cleared output.
#include "common.h"

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;

__global__ void __launch_bounds__(kThreads) verify_kernel(const uint32_t* __restrict__ page_tags,
                                                          int32_t num_pages, int32_t page_size,
                                                          const int32_t* __restrict__ block_table,
                                                          const uint32_t* __restrict__ expected,
                                                          const int32_t* __restrict__ seq_lens,
                                                          int32_t max_pages,
                                                          uint8_t* __restrict__ abort_out) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int32_t L = seq_lens[b];
  const int64_t need = L > 0 ? (static_cast<int64_t>(L) + page_size - 1) / page_size : 0;
  // a request needing more pages than its row holds cannot be mapped
  int bad = need > max_pages ? 1 : 0;
  const int64_t n = bad ? 0 : need;
  const int32_t* row = block_table + static_cast<int64_t>(b) * max_pages;
  const uint32_t* exp = expected + static_cast<int64_t>(b) * max_pages;
  for (int64_t j0 = 0; j0 < n; j0 += kThreads * kUnroll) {
    int32_t pid[kUnroll];
    uint32_t want[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t j = j0 + u * kThreads + tid;
      pid[u] = 0;
      want[u] = 0;
      if (j < n) {
        pid[u] = row[j];
        want[u] = exp[j];
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t j = j0 + u * kThreads + tid;
      if (j < n) {
        const bool in_pool = pid[u] >= 0 && pid[u] < num_pages;
        const uint32_t have = in_pool ? page_tags[pid[u]] : 0u;
        bad |= (!in_pool || have != want[u]) ? 1 : 0;
      }
    }
  }
  bad = __syncthreads_or(bad);
  if (tid == 0) abort_out[b] = bad ? 1 : 0;
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
  verify_kernel<<<batch, kThreads, 0, stream>>>(cache->page_tags, cache->num_pages,
                                                cache->page_size, block_table, expected_tags,
                                                seq_lens, max_pages, abort_out);
  return pkv::launch_status();
}
