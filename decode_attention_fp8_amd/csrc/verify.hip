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
#include "step.h"

namespace {

constexpr int kThreads = 256;

__global__ void __launch_bounds__(kThreads) verify_kernel(const uint32_t* __restrict__ page_tags,
                                                          int32_t num_pages, int32_t page_size,
                                                          const int32_t* __restrict__ block_table,
                                                          const uint32_t* __restrict__ expected,
                                                          const int32_t* __restrict__ seq_lens,
                                                          int32_t max_pages,
                                                          uint8_t* __restrict__ abort_out) {
  const int b = blockIdx.x;
  const int bad = pkv::check_request(page_tags, num_pages, page_size, block_table, expected,
                                     seq_lens, max_pages, b);
  if (threadIdx.x == 0) abort_out[b] = bad ? 1 : 0;
}

// The rows of one new token for one pool (K or V): heads x dim / 16 chunks of
// 16 values, chunk i taken by thread i (i < 256 per round). With scales set
// at append, a row's dim / 16 threads are consecutive lanes of one wave (a
// power of two, aligned) and share the row's largest magnitude by shuffles.
// The 16 values (32 bytes) of chunk i of a new token's rows.
struct Chunk {
  uint4 w0, w1;
};

__device__ __forceinline__ Chunk load_chunk(const uint16_t* __restrict__ src, int dim, int chunks,
                                            int i) {
  const int h = i / chunks;
  const int c = i - h * chunks;
  return Chunk{*reinterpret_cast<const uint4*>(src + h * dim + c * 16),
               *reinterpret_cast<const uint4*>(src + h * dim + c * 16 + 8)};
}

template <bool kE4M3, bool kRows>
__device__ __forceinline__ void store_chunk(const Chunk& v, int i, uint8_t* pool, const float* scale,
                                            float* row_scale, int heads, int chunks, int pool_dim,
                                            int page_size, int64_t page, int row) {
  {
    const int h = i / chunks;
    const int c = i - h * chunks;
    const uint4 w0 = v.w0, w1 = v.w1;
    const int64_t dst = ((page * heads + h) * page_size + row) * pool_dim + c * 16;
    if constexpr (kE4M3) {
      float s;
      if constexpr (kRows) {
        float m = pkv::abs_max16(w0, w1);
        for (int off = 1; off < chunks; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));
        s = m == 0.0f ? 1.0f : __fdiv_rn(m, 448.0f);
        if (c == 0) row_scale[(page * heads + h) * page_size + row] = s;
      } else {
        s = scale[h];
      }
      *reinterpret_cast<uint4*>(pool + dst) = pkv::encode16(w0, w1, s);
    } else {
      uint4* d = reinterpret_cast<uint4*>(pool + dst * 2);
      d[0] = w0;
      d[1] = w1;
    }
  }
}

template <bool kE4M3, bool kRows>
__device__ __forceinline__ void append_token(const uint16_t* __restrict__ src, uint8_t* pool,
                                             const float* scale, float* row_scale, int heads,
                                             int dim, int pool_dim, int page_size, int64_t page,
                                             int row) {
  const int chunks = dim / 16;
  const int total = heads * chunks;
  for (int i = threadIdx.x; i < total; i += kThreads)
    store_chunk<kE4M3, kRows>(load_chunk(src, dim, chunks, i), i, pool, scale, row_scale, heads,
                              chunks, pool_dim, page_size, page, row);
}

struct Pool {
  uint8_t* pool;
  const float* scale;
  float* row_scale;
  int dim, pool_dim;
};

// pkv_verify_append: workgroup b checks request b, writes its flag and, if
// the request stands, appends its new token (K then V rows) at slot[b]; with
// slot NULL, at the row of the request's last token (position
// seq_lens[b] - 1 of its block table), which a standing request has in the
// pool.
template <bool kE4M3, bool kRows>
__global__ void __launch_bounds__(kThreads) verify_append_kernel(
    const uint32_t* __restrict__ page_tags, int32_t num_pages, int32_t page_size,
    const int32_t* __restrict__ block_table, const uint32_t* __restrict__ expected,
    const int32_t* __restrict__ seq_lens, int32_t max_pages, uint8_t* __restrict__ abort_out,
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const int32_t* __restrict__ slot, Pool kp, Pool vp, int heads, int64_t n_slots) {
  const int b = blockIdx.x;
  const int i = threadIdx.x;
  // the slot and, when each pool's chunks fit one pass, the new token's
  // values are loaded before the check, so their latency passes with it
  // (they are stored only if the request stands)
  int64_t s = slot ? slot[b] : -1;
  const uint16_t* ksrc = k_new + static_cast<int64_t>(b) * heads * kp.dim;
  const uint16_t* vsrc = v_new ? v_new + static_cast<int64_t>(b) * heads * vp.dim : nullptr;
  const int kch = kp.dim / 16, vch = vp.dim / 16;
  const int ktot = heads * kch, vtot = vsrc ? heads * vch : 0;
  const bool one_pass = ktot <= kThreads && vtot <= kThreads;
  Chunk kv{}, vv{};
  if (one_pass && i < ktot) kv = load_chunk(ksrc, kp.dim, kch, i);
  if (one_pass && i < vtot) vv = load_chunk(vsrc, vp.dim, vch, i);
  // no recorded tags (the step without the check): every request stands
  const int bad = expected ? pkv::check_request(page_tags, num_pages, page_size, block_table,
                                                expected, seq_lens, max_pages, b)
                           : 0;
  if (threadIdx.x == 0) abort_out[b] = bad ? 1 : 0;
  if (bad) return;
  if (!slot) {
    const int32_t L = seq_lens[b];
    // no position (or one past the block-table row): nothing to append
    if (L < 1 || (L - 1) / page_size >= max_pages) return;
    const int32_t pid = block_table[static_cast<int64_t>(b) * max_pages + (L - 1) / page_size];
    s = static_cast<int64_t>(pid) * page_size + (L - 1) % page_size;
  }
  if (s < 0 || s >= n_slots) return;
  const int64_t page = s / page_size;
  const int row = s - static_cast<int>(page) * page_size;
  if (one_pass) {
    if (i < ktot)
      store_chunk<kE4M3, kRows>(kv, i, kp.pool, kp.scale, kp.row_scale, heads, kch, kp.pool_dim,
                                page_size, page, row);
    if (i < vtot)
      store_chunk<kE4M3, kRows>(vv, i, vp.pool, vp.scale, vp.row_scale, heads, vch, vp.pool_dim,
                                page_size, page, row);
    return;
  }
  append_token<kE4M3, kRows>(ksrc, kp.pool, kp.scale, kp.row_scale, heads, kp.dim, kp.pool_dim,
                             page_size, page, row);
  if (vsrc)
    append_token<kE4M3, kRows>(vsrc, vp.pool, vp.scale, vp.row_scale, heads, vp.dim, vp.pool_dim,
                               page_size, page, row);
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

int verify_append_impl(const pkv_cache* cache, const int32_t* block_table,
                       const uint32_t* expected_tags, const int32_t* seq_lens, int32_t batch,
                       int32_t max_pages, uint8_t* abort_out, const void* k_new,
                       const void* v_new, const int32_t* slot, hipStream_t stream) {
  int st = pkv::check_cache(cache);
  if (st) return st;
  if (expected_tags && !cache->page_tags) return PKV_EINVAL;
  if (!block_table || !seq_lens || !abort_out || batch < 0 || max_pages < 1) return PKV_EINVAL;
  const bool latent = cache->v_pool == nullptr;
  if (!k_new || (latent && v_new) || (!latent && !v_new)) return PKV_EINVAL;
  auto misaligned = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; };
  if (misaligned(k_new) || (v_new && misaligned(v_new)) || misaligned(cache->k_pool) ||
      (cache->v_pool && misaligned(cache->v_pool)))
    return PKV_EINVAL;
  const bool rows = cache->k_row_scale != nullptr;
  if (rows && (!pkv::row_lanes_ok(cache->head_dim_k) || !pkv::row_lanes_ok(cache->head_dim_v)))
    return PKV_EUNSUPPORTED;
  if (batch == 0) return PKV_OK;
  const int64_t n_slots = static_cast<int64_t>(cache->num_pages) * cache->page_size;
  const Pool kp{static_cast<uint8_t*>(cache->k_pool), cache->k_scale, cache->k_row_scale,
                cache->head_dim_k, cache->head_dim_k};
  const Pool vp{static_cast<uint8_t*>(cache->v_pool), cache->v_scale, cache->v_row_scale,
                cache->head_dim_v, cache->head_dim_v};
  const auto* kn = static_cast<const uint16_t*>(k_new);
  const auto* vn = static_cast<const uint16_t*>(v_new);
  const auto* tags = cache->page_tags;
  if (cache->dtype == PKV_KV_BF16) {
    verify_append_kernel<false, false><<<batch, kThreads, 0, stream>>>(
        tags, cache->num_pages, cache->page_size, block_table, expected_tags, seq_lens, max_pages,
        abort_out, kn, vn, slot, kp, vp, cache->num_kv_heads, n_slots);
  } else if (rows) {
    verify_append_kernel<true, true><<<batch, kThreads, 0, stream>>>(
        tags, cache->num_pages, cache->page_size, block_table, expected_tags, seq_lens, max_pages,
        abort_out, kn, vn, slot, kp, vp, cache->num_kv_heads, n_slots);
  } else {
    verify_append_kernel<true, false><<<batch, kThreads, 0, stream>>>(
        tags, cache->num_pages, cache->page_size, block_table, expected_tags, seq_lens, max_pages,
        abort_out, kn, vn, slot, kp, vp, cache->num_kv_heads, n_slots);
  }
  return pkv::launch_status();
}

extern "C" int pkv_verify_append(const pkv_cache* cache, const int32_t* block_table,
                                 const uint32_t* expected_tags, const int32_t* seq_lens,
                                 int32_t batch, int32_t max_pages, uint8_t* abort_out,
                                 const void* k_new, const void* v_new, const int32_t* slot,
                                 hipStream_t stream) {
  if (!slot || !expected_tags) return PKV_EINVAL;
  return verify_append_impl(cache, block_table, expected_tags, seq_lens, batch, max_pages,
                            abort_out, k_new, v_new, slot, stream);
}
