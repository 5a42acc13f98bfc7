// pkv_append: quantise-on-append of new K/V rows into cache pages.
//
// "Smaller, faster, safer", section "Quantizing the KV cache": the cache is
// held as e4m3 instead of BF16. Each value x of kv head h becomes
// RNE_SAT(fl32(x / scale[h])): a correctly rounded float32 division, then
// round-to-nearest-even onto the OCP E4M3 grid, saturating at +-448.
//
// One thread owns 16 consecutive values of one (token, kv head) row: it
// reads 32 bytes of bf16 and writes one 16-byte chunk of codes (32 bytes for
// a bf16 cache), so a wave writes whole rows with 16-byte stores.
//
// With scales set at append (one per row), a row's threads are consecutive
// lanes of one wave (dim / 16 of them, a power of two): they share the row's
// largest magnitude by shuffles, and the row's first thread stores its scale
// fl32(amax / 448) (1 for an all-zero row).
#include "common.h"

namespace {

struct AppendArgs {
  const uint16_t* src;  // bf16 [n][heads][dim]
  uint8_t* pool;        // [pages][heads][P][dim] elements of elem_bytes
  const float* scale;   // [heads] (e4m3 only)
  float* row_scale;     // [pages][heads][P]: scales set at append, or NULL
  int dim;              // elements per row
  int pool_dim;         // row length in the pool (>= dim; latent rows)
};

template <bool kE4M3, bool kRows>
__global__ void __launch_bounds__(256) append_kernel(AppendArgs a, const int32_t* __restrict__ slot,
                                                     const int32_t* __restrict__ token_req,
                                                     const uint8_t* __restrict__ abort_flags,
                                                     int64_t n_tokens, int heads, int page_size,
                                                     int64_t n_slots) {
  const int chunks = a.dim / 16;
  const int64_t per_token = static_cast<int64_t>(heads) * chunks;
  const int64_t total = n_tokens * per_token;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t tok = i / per_token;
    const int rem = static_cast<int>(i - tok * per_token);
    const int h = rem / chunks;
    const int c = rem - h * chunks;
    const int32_t s = slot[tok];
    if (s < 0 || s >= n_slots) continue;
    if (token_req && abort_flags && abort_flags[token_req[tok]]) continue;
    const int64_t page = s / page_size;
    const int row = s - static_cast<int>(page) * page_size;
    const uint16_t* src = a.src + (tok * heads + h) * a.dim + c * 16;
    const uint4 w0 = *reinterpret_cast<const uint4*>(src);
    const uint4 w1 = *reinterpret_cast<const uint4*>(src + 8);
    const int64_t dst_elem = ((page * heads + h) * page_size + row) * a.pool_dim + c * 16;
    if constexpr (kE4M3) {
      float scale;
      if constexpr (kRows) {
        // the row's lanes are aligned groups of `chunks` lanes, all active
        // or all skipped together
        float m = pkv::abs_max16(w0, w1);
        for (int off = 1; off < chunks; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));
        scale = m == 0.0f ? 1.0f : __fdiv_rn(m, 448.0f);
        if (c == 0) a.row_scale[(page * heads + h) * page_size + row] = scale;
      } else {
        scale = a.scale[h];
      }
      *reinterpret_cast<uint4*>(a.pool + dst_elem) = pkv::encode16(w0, w1, scale);
    } else {
      uint4* dst = reinterpret_cast<uint4*>(a.pool + dst_elem * 2);
      dst[0] = w0;
      dst[1] = w1;
    }
  }
}

template <bool kE4M3, bool kRows = false>
int launch(const AppendArgs& a, const int32_t* slot, const int32_t* token_req,
           const uint8_t* abort_flags, int64_t n, int heads, int page_size, int64_t n_slots,
           hipStream_t stream) {
  const int64_t total = n * heads * (a.dim / 16);
  if (total == 0) return PKV_OK;
  const int blocks = static_cast<int>(std::min<int64_t>(pkv::cdiv(total, 256), 65536));
  append_kernel<kE4M3, kRows><<<blocks, 256, 0, stream>>>(a, slot, token_req, abort_flags, n,
                                                          heads, page_size, n_slots);
  return pkv::launch_status();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" int pkv_append(const pkv_cache* cache, const void* k_new, const void* v_new,
                          const int32_t* slot, const int32_t* token_req,
                          const uint8_t* abort_flags, int64_t n_tokens, hipStream_t stream) {
  int st = pkv::check_cache(cache);
  if (st) return st;
  const bool latent = cache->v_pool == nullptr;
  if (!k_new || !slot || n_tokens < 0 || (latent && v_new) || (!latent && !v_new))
    return PKV_EINVAL;
  if (!aligned16(k_new) || (v_new && !aligned16(v_new)) || !aligned16(cache->k_pool) ||
      (cache->v_pool && !aligned16(cache->v_pool)))
    return PKV_EINVAL;
  const bool e4m3 = cache->dtype == PKV_KV_E4M3;
  const int64_t n_slots = static_cast<int64_t>(cache->num_pages) * cache->page_size;
  if (cache->k_row_scale) {
    if (!pkv::row_lanes_ok(cache->head_dim_k) || !pkv::row_lanes_ok(cache->head_dim_v))
      return PKV_EUNSUPPORTED;
    AppendArgs k{static_cast<const uint16_t*>(k_new), static_cast<uint8_t*>(cache->k_pool),
                 nullptr, cache->k_row_scale, cache->head_dim_k, cache->head_dim_k};
    st = launch<true, true>(k, slot, token_req, abort_flags, n_tokens, cache->num_kv_heads,
                            cache->page_size, n_slots, stream);
    if (st) return st;
    AppendArgs v{static_cast<const uint16_t*>(v_new), static_cast<uint8_t*>(cache->v_pool),
                 nullptr, cache->v_row_scale, cache->head_dim_v, cache->head_dim_v};
    return launch<true, true>(v, slot, token_req, abort_flags, n_tokens, cache->num_kv_heads,
                              cache->page_size, n_slots, stream);
  }
  AppendArgs k{static_cast<const uint16_t*>(k_new), static_cast<uint8_t*>(cache->k_pool),
               cache->k_scale, nullptr, cache->head_dim_k, cache->head_dim_k};
  st = e4m3 ? launch<true>(k, slot, token_req, abort_flags, n_tokens, cache->num_kv_heads,
                           cache->page_size, n_slots, stream)
            : launch<false>(k, slot, token_req, abort_flags, n_tokens, cache->num_kv_heads,
                            cache->page_size, n_slots, stream);
  if (st || latent) return st;
  AppendArgs v{static_cast<const uint16_t*>(v_new), static_cast<uint8_t*>(cache->v_pool),
               cache->v_scale, nullptr, cache->head_dim_v, cache->head_dim_v};
  return e4m3 ? launch<true>(v, slot, token_req, abort_flags, n_tokens, cache->num_kv_heads,
                             cache->page_size, n_slots, stream)
              : launch<false>(v, slot, token_req, abort_flags, n_tokens, cache->num_kv_heads,
                              cache->page_size, n_slots, stream);
}
