// pkv_requantize_pages: prefill -> decode handoff of whole cache pages.
//
// "Smaller, faster, safer", section "Quantizing the KV cache": decode holds
// its KV cache as e4m3 while the prefill side keeps BF16, so the pages a
// prefill produced are re-encoded on their way into a decode pool. Section
// "Protecting a shared KV cache": a page's tag changes whenever it is
// (re)allocated; the handoff writes the destination pages' new tags.
//
// Each value is encoded exactly as pkv_append encodes a new value:
// RNE_SAT(fl32(x / scale[h])) with the destination pool's static scale.
//
// One workgroup per (page pair, K|V): a page of one pool is a contiguous run
// of heads x P rows; its 256 threads walk it in 16-value chunks (32 bytes of
// bf16 in, one 16-byte chunk of codes out), so the page streams with 16-byte
// loads and stores. HBM-bound: 3 bytes moved per value.
#include "common.h"

namespace {

struct RequantArgs {
  const uint16_t* src;  // bf16 pool [pages][heads][P][row]
  uint8_t* dst;         // e4m3 pool [pages][heads][P][row]
  const float* scale;   // [heads]
  int row;              // values per row (head dim, or the latent row width)
};

__global__ void __launch_bounds__(256) requant_kernel(RequantArgs k, RequantArgs v,
                                                      const int32_t* __restrict__ src_pages,
                                                      const int32_t* __restrict__ dst_pages,
                                                      const uint32_t* __restrict__ new_tags,
                                                      uint32_t* __restrict__ dst_tags,
                                                      int n_src, int n_dst, int heads,
                                                      int page_size) {
  const int i = blockIdx.x;
  const RequantArgs a = blockIdx.y == 0 ? k : v;
  const int32_t sp = src_pages[i], dp = dst_pages[i];
  if (sp < 0 || sp >= n_src || dp < 0 || dp >= n_dst) return;
  const int per_head = page_size * a.row / 16;  // chunks of one (page, head) block
  const int total = heads * per_head;
  const int64_t page_vals = static_cast<int64_t>(heads) * page_size * a.row;
  const uint4* src = reinterpret_cast<const uint4*>(a.src + sp * page_vals);
  uint4* dst = reinterpret_cast<uint4*>(a.dst + dp * page_vals);
  // both pages are touched once: non-temporal loads and stores keep them out
  // of the caches' reuse
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4* src4 = reinterpret_cast<const u32x4*>(src);
  u32x4* dst4 = reinterpret_cast<u32x4*>(dst);
  for (int c = threadIdx.x; c < total; c += blockDim.x) {
    const int h = c / per_head;
    const u32x4 w0 = __builtin_nontemporal_load(src4 + 2 * c);
    const u32x4 w1 = __builtin_nontemporal_load(src4 + 2 * c + 1);
    const uint4 e = pkv::encode16(make_uint4(w0.x, w0.y, w0.z, w0.w),
                                  make_uint4(w1.x, w1.y, w1.z, w1.w), a.scale[h]);
    __builtin_nontemporal_store(u32x4{e.x, e.y, e.z, e.w}, dst4 + c);
  }
  if (blockIdx.y == 0 && threadIdx.x == 0 && new_tags) dst_tags[dp] = new_tags[i];
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" int pkv_requantize_pages(const pkv_cache* src, const pkv_cache* dst,
                                    const int32_t* src_pages, const int32_t* dst_pages,
                                    const uint32_t* new_tags, uint32_t* dst_tags,
                                    int32_t n_pages, hipStream_t stream) {
  int st = pkv::check_cache(src);
  if (st) return st;
  st = pkv::check_cache(dst);
  if (st) return st;
  if (src->dtype != PKV_KV_BF16 || dst->dtype != PKV_KV_E4M3) return PKV_EINVAL;
  if (dst->k_row_scale) return PKV_EUNSUPPORTED;  // pages of static-scale pools only
  if (src->page_size != dst->page_size || src->num_kv_heads != dst->num_kv_heads ||
      src->head_dim_k != dst->head_dim_k || src->head_dim_v != dst->head_dim_v ||
      (src->v_pool == nullptr) != (dst->v_pool == nullptr))
    return PKV_EINVAL;
  if (!src_pages || !dst_pages || n_pages < 0 || (new_tags == nullptr) != (dst_tags == nullptr))
    return PKV_EINVAL;
  if (!aligned16(src->k_pool) || !aligned16(dst->k_pool) ||
      (src->v_pool && (!aligned16(src->v_pool) || !aligned16(dst->v_pool))))
    return PKV_EINVAL;
  if (n_pages == 0) return PKV_OK;
  const bool latent = src->v_pool == nullptr;
  RequantArgs k{static_cast<const uint16_t*>(src->k_pool), static_cast<uint8_t*>(dst->k_pool),
                dst->k_scale, src->head_dim_k};
  RequantArgs v = k;
  if (!latent)
    v = RequantArgs{static_cast<const uint16_t*>(src->v_pool), static_cast<uint8_t*>(dst->v_pool),
                    dst->v_scale, src->head_dim_v};
  dim3 grid(static_cast<uint32_t>(n_pages), latent ? 1 : 2);
  requant_kernel<<<grid, 256, 0, stream>>>(k, v, src_pages, dst_pages, new_tags, dst_tags,
                                           src->num_pages, dst->num_pages, src->num_kv_heads,
                                           src->page_size);
  return pkv::launch_status();
}
