// pkv_decode_attn_static: pkv_decode_attn followed by pkv_combine, with the
// split partials in a fixed device array of the library, for callers that
// cannot allocate (code under graph capture, serving loops that forbid
// hipMalloc).
//
// The array is a file-scope __device__ variable: every GPU the library runs
// on holds one copy of it, at its own address, until the process ends. Its
// address is looked up once per device (hipGetSymbolAddress, with that
// device current) and only that address is handed to kernels; in host code
// the variable's own name is not a device address. Every call on one GPU
// shares its copy: calls that overlap in time on one GPU race.
#include <mutex>

#include "common.h"

namespace {

constexpr int64_t kScratchBytes = PKV_STATIC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// This device's copy of the array (looked up on its first use).
int scratch_for_current_device(uint8_t** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return PKV_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return PKV_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PKV_EHIP;
    g_scratch[dev] = p;
  }
  *out = static_cast<uint8_t*>(g_scratch[dev]);
  return PKV_OK;
}

}  // namespace

extern "C" int pkv_decode_attn_static(const pkv_cache* cache, const void* q, int32_t num_q_heads,
                                      const int32_t* block_table, const int32_t* seq_lens,
                                      int32_t batch, int32_t max_pages, int32_t max_seq_len,
                                      const uint8_t* abort_flags, float sm_scale,
                                      int32_t split_tokens, void* out, float* lse_out,
                                      hipStream_t stream) {
  int st = pkv::check_cache(cache);
  if (st) return st;
  if (!q || !block_table || !seq_lens || !out) return PKV_EINVAL;
  if (batch < 0 || max_pages < 1 || max_seq_len < 0 || num_q_heads < 1) return PKV_EINVAL;
  if (split_tokens < cache->page_size || split_tokens % cache->page_size) return PKV_EINVAL;
  const int64_t n_splits = std::max<int64_t>(1, pkv::cdiv(max_seq_len, split_tokens));
  const int64_t rows = static_cast<int64_t>(batch) * num_q_heads * n_splits;
  const int64_t o_bytes = (rows * cache->head_dim_v * 4 + 255) / 256 * 256;
  if (o_bytes + rows * 4 > kScratchBytes) return PKV_EINVAL;
  if (batch == 0) return PKV_OK;
  uint8_t* base = nullptr;
  st = scratch_for_current_device(&base);
  if (st) return st;
  float* o_part = reinterpret_cast<float*>(base);
  float* lse_part = reinterpret_cast<float*>(base + o_bytes);
  st = pkv_decode_attn(cache, q, num_q_heads, block_table, seq_lens, batch, max_pages,
                       max_seq_len, abort_flags, sm_scale, split_tokens,
                       static_cast<int32_t>(n_splits), o_part, lse_part, stream);
  if (st) return st;
  return pkv_combine(o_part, lse_part, seq_lens, batch, num_q_heads, cache->head_dim_v,
                     split_tokens, static_cast<int32_t>(n_splits), max_seq_len, abort_flags, out,
                     lse_out, stream);
}
