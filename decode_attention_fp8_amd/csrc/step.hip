// pkv_step_decode, pkv_step_combine: one decode step (the tag check, the
// append of each request's new token at its last position, split-KV decode
// and the merge) in two launches instead of three.
//
// "Smaller, faster, safer", section "Protecting a shared KV cache": the
// mapping of a request is checked before anything it reads is returned, and
// an aborted request writes nothing to the cache. Section "Quantizing the KV
// cache": the new token's K and V are stored as e4m3 under the kv head's
// scale, and the attention kernel converts codes as it reads them.
//
// The two-launch form moves the check into the decode launch (each split's
// units check that split's pages; the splits cover the request) and the
// append into the combine launch (once every split's verdict is in). The
// decode reads the new token's row from its values, encoded exactly as the
// append encodes them, so the result is the one of
//   pkv_verify_append (slot = the row of position seq_lens[b] - 1)
//   -> pkv_decode_attn (abort flags) -> pkv_combine (abort flags)
// bit for bit. Shapes without the two-launch form run those three launches.
#include "common.h"
#include "decode_params.h"
#include "step.h"

bool step_two_launch(const pkv_cache* cache, int32_t num_q_heads, int32_t split_tokens) {
  if (!cache || !cache->v_pool || cache->k_row_scale || cache->num_kv_heads < 1) return false;
  if (cache->head_dim_k != 128 || cache->head_dim_v != 128) return false;
  if (num_q_heads < 1 || num_q_heads % cache->num_kv_heads) return false;
  const int G = num_q_heads / cache->num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return false;
  return split_tokens >= cache->page_size && split_tokens <= 128 * cache->page_size &&
         gqa_mfma_path_supported(128, 128, G, false, split_tokens, cache->page_size);
}

namespace {

bool misaligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

int check_step_inputs(const pkv_cache* cache, const void* k_new, const void* v_new,
                      const uint32_t* expected_tags, const uint8_t* unit_flags,
                      const uint8_t* abort_out) {
  const int st = pkv::check_cache(cache);
  if (st) return st;
  const bool latent = cache->v_pool == nullptr;
  if ((expected_tags && !cache->page_tags) || !unit_flags || !abort_out || !k_new ||
      (latent && v_new) || (!latent && !v_new))
    return PKV_EINVAL;
  if (misaligned16(k_new) || (v_new && misaligned16(v_new))) return PKV_EINVAL;
  return PKV_OK;
}

}  // namespace

extern "C" int pkv_step_decode(const pkv_cache* cache, const void* q, int32_t num_q_heads,
                               const void* k_new, const void* v_new, const int32_t* block_table,
                               const uint32_t* expected_tags, const int32_t* seq_lens,
                               int32_t batch, int32_t max_pages, int32_t max_seq_len,
                               float sm_scale, int32_t split_tokens, int32_t max_splits,
                               float* o_part, float* lse_part, uint8_t* unit_flags,
                               uint8_t* abort_out, hipStream_t stream) {
  int st = check_step_inputs(cache, k_new, v_new, expected_tags, unit_flags, abort_out);
  if (st) return st;
  const bool two = step_two_launch(cache, num_q_heads, split_tokens);
  const StepDecodeInputs in{expected_tags, unit_flags, static_cast<const uint16_t*>(k_new),
                            static_cast<const uint16_t*>(v_new)};
  // every argument is checked before anything is launched
  st = decode_attn_impl(cache, q, num_q_heads, block_table, seq_lens, batch, max_pages,
                        max_seq_len, two ? nullptr : abort_out, sm_scale, split_tokens,
                        max_splits, o_part, lse_part, two ? &in : nullptr, stream, true);
  if (st) return st;
  if (two)
    return decode_attn_impl(cache, q, num_q_heads, block_table, seq_lens, batch, max_pages,
                            max_seq_len, nullptr, sm_scale, split_tokens, max_splits, o_part,
                            lse_part, &in, stream, false);
  st = verify_append_impl(cache, block_table, expected_tags, seq_lens, batch, max_pages,
                          abort_out, k_new, v_new, nullptr, stream);
  if (st) return st;
  return decode_attn_impl(cache, q, num_q_heads, block_table, seq_lens, batch, max_pages,
                          max_seq_len, abort_out, sm_scale, split_tokens, max_splits, o_part,
                          lse_part, nullptr, stream, false);
}

extern "C" int pkv_step_combine(const pkv_cache* cache, int32_t num_q_heads, const void* k_new,
                                const void* v_new, const int32_t* block_table,
                                const uint32_t* expected_tags, const int32_t* seq_lens,
                                int32_t batch, int32_t max_pages, int32_t max_seq_len,
                                int32_t split_tokens, int32_t max_splits, const float* o_part,
                                const float* lse_part, const uint8_t* unit_flags,
                                uint8_t* abort_out, void* out, float* lse_out,
                                hipStream_t stream) {
  const int st = check_step_inputs(cache, k_new, v_new, expected_tags, unit_flags, abort_out);
  if (st) return st;
  if (!block_table || max_pages < 1) return PKV_EINVAL;
  if (!step_two_launch(cache, num_q_heads, split_tokens))
    return combine_impl(o_part, lse_part, seq_lens, batch, num_q_heads, cache->head_dim_v,
                        split_tokens, max_splits, max_seq_len, abort_out, out, lse_out, nullptr,
                        stream);
  StepCombineArgs sa{};
  sa.unit_flags = unit_flags;
  sa.abort_out = abort_out;
  sa.block_table = block_table;
  sa.expected_tags = expected_tags;
  sa.page_tags = cache->page_tags;
  sa.num_pages = cache->num_pages;
  sa.page_size = cache->page_size;
  sa.max_pages = max_pages;
  sa.group = num_q_heads / cache->num_kv_heads;
  sa.kv_heads = cache->num_kv_heads;
  sa.head_dim = cache->head_dim_k;
  sa.k_pool = static_cast<uint8_t*>(cache->k_pool);
  sa.v_pool = static_cast<uint8_t*>(cache->v_pool);
  sa.k_scale = cache->k_scale;
  sa.v_scale = cache->v_scale;
  sa.k_new = static_cast<const uint16_t*>(k_new);
  sa.v_new = static_cast<const uint16_t*>(v_new);
  sa.e4m3 = cache->dtype == PKV_KV_E4M3;
  return combine_impl(o_part, lse_part, seq_lens, batch, num_q_heads, cache->head_dim_v,
                      split_tokens, max_splits, max_seq_len, nullptr, out, lse_out, &sa, stream);
}

extern "C" int pkv_step_launches(const pkv_cache* cache, int32_t num_q_heads,
                                 int32_t split_tokens) {
  // the geometry only (pools and scales are not read)
  if (!cache || cache->num_kv_heads < 1 || !pkv::valid_page_size(cache->page_size))
    return PKV_EINVAL;
  return step_two_launch(cache, num_q_heads, split_tokens) ? 2 : 3;
}
