// Launch parameters shared by the decode kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

struct DecodeParams {
  const void* k_pool;
  const void* v_pool;  // == k_pool for the latent layout
  const float* k_scale;
  const float* v_scale;
  const float* k_row_scale;  // [pages][kv heads][P] scales set at append, or NULL
  const float* v_row_scale;
  const uint16_t* q;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const uint8_t* abort_flags;
  float* o_part;
  float* lse_part;
  int num_pages, page_size, num_kv_heads, num_q_heads, max_pages, max_seq_len;
  int split_tokens, max_splits, head_groups;
  int batch;
  int q_len;            // query positions per request (drafts verified together)
  int v_row;            // elements per V row in v_pool
  float sm_scale_log2;  // sm_scale * log2(e)
  // a step in two launches (grouped-query MFMA kernel only): the units of
  // kv head 0 check their split's pages against the recorded tags and write
  // unit_flags[b][c]; each request's last unit takes the new token (row L - 1)
  // from k_new / v_new instead of the pool. NULL otherwise.
  const uint32_t* page_tags;
  const uint32_t* expected_tags;
  uint8_t* unit_flags;
  const uint16_t* k_new;
  const uint16_t* v_new;
};

// grouped-query kernel on MFMA for an e4m3 or bf16 cache, head dim 128, up
// to 16 query heads per kv head
bool gqa_mfma_path_supported(int dk, int dv, int group, bool latent, int split_tokens,
                             int page_size);
int launch_decode_gqa_mfma(const DecodeParams& p, bool e4m3, int n_split_blocks, int batch,
                           hipStream_t stream);
// the same kernel with the tag check and the new token folded in (p.unit_flags set)
int launch_decode_gqa_mfma_step(const DecodeParams& p, bool e4m3, int n_split_blocks, int batch,
                                hipStream_t stream);

// several query positions per request (a token and its drafts), e4m3, head dim 128
bool drafts_path_supported(int dk, int dv, bool latent, bool e4m3);
int launch_decode_drafts(const DecodeParams& p, int n_split_blocks, int batch, int row_groups,
                         hipStream_t stream);

// wide-head kernel for one latent kv head (576 / 512), page size 64
bool mla_fast_path_supported(int dk, int dv, int num_kv_heads, int num_q_heads, int page_size,
                             int split_tokens);
int launch_decode_mla(const DecodeParams& p, bool e4m3, int n_split_blocks, int batch,
                      hipStream_t stream);
