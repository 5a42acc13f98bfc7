// A decode step in two launches (internal): the decode kernel's step form
// checks each split's pages and reads the new token from its values, the
// combine's step form merges the verdicts and appends the new token.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv.h"

// What the combine's step form needs beyond the partials.
struct StepCombineArgs {
  const uint8_t* unit_flags;  // [batch][max_splits], the decode units' verdicts
  uint8_t* abort_out;         // [batch]
  const int32_t* block_table;
  const uint32_t* expected_tags;
  const uint32_t* page_tags;
  int num_pages, page_size, max_pages;
  int group;     // query heads per kv head
  int kv_heads;
  int head_dim;  // of K and V (equal)
  uint8_t* k_pool;
  uint8_t* v_pool;
  const float* k_scale;
  const float* v_scale;
  const uint16_t* k_new;  // bf16 [batch][kv_heads][head_dim]
  const uint16_t* v_new;
  bool e4m3;
};

// Inputs of the decode kernel's step form.
struct StepDecodeInputs {
  const uint32_t* expected_tags;
  uint8_t* unit_flags;
  const uint16_t* k_new;
  const uint16_t* v_new;
};

// The split-KV decode entry's work, with the step form's inputs (NULL: the
// plain decode of pkv_decode_attn). validate_only: every check, no launch.
int decode_attn_impl(const pkv_cache* cache, const void* q, int32_t num_q_heads,
                     const int32_t* block_table, const int32_t* seq_lens, int32_t batch,
                     int32_t max_pages, int32_t max_seq_len, const uint8_t* abort_flags,
                     float sm_scale, int32_t split_tokens, int32_t max_splits, float* o_part,
                     float* lse_part, const StepDecodeInputs* step, hipStream_t stream,
                     bool validate_only);

// pkv_combine's work; with sa non-NULL, the step form (head dim 128 only).
int combine_impl(const float* o_part, const float* lse_part, const int32_t* seq_lens,
                 int32_t batch, int32_t num_q_heads, int32_t head_dim_v, int32_t split_tokens,
                 int32_t max_splits, int32_t max_seq_len, const uint8_t* abort_flags, void* out,
                 float* lse_out, const StepCombineArgs* sa, hipStream_t stream);

// pkv_verify_append's work; slot NULL appends at each request's last row.
int verify_append_impl(const pkv_cache* cache, const int32_t* block_table,
                       const uint32_t* expected_tags, const int32_t* seq_lens, int32_t batch,
                       int32_t max_pages, uint8_t* abort_out, const void* k_new,
                       const void* v_new, const int32_t* slot, hipStream_t stream);

// The shapes the two-launch step form covers: the grouped-query MFMA kernel
// (head dim 128, up to 16 query heads per kv head) with static scales or a
// bf16 cache, at most 128 pages per split.
bool step_two_launch(const pkv_cache* cache, int32_t num_q_heads, int32_t split_tokens);
