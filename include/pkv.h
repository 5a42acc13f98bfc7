/*
 * pkv — FP8 (OCP E4M3) paged KV cache and single-token decode attention
 * for AMD Instinct MI355X (gfx950).
 *
 * Method: "Smaller, faster, safer: running Kimi and GLM at scale"
 * (Cloudflare blog).
 *   - Section "Quantizing the KV cache": keys and values are cached as
 *     8-bit floats (e4m3) instead of BF16, which halves the cache; the
 *     attention kernel converts the cached values as it reads them.
 *   - Section "Protecting a shared KV cache": every physical page has a
 *     tag that changes when the page is reallocated; the server records
 *     the pages and tags each request expects; before decode reads the
 *     cache the mapping is checked in a separate batch pass, and any
 *     request with a mismatch is aborted; with checking off, a no-op
 *     tracker costs nothing.
 *
 * A decode step is four calls on one stream, in this order:
 *   pkv_verify -> pkv_append -> pkv_decode_attn -> pkv_combine
 * The abort flags written by pkv_verify reach the later calls through
 * device memory, ordered by the stream; passing abort_flags == NULL to a
 * call is the no-op tracker (nothing is checked, nothing is skipped).
 *
 * Conventions for every entry point:
 *   - All array pointers are DEVICE pointers owned by the caller; the
 *     library keeps no reference after the call returns.
 *   - The library allocates no memory, never synchronises the host, throws
 *     nothing across this interface and keeps no state between calls.
 *   - Work is enqueued on `stream` (NULL = the null stream) and runs
 *     asynchronously; results are valid once the stream reaches them.
 *   - Return value: PKV_OK, or a negative pkv_status. Argument errors are
 *     detected on the host before anything is enqueued. PKV_EHIP means a
 *     launch failed (hipGetLastError); the stream's earlier work is intact.
 *   - A tag mismatch is data, not an error: it appears only in the flags.
 *   - bf16 means IEEE-754 binary32 truncated to its upper 16 bits (brain
 *     float), stored as uint16; e4m3 means OCP 8-bit float E4M3 (bias 7,
 *     max 448, NaN S.1111.111, no infinity) stored as uint8.
 */
#ifndef PKV_H
#define PKV_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pkv_status {
  PKV_OK = 0,
  PKV_EINVAL = -1,        /* a pointer, size or layout argument is invalid */
  PKV_EUNSUPPORTED = -2,  /* valid arguments, but no kernel for that shape */
  PKV_EHIP = -3           /* a HIP launch or runtime call failed */
} pkv_status;

typedef enum pkv_kv_dtype {
  PKV_KV_E4M3 = 1,  /* one byte per element, dequantised with a scale */
  PKV_KV_BF16 = 2   /* two bytes per element, used as stored */
} pkv_kv_dtype;

/*
 * The paged cache (caller-owned device memory).
 *
 * Layout (section "Protecting a shared KV cache" has requests share pages
 * of one physical cache; the pages give no layout, this one is chosen so a
 * (page, kv head) block is one contiguous run of page_size rows):
 *   k_pool: [num_pages][num_kv_heads][page_size][head_dim_k]
 *   v_pool: [num_pages][num_kv_heads][page_size][head_dim_v]
 * Token t of a request is in page block_table[t / page_size], row
 * t % page_size; one tag per page id covers K and V of every kv head.
 *
 * Latent layout (v_pool == NULL): one row of head_dim_k values per token
 * and kv head, and V is the first head_dim_v values of the same row (read
 * once, dequantised with k_scale).
 *
 * k_scale, v_scale: float32 [num_kv_heads], the dequantisation scale of
 *   each kv head (equal entries = one scale per tensor); an e4m3 code c
 *   stands for decode(c) * scale. Ignored for PKV_KV_BF16 (may be NULL).
 * page_tags: uint32 [num_pages], the current tag of each physical page;
 *   read only by pkv_verify (may be NULL otherwise).
 */
typedef struct pkv_cache {
  void* k_pool;
  void* v_pool;
  int32_t dtype;        /* pkv_kv_dtype */
  int32_t num_pages;    /* >= 1 */
  int32_t page_size;    /* tokens per page: 16, 32 or 64 */
  int32_t num_kv_heads; /* >= 1 */
  int32_t head_dim_k;   /* multiple of 16 */
  int32_t head_dim_v;   /* multiple of 16; <= head_dim_k when latent */
  const float* k_scale;
  const float* v_scale;
  const uint32_t* page_tags;
  /* Scales set at append, one per cached row (e4m3, separate K and V pools
   * only): float32 [num_pages][num_kv_heads][page_size], indexed like the
   * rows. When both are non-NULL, pkv_append gives each new row the scale
   * fl32(amax(row) / 448) (1 for an all-zero row), stores it here and
   * encodes the row under it, and decode reads each row with its own
   * scale; k_scale and v_scale are then not used. Both NULL: the static
   * per-head scales. */
  float* k_row_scale;
  float* v_row_scale;
} pkv_cache;

/*
 * Per-head (or per-tensor) e4m3 scales from the largest magnitude.
 * Section "Quantizing the KV cache" gives no scale rule; this library's is
 * a static scale s = fl32(amax / 448) (a correctly rounded float32
 * division; s = 1 when amax = 0), 448 being the largest e4m3 magnitude.
 *
 *   x:         bf16 [n_rows][num_heads][head_dim], e.g. all K rows.
 *   per_head:  nonzero -> scale_out[h] from head h's values only;
 *              zero    -> every scale_out[h] from the whole tensor.
 *   scale_out: float32 [num_heads]; also used as scratch during the call.
 * NaN inputs give a NaN scale. EINVAL: NULL pointer, n_rows < 1,
 * num_heads < 1, head_dim not a multiple of 8.
 */
int pkv_scales_from_amax(const void* x, int64_t n_rows, int32_t num_heads,
                         int32_t head_dim, int32_t per_head, float* scale_out,
                         hipStream_t stream);

/*
 * Quantise-on-append (section "Quantizing the KV cache": the cache is held
 * in e4m3).
 *
 * For every token i < n_tokens with slot[i] >= 0, every kv head h and
 * dimension d:
 *   e4m3: pool[slot/P][h][slot%P][d] = RNE_SAT(fl32(x / scale[h]))
 *         (round to nearest, ties to even; |y| >= 448 and infinities become
 *          +-448; NaN becomes the NaN code of its sign; -0 stays -0)
 *   bf16: the value is copied unchanged.
 *   k_new: bf16 [n_tokens][num_kv_heads][head_dim_k]
 *   v_new: bf16 [n_tokens][num_kv_heads][head_dim_v]; must be NULL for the
 *          latent layout (V lives inside the K row).
 *   slot:  int32 [n_tokens], page * page_size + row; < 0 = skip the token;
 *          slots past the pool (>= num_pages * page_size) are skipped too.
 *   token_req, abort_flags: when both are non-NULL, token i is skipped if
 *          abort_flags[token_req[i]] != 0 (an aborted request writes
 *          nothing). token_req: int32 [n_tokens]; abort_flags: uint8 [B].
 * Two tokens with the same slot in one call race (either may win).
 * EINVAL: NULL pool/scale/k_new/slot, v_new given for latent or missing
 * otherwise, n_tokens < 0, invalid cache geometry.
 */
int pkv_append(const pkv_cache* cache, const void* k_new, const void* v_new,
               const int32_t* slot, const int32_t* token_req,
               const uint8_t* abort_flags, int64_t n_tokens, hipStream_t stream);

/*
 * Integrity check (section "Protecting a shared KV cache"): for each
 * request b with n = ceil(seq_lens[b] / page_size) pages,
 *   abort_out[b] = 1 if some j < n has block_table[b][j] outside
 *                  [0, num_pages), or page_tags[block_table[b][j]] !=
 *                  expected_tags[b][j], or j >= max_pages; else 0.
 * Entries past n are ignored. A separate launch: the decode kernel reads
 * the flags after it, never alongside it.
 *
 *   block_table:   int32  [batch][max_pages]
 *   expected_tags: uint32 [batch][max_pages], the tags recorded by the caller
 *   seq_lens:      int32  [batch], tokens of each request including the one
 *                  appended this step (<= 0 = empty request, never aborted)
 *   abort_out:     uint8  [batch], fully overwritten.
 * EINVAL: NULL pointers (cache->page_tags included), batch < 0,
 * max_pages < 1.
 */
int pkv_verify(const pkv_cache* cache, const int32_t* block_table,
               const uint32_t* expected_tags, const int32_t* seq_lens,
               int32_t batch, int32_t max_pages, uint8_t* abort_out,
               hipStream_t stream);

/*
 * pkv_verify and then pkv_append of one new token per request, in one launch
 * (sections "Protecting a shared KV cache" and "Quantizing the KV cache":
 * the mapping is checked before anything reads or writes the request's
 * pages; an aborted request writes nothing).
 *
 * For each request b < batch: abort_out[b] as pkv_verify computes it; then,
 * unless abort_out[b] is set or slot[b] < 0 (or past the pool), the rows
 * k_new[b] (and v_new[b]) are written at slot[b] exactly as pkv_append
 * writes them (static scales, scales set at append, or a bf16 copy).
 *   k_new: bf16 [batch][num_kv_heads][head_dim_k]; v_new: bf16
 *          [batch][num_kv_heads][head_dim_v], NULL for the latent layout
 *   slot:  int32 [batch]
 *   other arguments as for pkv_verify.
 * One workgroup per request: a request's flag and its append are in the
 * same workgroup, so no other ordering is needed. Two requests with the same
 * slot race. Errors as for pkv_verify and pkv_append.
 */
int pkv_verify_append(const pkv_cache* cache, const int32_t* block_table,
                      const uint32_t* expected_tags, const int32_t* seq_lens, int32_t batch,
                      int32_t max_pages, uint8_t* abort_out, const void* k_new,
                      const void* v_new, const int32_t* slot, hipStream_t stream);

/*
 * Split-KV paged decode attention (section "Quantizing the KV cache": the
 * FP8 kernel converts values as it reads them; section "Protecting a shared
 * KV cache": paged attention over a shared physical cache).
 *
 * For request b (skipped entirely when abort_flags != NULL and
 * abort_flags[b] != 0), split c < ceil(L / split_tokens) covering tokens
 * [c*S, min((c+1)*S, L)), and query head h reading kv head
 * g = h / (num_q_heads / num_kv_heads):
 *   s_t        = sm_scale * sum_d q[b][h][d] * K[t][g][d]
 *   o_part     = sum_t exp(s_t - m) * V[t][g][:] / sum_t exp(s_t - m)
 *   lse_part   = m + ln sum_t exp(s_t - m)        (natural log)
 * where K, V are the dequantised cached values (code * scale for e4m3).
 *
 *   q:        bf16 [batch][num_q_heads][head_dim_k]
 *   block_table, seq_lens, max_pages: as for pkv_verify.
 *   max_seq_len: an upper bound on every seq_lens[b], used to size the
 *            launch; must satisfy max_seq_len <= max_pages * page_size and
 *            ceil(max_seq_len / split_tokens) <= max_splits. A request with
 *            seq_lens[b] > max_seq_len gets NaN outputs from pkv_combine.
 *   split_tokens: S, a positive multiple of page_size.
 *   o_part:   float32 [batch][num_q_heads][max_splits][head_dim_v]
 *   lse_part: float32 [batch][num_q_heads][max_splits]
 * Only the splits a request has are written; aborted requests write
 * nothing. For the latent layout with query heads in multiples of 128, the
 * launch gives every compute unit an equal share of the batch's tokens, cut
 * at split boundaries: a run of consecutive splits of one request decoded
 * together writes its partial in its first split's row, and the other rows
 * of the run get lse_part = -inf with o_part left unwritten (pkv_combine
 * skips such rows; the merge is the same). A block-table entry outside
 * [0, num_pages) is never read: its tokens are left out (pkv_verify turns
 * such requests into aborts).
 * EINVAL: NULL pointers, num_q_heads not a multiple of num_kv_heads,
 * split_tokens invalid, max_seq_len or max_splits inconsistent.
 * EUNSUPPORTED: a shape with no kernel; supported are
 *   grouped-query: head_dim_k == head_dim_v in {64, 128},
 *                  num_q_heads / num_kv_heads in {1, 2, 4, 8, 16};
 *   latent:        head_dim_k == 576, head_dim_v == 512, one kv head,
 *                  num_q_heads a multiple of 16.
 */
int pkv_decode_attn(const pkv_cache* cache, const void* q, int32_t num_q_heads,
                    const int32_t* block_table, const int32_t* seq_lens,
                    int32_t batch, int32_t max_pages, int32_t max_seq_len,
                    const uint8_t* abort_flags, float sm_scale,
                    int32_t split_tokens, int32_t max_splits, float* o_part,
                    float* lse_part, hipStream_t stream);

/*
 * Log-sum-exp merge of the split partials (not on the pages; a reordering
 * of the same softmax sum). For request b with n = ceil(L / split_tokens)
 * splits:
 *   M = max_c lse_c, w_c = exp(lse_c - M),
 *   out[b][h] = bf16_RNE( sum_c w_c * o_c / sum_c w_c ),
 * where a row with lse_c = -inf adds nothing and its o_c is not read,
 *   lse_out[b][h] = M + ln sum_c w_c.
 * Aborted (abort_flags[b] != 0) or empty (L <= 0) requests get out = 0 and
 * lse_out = -inf; a request with L > max_seq_len gets NaN.
 *   o_part, lse_part, split_tokens, max_splits, max_seq_len: as passed to
 *            pkv_decode_attn.
 *   out:     bf16 [batch][num_q_heads][head_dim_v]
 *   lse_out: float32 [batch][num_q_heads], or NULL.
 * EINVAL: NULL pointers, non-positive sizes, head_dim_v not a multiple of 8,
 * ceil(max_seq_len / split_tokens) > max_splits.
 * EUNSUPPORTED: head_dim_v not in {64, 128, 256, 512}.
 */
int pkv_combine(const float* o_part, const float* lse_part,
                const int32_t* seq_lens, int32_t batch, int32_t num_q_heads,
                int32_t head_dim_v, int32_t split_tokens, int32_t max_splits,
                int32_t max_seq_len, const uint8_t* abort_flags, void* out,
                float* lse_out, hipStream_t stream);

/*
 * One decode step in two launches (sections "Protecting a shared KV cache"
 * and "Quantizing the KV cache": the mapping is checked before anything read
 * through it is returned, an aborted request writes nothing, the new token
 * is stored as e4m3 under its kv head's scale and the attention kernel
 * converts codes as it reads them). pkv_step_decode then pkv_step_combine,
 * on one stream with the same arguments, give the abort flags, cache
 * contents, out and lse_out of
 *   pkv_verify_append(cache, block_table, expected_tags, seq_lens, batch,
 *                     max_pages, abort_out, k_new, v_new, slot)
 *   pkv_decode_attn(..., abort_flags = abort_out, ...)
 *   pkv_combine(..., abort_flags = abort_out, out, lse_out)
 * bit for bit, with each request's new token at the row of its last
 * position: slot[b] = block_table[b][(L-1) / P] * P + (L-1) % P for
 * L = seq_lens[b] >= 1 (no token when L <= 0, when (L-1) / P >= max_pages,
 * or when that page lies outside the pool: cases only a step without the
 * check can reach, since the check aborts such a request).
 *
 * Two-launch form (separate K and V pools, head_dim_k == head_dim_v == 128,
 * e4m3 with per-head scales or bf16, up to 16 query heads per kv head,
 * split_tokens <= 128 * page_size): pkv_step_decode decodes every request;
 * the units of kv head 0 check their split's pages and write
 * unit_flags[b][c], and each request's last split reads the new token's row
 * from k_new / v_new (encoded as pkv_append encodes it) instead of the pool.
 * pkv_step_combine ORs a request's flags into abort_out[b] (checking a
 * request with seq_lens[b] > max_seq_len, which has no units, in full),
 * appends the new token of each request that stands, and merges. Other
 * shapes: pkv_step_decode runs the check-and-append and the decode launches,
 * pkv_step_combine the merge.
 *
 *   k_new, v_new: bf16 [batch][num_kv_heads][head_dim], 16-byte aligned;
 *                 v_new NULL for the latent layout
 *   expected_tags: as for pkv_verify, or NULL for the step without the
 *                 check (no tag is read, every request stands)
 *   unit_flags:   uint8 [batch][max_splits], scratch between the two calls
 *   abort_out:    uint8 [batch], final after pkv_step_combine
 *   o_part, lse_part: scratch as for pkv_decode_attn (in the two-launch form
 *                 an aborted request's partials are computed too)
 *   other arguments as for pkv_verify_append, pkv_decode_attn, pkv_combine.
 * A request's new row must not lie inside another request's context in the
 * same step (the three-launch order would show it to that request; here the
 * other request reads the pool's previous row). Device pointers,
 * caller-owned. Errors: those of the three calls (checked before anything is
 * launched); EINVAL also for NULL unit_flags / abort_out, expected_tags
 * without cache->page_tags, or misaligned k_new / v_new.
 */
int pkv_step_decode(const pkv_cache* cache, const void* q, int32_t num_q_heads,
                    const void* k_new, const void* v_new, const int32_t* block_table,
                    const uint32_t* expected_tags, const int32_t* seq_lens, int32_t batch,
                    int32_t max_pages, int32_t max_seq_len, float sm_scale,
                    int32_t split_tokens, int32_t max_splits, float* o_part, float* lse_part,
                    uint8_t* unit_flags, uint8_t* abort_out, hipStream_t stream);
int pkv_step_combine(const pkv_cache* cache, int32_t num_q_heads, const void* k_new,
                     const void* v_new, const int32_t* block_table,
                     const uint32_t* expected_tags, const int32_t* seq_lens, int32_t batch,
                     int32_t max_pages, int32_t max_seq_len, int32_t split_tokens,
                     int32_t max_splits, const float* o_part, const float* lse_part,
                     const uint8_t* unit_flags, uint8_t* abort_out, void* out,
                     float* lse_out, hipStream_t stream);
/* Host only: 2 if the step of this shape runs in two launches, 3 if the two
 * calls run the three. Reads the cache's geometry (NULL-ness of v_pool and
 * k_row_scale, head dims, page size, kv heads); EINVAL for NULL or an
 * invalid page size or kv head count. */
int pkv_step_launches(const pkv_cache* cache, int32_t num_q_heads, int32_t split_tokens);

/*
 * Decode attention of a token and its drafts verified together (Cloudflare's
 * post on serving extra-large models, speculative decoding section: a draft
 * model proposes a few future tokens and the target model checks them in
 * one forward pass; "Smaller, faster, safer", section "Quantizing the KV
 * cache": the cache is read as e4m3).
 *
 * Request b's last q_len cached tokens are the current token and its q_len - 1
 * drafts (appended this step). Query position j < q_len, the token at
 * position L - q_len + j, attends to cached tokens 0 .. L - q_len + j only:
 * for split c and query row (j, h),
 *   o_part / lse_part as for pkv_decode_attn over the tokens
 *   [c*S, min((c+1)*S, L - q_len + j + 1)), with o = 0 and lse = -inf where
 *   that range is empty.
 *   q:        bf16 [batch][q_len][num_q_heads][head_dim_k]
 *   o_part:   float32 [batch][q_len * num_q_heads][max_splits][head_dim_v]
 *   lse_part: float32 [batch][q_len * num_q_heads][max_splits]
 * Every split c < ceil(L / S) of every query row is written, so pkv_combine
 * with num_q_heads' = q_len * num_q_heads merges them into
 * out bf16 [batch][q_len][num_q_heads][head_dim_v].
 * Other arguments and errors as for pkv_decode_attn; also EINVAL for
 * q_len outside [1, 64]. EUNSUPPORTED unless the cache is e4m3 with
 * separate K and V pools and head_dim_k == head_dim_v == 128, and for
 * split_tokens > 128 * page_size (a split's page ids are held in registers).
 */
int pkv_decode_attn_drafts(const pkv_cache* cache, const void* q, int32_t num_q_heads,
                           int32_t q_len, const int32_t* block_table, const int32_t* seq_lens,
                           int32_t batch, int32_t max_pages, int32_t max_seq_len,
                           const uint8_t* abort_flags, float sm_scale, int32_t split_tokens,
                           int32_t max_splits, float* o_part, float* lse_part,
                           hipStream_t stream);

/*
 * Prefill -> decode handoff of whole pages (section "Quantizing the KV
 * cache": decode holds the cache as e4m3 while prefill keeps BF16, so a
 * prefill's pages are re-encoded on their way into the decode pool; section
 * "Protecting a shared KV cache": a page's tag changes whenever it is
 * reallocated).
 *
 * For every pair i < n_pages, kv head h, row r < page_size and dim d:
 *   dst->k_pool[dst_pages[i]][h][r][d] =
 *       RNE_SAT(fl32(src->k_pool[src_pages[i]][h][r][d] / dst->k_scale[h]))
 *   (V likewise from dst->v_scale; a latent cache converts its whole rows)
 *   dst_tags[dst_pages[i]] = new_tags[i]        (when both are non-NULL)
 * with the encoding of pkv_append. The scales are the destination pool's
 * (set once, e.g. by pkv_scales_from_amax over the prefill pool viewed as
 * [pages][num_kv_heads][page_size * head_dim]); values beyond them saturate.
 *   src:       a PKV_KV_BF16 cache; dst: a PKV_KV_E4M3 cache with the same
 *              page size, kv heads, head dims and layout (separate or latent V)
 *   src_pages, dst_pages: int32 [n_pages] device arrays; a pair naming a
 *              page outside its pool is skipped (nothing written)
 *   new_tags:  uint32 [n_pages] or NULL; dst_tags: uint32 [dst num_pages]
 *              (the destination's page tags) or NULL; both or neither
 * Two pairs with the same destination page race. Device pointers, caller-owned.
 * EINVAL: NULL pointers, dtypes or geometries that do not match, only one of
 * new_tags / dst_tags, n_pages < 0, pools not 16-byte aligned.
 */
int pkv_requantize_pages(const pkv_cache* src, const pkv_cache* dst,
                         const int32_t* src_pages, const int32_t* dst_pages,
                         const uint32_t* new_tags, uint32_t* dst_tags, int32_t n_pages,
                         hipStream_t stream);

/*
 * INT4 weight-only linear layer of the decode phase ("Smaller, faster,
 * safer", section on model weights: GLM's weights held as 4-bit integers for
 * decode, where each token streams them out of GPU memory).
 *
 *   y[b][r] = bf16_RNE( sum_k x[b][k] * q[r][k] * scales[k / 128][r] )
 * for b < batch, r < n, with q[r][k] the 4-bit two's-complement code of
 * input k of row r (-8 .. 7).
 *   x:      bf16 [batch][k]
 *   w:      uint8 [n][k / 2]; input k of row r in byte k / 2 of the row,
 *           even k in the low nibble (bits 0..3), odd k in the high nibble
 *   scales: bf16 [k / 128][n] (group-major: one group's scales of
 *           consecutive rows are contiguous)
 *   y:      bf16 [batch][n], fully written
 *   workspace: device scratch of at least pkv_int4_linear_workspace(batch,
 *           n, k) bytes, 16-byte aligned, or NULL. Above 8 tokens, when the
 *           rows alone give too few workgroups, the inputs are split over
 *           several workgroups that leave fp32 partial sums here, and a
 *           second kernel adds them up. Overwritten; nothing is kept between
 *           calls, but calls sharing a workspace must not overlap in time.
 *           Without a workspace such a call takes a slower kernel.
 * Accumulation is fp32. Device pointers, caller-owned; x, w, scales and
 * workspace 16-byte aligned. EINVAL: NULL pointers, batch outside [1, 64],
 * n not a multiple of 32, k not a multiple of 1024, misaligned pointers.
 */
int pkv_int4_linear(const void* x, const uint8_t* w, const void* scales, int32_t batch,
                    int32_t n, int32_t k, void* y, void* workspace, hipStream_t stream);

/*
 * Bytes of workspace pkv_int4_linear wants for this layer and batch (0: it
 * needs none): the fp32 partial sums. EINVAL for batch outside [1, 64] or
 * n, k < 1.
 */
int64_t pkv_int4_linear_workspace(int32_t batch, int32_t n, int32_t k);

/*
 * Host helper: a split size for pkv_decode_attn on this cache and batch.
 *   num_q_heads   query heads of the batch (as passed to pkv_decode_attn)
 *   batch         requests in the batch
 *   total_tokens  sum of the requests' lengths (as in seq_lens), or 0 if
 *                 unknown (then batch * max_seq_len is assumed)
 *   max_seq_len   longest request
 * The result is a multiple of page_size, chosen for the kernel that will
 * run: as long as possible (fewer partial rows to write and merge) while the
 * batch still splits into enough work units to occupy every compute unit.
 * Only the cache's geometry (dtype, page size, heads, dims, latent layout)
 * is read; no pointer in it is used. Returns a positive token count, or
 * PKV_EINVAL.
 */
int32_t pkv_suggest_split(const pkv_cache* cache, int32_t num_q_heads, int32_t batch,
                          int64_t total_tokens, int32_t max_seq_len);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops that forbid hipMalloc): pkv_decode_attn followed by
 * pkv_combine on `stream`, with the split partials (o_part, lse_part) held in
 * a fixed array of PKV_STATIC_SCRATCH_BYTES inside the library instead of
 * caller buffers. Calls no allocating routine.
 *
 * Arguments and results as for pkv_decode_attn then pkv_combine with
 * max_splits = max(1, ceil(max_seq_len / split_tokens)); the caller passes
 * only the inputs and the outputs:
 *   out:     bf16 [batch][num_q_heads][head_dim_v]
 *   lse_out: float32 [batch][num_q_heads], or NULL.
 * The partials need batch * num_q_heads * max_splits * (head_dim_v + 1) * 4
 * bytes (the first part rounded up to 256); above PKV_STATIC_SCRATCH_BYTES
 * the call returns PKV_EINVAL and enqueues nothing (the allocating pair then
 * serves). Each GPU holds one copy of the array from the first call on it
 * until the process ends; every call on that GPU shares it, so calls that
 * overlap in time on one GPU (two streams, two threads) race and must be
 * ordered by the caller. Nothing in it needs clearing between calls.
 * Errors: as for pkv_decode_attn and pkv_combine; PKV_EHIP if the array's
 * address cannot be obtained.
 */
#define PKV_STATIC_SCRATCH_BYTES (64ll << 20)
int pkv_decode_attn_static(const pkv_cache* cache, const void* q, int32_t num_q_heads,
                           const int32_t* block_table, const int32_t* seq_lens,
                           int32_t batch, int32_t max_pages, int32_t max_seq_len,
                           const uint8_t* abort_flags, float sm_scale, int32_t split_tokens,
                           void* out, float* lse_out, hipStream_t stream);

/*
 * Measurement helper, not part of the method: writes `value` to n_words
 * consecutive uint32 words of dst (device pointer, 16-byte aligned,
 * caller-owned) with a plain write kernel. Writing a buffer several times
 * the 256 MB last-level cache between timed decode steps evicts the
 * previous step's lines, as the model's other layers do in serving.
 * EINVAL: NULL or misaligned dst, n_words < 0.
 */
int pkv_fill_u32(void* dst, int64_t n_words, uint32_t value, hipStream_t stream);

/*
 * Measurement helper, not part of the method: reads the whole 16-byte words
 * of n_words uint32 words of src (device pointer, 16-byte aligned) and XORs
 * what it read into *sink (one device word, caller-owned). Read after
 * pkv_fill_u32 over the same buffer, it evicts the dirty lines the fill
 * left, so their write-back is not charged to the next timed step.
 * EINVAL: NULL or misaligned pointers, n_words < 0.
 */
int pkv_read_u32(const void* src, int64_t n_words, uint32_t* sink, hipStream_t stream);

/* Host helper: a static string naming a status code. */
const char* pkv_strerror(int32_t status);

/* Host helper: library version, major * 10000 + minor * 100 + patch. */
int32_t pkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
