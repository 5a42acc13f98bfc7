// pkv_decode_attn: split-KV paged decode attention over an e4m3 or bf16 cache.
//
// "Smaller, faster, safer", section "Quantizing the KV cache": the FP8
// attention kernel converts cached values as it reads them. Section
// "Protecting a shared KV cache": the pages of one physical cache are
// shared by many requests (paged attention), and a request flagged by the
// separate tag check is never read.
//
// This file holds the entry point and the generic kernel used for shapes
// without a specialised one (decode_gqa_mfma.hip covers head dim 128 with up
// to 16 query heads per kv head, decode_mla.hip the latent layout).
//
// Work unit = (request b, kv head g, group of NH query heads, split c).
// A workgroup of four waves takes one work unit; wave w handles tokens
// c*S + w, c*S + w + 4, ...; lane l owns dimensions l, l + 64, ... of the
// head. Scores are reduced across the wave, each wave keeps its own online
// softmax state, and the four states are merged through LDS at the end.
#include "common.h"
#include "decode_params.h"
#include "step.h"

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// OCP E4M3 code -> float: 1.mmm * 2^(e-7), or 0.mmm * 2^-6 below; S.1111.111 is NaN.
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float v = e ? ldexpf(static_cast<float>(8u + m), static_cast<int>(e) - 10)
              : static_cast<float>(m) * 0.001953125f;
  if (e == 15u && m == 7u) v = NAN;
  return (c & 0x80u) ? -v : v;
}

template <bool kE4M3>
__device__ __forceinline__ float load_kv(const void* base, int64_t idx) {
  if constexpr (kE4M3) {
    return e4m3_value(static_cast<const uint8_t*>(base)[idx]);
  } else {
    return pkv::bf16_to_f32(static_cast<const uint16_t*>(base)[idx]);
  }
}

using Params = DecodeParams;

template <bool kE4M3, int DK, int DV, int NH>
__global__ void __launch_bounds__(256) decode_kernel(Params p) {
  constexpr int KPL = DK / pkv::kWave;  // K dims per lane
  constexpr int VPL = DV / pkv::kWave;  // V dims per lane
  constexpr int kWaves = 4;
  const int c = blockIdx.x;
  const int g = blockIdx.y / p.head_groups;
  const int hg = blockIdx.y - g * p.head_groups;
  const int b = blockIdx.z;
  const int lane = threadIdx.x % pkv::kWave;
  const int wave = threadIdx.x / pkv::kWave;
  const int G = p.num_q_heads / p.num_kv_heads;
  const int h0 = g * G + hg * NH;

  if (p.abort_flags && p.abort_flags[b]) return;
  const int L = p.seq_lens[b];
  if (L > p.max_seq_len) return;
  const int t_begin = c * p.split_tokens;
  if (t_begin >= L) return;
  const int t_end = min(L, t_begin + p.split_tokens);

  float q[NH][KPL];
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int i = 0; i < KPL; ++i)
      q[h][i] = pkv::bf16_to_f32(p.q[(static_cast<int64_t>(b) * p.num_q_heads + h0 + h) * DK +
                                     lane + pkv::kWave * i]);

  const float ks = kE4M3 ? p.k_scale[g] : 1.0f;
  const float vs = kE4M3 ? p.v_scale[g] : 1.0f;
  float m[NH], l[NH], acc[NH][VPL];
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.0f;
#pragma unroll
    for (int i = 0; i < VPL; ++i) acc[h][i] = 0.0f;
  }

  const int32_t* bt = p.block_table + static_cast<int64_t>(b) * p.max_pages;
  for (int t = t_begin + wave; t < t_end; t += kWaves) {
    const int32_t page = bt[t / p.page_size];
    if (page < 0 || page >= p.num_pages) continue;
    const int row = t % p.page_size;
    const int64_t krow = ((static_cast<int64_t>(page) * p.num_kv_heads + g) * p.page_size + row);
    float kv[KPL];
#pragma unroll
    for (int i = 0; i < KPL; ++i) kv[i] = load_kv<kE4M3>(p.k_pool, krow * DK + lane + pkv::kWave * i) * ks;
    float s[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      float part = 0.0f;
#pragma unroll
      for (int i = 0; i < KPL; ++i) part += q[h][i] * kv[i];
      for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off);
      s[h] = part * p.sm_scale_log2;  // log2 domain
    }
    float vv[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) vv[i] = load_kv<kE4M3>(p.v_pool, krow * p.v_row + lane + pkv::kWave * i) * vs;
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      const float mn = fmaxf(m[h], s[h]);
      const float alpha = exp2f(m[h] - mn);
      const float e = exp2f(s[h] - mn);
      l[h] = l[h] * alpha + e;
#pragma unroll
      for (int i = 0; i < VPL; ++i) acc[h][i] = acc[h][i] * alpha + e * vv[i];
      m[h] = mn;
    }
  }

  // merge the four waves' states
  __shared__ float sm[kWaves][NH][2];
  __shared__ float so[kWaves][NH][DV];
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      sm[wave][h][0] = m[h];
      sm[wave][h][1] = l[h];
    }
  }
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int i = 0; i < VPL; ++i) so[wave][h][lane + pkv::kWave * i] = acc[h][i];
  __syncthreads();

  const int64_t bh0 = static_cast<int64_t>(b) * p.num_q_heads + h0;
  for (int idx = threadIdx.x; idx < NH * DV; idx += blockDim.x) {
    const int h = idx / DV, d = idx - h * DV;
    float M = -INFINITY;
    bool nan = false;  // a NaN score (fmaxf leaves it out of M) reached a wave's state
    for (int w = 0; w < kWaves; ++w) {
      M = fmaxf(M, sm[w][h][0]);
      nan = nan || sm[w][h][1] != sm[w][h][1];
    }
    float den = 0.0f, num = 0.0f;
    if (M != -INFINITY) {
      for (int w = 0; w < kWaves; ++w) {
        const float f = exp2f(sm[w][h][0] - M);
        den += sm[w][h][1] * f;
        num += so[w][h][d] * f;
      }
    }
    const int64_t bh = bh0 + h;
    const bool any = M != -INFINITY || nan;
    p.o_part[(bh * p.max_splits + c) * DV + d] = M != -INFINITY ? num / den : (nan ? NAN : 0.0f);
    if (d == 0)
      p.lse_part[bh * p.max_splits + c] =
          M != -INFINITY ? (M + __log2f(den)) * kLn2 : (any ? NAN : -INFINITY);
  }
}

template <bool kE4M3, int DK, int DV, int NH>
int launch(const Params& p, int n_split_blocks, int batch, hipStream_t stream) {
  dim3 grid(n_split_blocks, p.num_kv_heads * p.head_groups, batch);
  decode_kernel<kE4M3, DK, DV, NH><<<grid, 256, 0, stream>>>(p);
  return pkv::launch_status();
}

template <bool kE4M3>
int dispatch(const Params& p, bool latent, int dk, int G, int n_split_blocks, int batch,
             hipStream_t stream) {
  if (latent) return launch<kE4M3, 576, 512, 4>(p, n_split_blocks, batch, stream);
  if (dk == 64) {
    switch (G) {
      case 1: return launch<kE4M3, 64, 64, 1>(p, n_split_blocks, batch, stream);
      case 2: return launch<kE4M3, 64, 64, 2>(p, n_split_blocks, batch, stream);
      case 4: return launch<kE4M3, 64, 64, 4>(p, n_split_blocks, batch, stream);
      default: return launch<kE4M3, 64, 64, 8>(p, n_split_blocks, batch, stream);
    }
  }
  switch (G) {
    case 1: return launch<kE4M3, 128, 128, 1>(p, n_split_blocks, batch, stream);
    case 2: return launch<kE4M3, 128, 128, 2>(p, n_split_blocks, batch, stream);
    case 4: return launch<kE4M3, 128, 128, 4>(p, n_split_blocks, batch, stream);
    default: return launch<kE4M3, 128, 128, 8>(p, n_split_blocks, batch, stream);
  }
}

}  // namespace

int decode_attn_impl(const pkv_cache* cache, const void* q, int32_t num_q_heads,
                     const int32_t* block_table, const int32_t* seq_lens, int32_t batch,
                     int32_t max_pages, int32_t max_seq_len, const uint8_t* abort_flags,
                     float sm_scale, int32_t split_tokens, int32_t max_splits, float* o_part,
                     float* lse_part, const StepDecodeInputs* step, hipStream_t stream,
                     bool validate_only) {
  int st = pkv::check_cache(cache);
  if (st) return st;
  if (!q || !block_table || !seq_lens || !o_part || !lse_part) return PKV_EINVAL;
  if (batch < 0 || max_pages < 1 || max_seq_len < 0 || max_splits < 1) return PKV_EINVAL;
  if (num_q_heads < 1 || num_q_heads % cache->num_kv_heads) return PKV_EINVAL;
  if (split_tokens < cache->page_size || split_tokens % cache->page_size) return PKV_EINVAL;
  if (static_cast<int64_t>(max_seq_len) > static_cast<int64_t>(max_pages) * cache->page_size)
    return PKV_EINVAL;
  const int64_t n_split_blocks = pkv::cdiv(max_seq_len, split_tokens);
  if (n_split_blocks > max_splits) return PKV_EINVAL;
  if (!(sm_scale == sm_scale)) return PKV_EINVAL;

  const bool latent = cache->v_pool == nullptr;
  const int G = num_q_heads / cache->num_kv_heads;
  const int dk = cache->head_dim_k, dv = cache->head_dim_v;
  int head_groups = 1;
  if (latent) {
    if (dk != 576 || dv != 512 || cache->num_kv_heads != 1 || num_q_heads % 16)
      return PKV_EUNSUPPORTED;
    head_groups = G / 4;
  } else {
    if (dk != dv || (dk != 64 && dk != 128)) return PKV_EUNSUPPORTED;
    if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return PKV_EUNSUPPORTED;
    head_groups = G > 8 ? G / 8 : 1;
  }
  if (batch == 0 || n_split_blocks == 0) return PKV_OK;
  if (batch > 65535 || static_cast<int64_t>(cache->num_kv_heads) * head_groups > 65535 ||
      n_split_blocks > (1 << 30))
    return PKV_EUNSUPPORTED;

  Params p{};
  p.k_pool = cache->k_pool;
  p.v_pool = latent ? cache->k_pool : cache->v_pool;
  p.k_scale = cache->k_scale;
  p.v_scale = latent ? cache->k_scale : cache->v_scale;
  p.k_row_scale = cache->k_row_scale;
  p.v_row_scale = cache->v_row_scale;
  p.q = static_cast<const uint16_t*>(q);
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.abort_flags = abort_flags;
  p.o_part = o_part;
  p.lse_part = lse_part;
  p.num_pages = cache->num_pages;
  p.page_size = cache->page_size;
  p.num_kv_heads = cache->num_kv_heads;
  p.num_q_heads = num_q_heads;
  p.max_pages = max_pages;
  p.max_seq_len = max_seq_len;
  p.split_tokens = split_tokens;
  p.max_splits = max_splits;
  p.head_groups = head_groups;
  p.batch = batch;
  p.q_len = 1;
  p.v_row = latent ? dk : dv;
  p.sm_scale_log2 = sm_scale * kLog2e;
  const bool e4m3 = cache->dtype == PKV_KV_E4M3;
  if (step) {
    // step form: every request is decoded (its flag is not known yet)
    if (validate_only) return PKV_OK;
    if (!step_two_launch(cache, num_q_heads, split_tokens) || abort_flags ||
        (step->expected_tags && !cache->page_tags) || !step->unit_flags || !step->k_new ||
        !step->v_new)
      return PKV_EINVAL;
    p.page_tags = cache->page_tags;
    p.expected_tags = step->expected_tags;
    p.unit_flags = step->unit_flags;
    p.k_new = step->k_new;
    p.v_new = step->v_new;
    return launch_decode_gqa_mfma_step(p, e4m3, static_cast<int>(n_split_blocks), batch, stream);
  }
  if (cache->k_row_scale) {
    // scales set at append: the grouped-query MFMA kernel reads them
    if (!gqa_mfma_path_supported(dk, dv, G, latent, split_tokens, cache->page_size))
      return PKV_EUNSUPPORTED;
    if (validate_only) return PKV_OK;
    return launch_decode_gqa_mfma(p, true, static_cast<int>(n_split_blocks), batch, stream);
  }
  if (validate_only) return PKV_OK;
  if (latent && mla_fast_path_supported(dk, dv, cache->num_kv_heads, num_q_heads,
                                        cache->page_size, split_tokens))
    return launch_decode_mla(p, e4m3, static_cast<int>(n_split_blocks), batch, stream);
  if (gqa_mfma_path_supported(dk, dv, G, latent, split_tokens, cache->page_size))
    return launch_decode_gqa_mfma(p, e4m3, static_cast<int>(n_split_blocks), batch, stream);
  return e4m3 ? dispatch<true>(p, latent, dk, G, static_cast<int>(n_split_blocks), batch, stream)
              : dispatch<false>(p, latent, dk, G, static_cast<int>(n_split_blocks), batch, stream);
}

extern "C" int pkv_decode_attn(const pkv_cache* cache, const void* q, int32_t num_q_heads,
                               const int32_t* block_table, const int32_t* seq_lens,
                               int32_t batch, int32_t max_pages, int32_t max_seq_len,
                               const uint8_t* abort_flags, float sm_scale, int32_t split_tokens,
                               int32_t max_splits, float* o_part, float* lse_part,
                               hipStream_t stream) {
  return decode_attn_impl(cache, q, num_q_heads, block_table, seq_lens, batch, max_pages,
                          max_seq_len, abort_flags, sm_scale, split_tokens, max_splits, o_part,
                          lse_part, nullptr, stream, false);
}

extern "C" int pkv_decode_attn_drafts(const pkv_cache* cache, const void* q, int32_t num_q_heads,
                                      int32_t q_len, const int32_t* block_table,
                                      const int32_t* seq_lens, int32_t batch, int32_t max_pages,
                                      int32_t max_seq_len, const uint8_t* abort_flags,
                                      float sm_scale, int32_t split_tokens, int32_t max_splits,
                                      float* o_part, float* lse_part, hipStream_t stream) {
  int st = pkv::check_cache(cache);
  if (st) return st;
  if (!q || !block_table || !seq_lens || !o_part || !lse_part) return PKV_EINVAL;
  if (batch < 0 || max_pages < 1 || max_seq_len < 0 || max_splits < 1) return PKV_EINVAL;
  if (q_len < 1 || q_len > 64) return PKV_EINVAL;
  if (num_q_heads < 1 || num_q_heads % cache->num_kv_heads) return PKV_EINVAL;
  if (split_tokens < cache->page_size || split_tokens % cache->page_size) return PKV_EINVAL;
  if (static_cast<int64_t>(max_seq_len) > static_cast<int64_t>(max_pages) * cache->page_size)
    return PKV_EINVAL;
  const int64_t n_split_blocks = pkv::cdiv(max_seq_len, split_tokens);
  if (n_split_blocks > max_splits) return PKV_EINVAL;
  if (!(sm_scale == sm_scale)) return PKV_EINVAL;
  const bool latent = cache->v_pool == nullptr;
  if (cache->k_row_scale) return PKV_EUNSUPPORTED;
  if (!drafts_path_supported(cache->head_dim_k, cache->head_dim_v, latent,
                             cache->dtype == PKV_KV_E4M3))
    return PKV_EUNSUPPORTED;
  if (batch == 0 || n_split_blocks == 0) return PKV_OK;
  const int G = num_q_heads / cache->num_kv_heads;
  const int row_groups = static_cast<int>((static_cast<int64_t>(q_len) * G + 31) / 32);
  Params p{};
  p.k_pool = cache->k_pool;
  p.v_pool = cache->v_pool;
  p.k_scale = cache->k_scale;
  p.v_scale = cache->v_scale;
  p.q = static_cast<const uint16_t*>(q);
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.abort_flags = abort_flags;
  p.o_part = o_part;
  p.lse_part = lse_part;
  p.num_pages = cache->num_pages;
  p.page_size = cache->page_size;
  p.num_kv_heads = cache->num_kv_heads;
  p.num_q_heads = num_q_heads;
  p.max_pages = max_pages;
  p.max_seq_len = max_seq_len;
  p.split_tokens = split_tokens;
  p.max_splits = max_splits;
  p.head_groups = 1;
  p.batch = batch;
  p.q_len = q_len;
  p.v_row = cache->head_dim_v;
  p.sm_scale_log2 = sm_scale * kLog2e;
  return launch_decode_drafts(p, static_cast<int>(n_split_blocks), batch, row_groups, stream);
}
