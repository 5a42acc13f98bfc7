// pkv_combine: log-sum-exp merge of split-KV partials into the bf16 output.
//
// Not a step of the pages: splitting a long context into chunks and merging
// the chunk results (o_c, lse_c) by
//   M = max_c lse_c, w_c = exp(lse_c - M), o = sum w_c o_c / sum w_c
// is a reordering of the same softmax sum. One workgroup per (request,
// query head); each thread owns 4 consecutive output values (16-byte reads
// of every split's partial row). exp runs as exp2 with log2(e) folded in.
#include "common.h"

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__global__ void __launch_bounds__(128) combine_kernel(const float* __restrict__ o_part,
                                                      const float* __restrict__ lse_part,
                                                      const int32_t* __restrict__ seq_lens,
                                                      int heads, int dv, int split_tokens,
                                                      int max_splits, int max_seq_len,
                                                      const uint8_t* __restrict__ abort_flags,
                                                      uint16_t* __restrict__ out,
                                                      float* __restrict__ lse_out) {
  const int b = blockIdx.y;
  const int h = blockIdx.x;
  const int64_t bh = static_cast<int64_t>(b) * heads + h;
  const int32_t L = seq_lens[b];
  const bool aborted = abort_flags && abort_flags[b];
  const bool overflow = L > max_seq_len;
  const int n = (overflow || aborted || L <= 0) ? 0 : (L + split_tokens - 1) / split_tokens;
  const float* lse = lse_part + bh * max_splits;
  const float* op = o_part + bh * max_splits * dv;

  float M = -INFINITY;
  for (int c = 0; c < n; ++c) M = fmaxf(M, lse[c]);
  float den = 0.0f;
  for (int c = 0; c < n; ++c) den += exp2f((lse[c] - M) * kLog2e);

  for (int d0 = threadIdx.x * 4; d0 < dv; d0 += blockDim.x * 4) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < n; ++c) {
      const float w = exp2f((lse[c] - M) * kLog2e);
      const float4 v = *reinterpret_cast<const float4*>(op + static_cast<int64_t>(c) * dv + d0);
      acc[0] += w * v.x;
      acc[1] += w * v.y;
      acc[2] += w * v.z;
      acc[3] += w * v.w;
    }
    uint16_t r[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float x = acc[k] / den;
      if (aborted || n == 0) x = 0.0f;
      if (overflow && !aborted) x = NAN;
      r[k] = pkv::f32_to_bf16_rne(x);
    }
    uint2 pk;
    pk.x = static_cast<uint32_t>(r[0]) | (static_cast<uint32_t>(r[1]) << 16);
    pk.y = static_cast<uint32_t>(r[2]) | (static_cast<uint32_t>(r[3]) << 16);
    *reinterpret_cast<uint2*>(out + bh * dv + d0) = pk;
  }
  if (lse_out && threadIdx.x == 0) {
    float l = M + __log2f(den) * kLn2;
    if (aborted || n == 0) l = -INFINITY;
    if (overflow && !aborted) l = NAN;
    lse_out[bh] = l;
  }
}

}  // namespace

extern "C" int pkv_combine(const float* o_part, const float* lse_part, const int32_t* seq_lens,
                           int32_t batch, int32_t num_q_heads, int32_t head_dim_v,
                           int32_t split_tokens, int32_t max_splits, int32_t max_seq_len,
                           const uint8_t* abort_flags, void* out, float* lse_out,
                           hipStream_t stream) {
  if (!o_part || !lse_part || !seq_lens || !out || batch < 0 || num_q_heads < 1 ||
      head_dim_v < 8 || head_dim_v % 8 || split_tokens < 1 || max_splits < 1 || max_seq_len < 0)
    return PKV_EINVAL;
  if (pkv::cdiv(max_seq_len, split_tokens) > max_splits) return PKV_EINVAL;
  if ((reinterpret_cast<uintptr_t>(o_part) & 15u) || (reinterpret_cast<uintptr_t>(out) & 7u))
    return PKV_EINVAL;
  if (batch == 0) return PKV_OK;
  if (batch > 65535) return PKV_EUNSUPPORTED;
  combine_kernel<<<dim3(num_q_heads, batch), 128, 0, stream>>>(
      o_part, lse_part, seq_lens, num_q_heads, head_dim_v, split_tokens, max_splits, max_seq_len,
      abort_flags,
      static_cast<uint16_t*>(out), lse_out);
  return pkv::launch_status();
}
