// pkv_combine: log-sum-exp merge of split-KV partials into the bf16 output.
//
// Not a step of the pages: splitting a long context into chunks and merging
// the chunk results (o_c, lse_c) by
//   M = max_c lse_c, w_c = exp(lse_c - M), o = sum w_c o_c / sum w_c
// is a reordering of the same softmax sum. exp runs as exp2 with log2(e)
// folded in.
#include "common.h"

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// One workgroup of four waves per (request, query head). The maximum lse is
// reduced over the whole workgroup; then wave w merges splits w, w+4, ...
// (each lane owns VPL consecutive values of the head) and the four partial
// sums meet in LDS.
template <int VPL>
__global__ void __launch_bounds__(256) combine_kernel(const float* __restrict__ o_part,
                                                      const float* __restrict__ lse_part,
                                                      const int32_t* __restrict__ seq_lens,
                                                      int heads, int split_tokens, int max_splits,
                                                      int max_seq_len,
                                                      const uint8_t* __restrict__ abort_flags,
                                                      uint16_t* __restrict__ out,
                                                      float* __restrict__ lse_out) {
  constexpr int kDv = VPL * 64;
  constexpr int kWaves = 4;
  const int b = blockIdx.y;
  const int h = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t bh = static_cast<int64_t>(b) * heads + h;
  const int32_t L = seq_lens[b];
  const bool aborted = abort_flags && abort_flags[b];
  const bool overflow = L > max_seq_len;
  const int n = (overflow || aborted || L <= 0) ? 0 : (L + split_tokens - 1) / split_tokens;
  const float* lse = lse_part + bh * max_splits;
  const float* op = o_part + bh * max_splits * kDv;

  __shared__ float red[kWaves];
  __shared__ float den_s[kWaves];
  __shared__ float acc_s[kWaves][kDv];

  float mx = -INFINITY;
  for (int c = threadIdx.x; c < n; c += blockDim.x) mx = fmaxf(mx, lse[c]);
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const bool empty = (M == -INFINITY);

  float acc[VPL];
#pragma unroll
  for (int k = 0; k < VPL; ++k) acc[k] = 0.0f;
  float den = 0.0f;
  if (!empty) {
    for (int c = wave; c < n; c += kWaves) {
      const float w = exp2f((lse[c] - M) * kLog2e);
      den += w;
      const float* src = op + static_cast<int64_t>(c) * kDv + lane * VPL;
      if constexpr (VPL == 1) {
        acc[0] += w * src[0];
      } else if constexpr (VPL == 2) {
        const float2 v = *reinterpret_cast<const float2*>(src);
        acc[0] += w * v.x;
        acc[1] += w * v.y;
      } else {
#pragma unroll
        for (int k = 0; k < VPL; k += 4) {
          const float4 v = *reinterpret_cast<const float4*>(src + k);
          acc[k] += w * v.x;
          acc[k + 1] += w * v.y;
          acc[k + 2] += w * v.z;
          acc[k + 3] += w * v.w;
        }
      }
    }
  }
#pragma unroll
  for (int k = 0; k < VPL; ++k) acc_s[wave][lane * VPL + k] = acc[k];
  if (lane == 0) den_s[wave] = den;
  __syncthreads();

  const float D = den_s[0] + den_s[1] + den_s[2] + den_s[3];
  for (int d = threadIdx.x; d < kDv; d += blockDim.x) {
    float x = (acc_s[0][d] + acc_s[1][d] + acc_s[2][d] + acc_s[3][d]) / D;
    if (aborted || n == 0 || empty) x = 0.0f;
    if (overflow && !aborted) x = NAN;
    out[bh * kDv + d] = pkv::f32_to_bf16_rne(x);
  }
  if (lse_out && threadIdx.x == 0) {
    float l = M + __log2f(D) * kLn2;
    if (aborted || n == 0 || empty) l = -INFINITY;
    if (overflow && !aborted) l = NAN;
    lse_out[bh] = l;
  }
}

template <int VPL>
int launch(const float* o_part, const float* lse_part, const int32_t* seq_lens, int batch,
           int heads, int split_tokens, int max_splits, int max_seq_len,
           const uint8_t* abort_flags, uint16_t* out, float* lse_out, hipStream_t stream) {
  combine_kernel<VPL><<<dim3(heads, batch), 256, 0, stream>>>(
      o_part, lse_part, seq_lens, heads, split_tokens, max_splits, max_seq_len, abort_flags, out,
      lse_out);
  return pkv::launch_status();
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
  if ((reinterpret_cast<uintptr_t>(o_part) & 15u) || (reinterpret_cast<uintptr_t>(out) & 1u))
    return PKV_EINVAL;
  if (batch == 0) return PKV_OK;
  if (batch > 65535 || num_q_heads > 65535) return PKV_EUNSUPPORTED;
  auto* o = static_cast<uint16_t*>(out);
  switch (head_dim_v) {
    case 64:
      return launch<1>(o_part, lse_part, seq_lens, batch, num_q_heads, split_tokens, max_splits,
                       max_seq_len, abort_flags, o, lse_out, stream);
    case 128:
      return launch<2>(o_part, lse_part, seq_lens, batch, num_q_heads, split_tokens, max_splits,
                       max_seq_len, abort_flags, o, lse_out, stream);
    case 256:
      return launch<4>(o_part, lse_part, seq_lens, batch, num_q_heads, split_tokens, max_splits,
                       max_seq_len, abort_flags, o, lse_out, stream);
    case 512:
      return launch<8>(o_part, lse_part, seq_lens, batch, num_q_heads, split_tokens, max_splits,
                       max_seq_len, abort_flags, o, lse_out, stream);
    default:
      return PKV_EUNSUPPORTED;
  }
}
