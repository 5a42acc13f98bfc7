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
constexpr int kDirectRows = 4;  // rows per thread group on the one-pass path

// One workgroup of 256 threads per (request, query head). The maximum lse is
// reduced over the workgroup. Then, 256 split rows at a time, the rows that
// hold tokens (lse > -inf; the latent kernel leaves the other rows of a run
// of splits it merged empty) are listed in LDS in split order, with their
// weights, and the threads split into P = 256 / (Dv / 4) groups: group sg
// merges listed rows sg, sg + P, ... with each thread owning one 16-byte
// chunk of the head, so a workgroup reads P whole split rows per step and
// consecutive steps' loads are independent. The P partial sums meet in LDS.
// The order of every sum is fixed, so the result is the same bits on every
// run.
//
// When every split row of a head fits in one pass (kRows rows per thread
// group, max_splits <= kP * kRows), the rows' lse and o chunks are all
// loaded at the start, beside the request's length: rows are bounded by
// max_splits, not by the length, so every load is in the buffers, and rows
// past the length are dropped afterwards. One memory round trip instead of
// three (length, lse, o).
template <int DV, bool kDirect>
__global__ void __launch_bounds__(256) combine_kernel(const float* __restrict__ o_part,
                                                      const float* __restrict__ lse_part,
                                                      const int32_t* __restrict__ seq_lens,
                                                      int heads, int split_tokens, int max_splits,
                                                      int max_seq_len,
                                                      const uint8_t* __restrict__ abort_flags,
                                                      uint16_t* __restrict__ out,
                                                      float* __restrict__ lse_out) {
  constexpr int kC = DV / 4;     // 16-byte chunks per split row
  constexpr int kP = 256 / kC;   // split rows merged side by side
  constexpr int kRows = kDirectRows;
  const int b = blockIdx.y;
  const int h = blockIdx.x;
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int sg = t / kC, ch = t % kC;
  const int64_t bh = static_cast<int64_t>(b) * heads + h;
  const int32_t L = seq_lens[b];
  const bool aborted = abort_flags && abort_flags[b];
  const bool overflow = L > max_seq_len;
  const int n = (overflow || aborted || L <= 0) ? 0 : (L + split_tokens - 1) / split_tokens;
  const float* lse = lse_part + bh * max_splits;
  const float4* op = reinterpret_cast<const float4*>(o_part + bh * max_splits * DV);

  __shared__ float red[4];
  __shared__ int any_s[4];
  __shared__ int cnt_s[4];
  __shared__ int idx_s[256];
  __shared__ float w_s[256];
  __shared__ float den_s[kP];
  __shared__ float4 acc_s[kP][kC];

  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  float den = 0.0f;
  float M;
  bool empty;
  if constexpr (kDirect) {
    // rows sg + kP j of this thread's group, all loaded at once
    float lr[kRows];
    float4 vr[kRows];
#pragma unroll
    for (int j = 0; j < kRows; ++j) {
      const int r = sg + kP * j;
      lr[j] = r < max_splits ? lse[r] : -INFINITY;
      vr[j] = r < max_splits ? op[static_cast<int64_t>(r) * kC + ch] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float mx = -INFINITY;
    bool any = false;
#pragma unroll
    for (int j = 0; j < kRows; ++j) {
      if (sg + kP * j >= n) lr[j] = -INFINITY;  // past the request's length
      mx = fmaxf(mx, lr[j]);
      any = any || lr[j] != -INFINITY;
    }
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    const bool wave_any = __ballot(any) != 0;
    if (lane == 0) {
      red[wave] = mx;
      any_s[wave] = wave_any;
    }
    __syncthreads();
    M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    // empty: no row holds a partial (a NaN lse is a partial: it makes the
    // output NaN, which fmaxf alone would hide)
    empty = (any_s[0] | any_s[1] | any_s[2] | any_s[3]) == 0;
    if (!empty) {
#pragma unroll
      for (int j = 0; j < kRows; ++j) {
        if (lr[j] != -INFINITY) {  // a row that holds a partial
          const float w = exp2f((lr[j] - M) * kLog2e);
          den += w;
          acc.x += w * vr[j].x;
          acc.y += w * vr[j].y;
          acc.z += w * vr[j].z;
          acc.w += w * vr[j].w;
        }
      }
    }
  } else {
  // the first 256 rows' lse, kept for the listing below
  const float lse0 = t < n ? lse[t] : -INFINITY;
  float mx = lse0;
  bool any = lse0 != -INFINITY;
  for (int c = t + 256; c < n; c += 256) {
    const float lc = lse[c];
    mx = fmaxf(mx, lc);
    any = any || lc != -INFINITY;
  }
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  const bool wave_any = __ballot(any) != 0;
  if (lane == 0) {
    red[wave] = mx;
    any_s[wave] = wave_any;
  }
  __syncthreads();
  M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  empty = (any_s[0] | any_s[1] | any_s[2] | any_s[3]) == 0;

  if (!empty) {
    for (int base = 0; base < n; base += 256) {
      const int c = base + t;
      const float lc = base == 0 ? lse0 : (c < n ? lse[c] : -INFINITY);
      const bool used = lc != -INFINITY;
      const uint64_t bal = __ballot(used);
      const int before = __popcll(bal & ((1ull << lane) - 1ull));
      if (lane == 0) cnt_s[wave] = __popcll(bal);
      __syncthreads();
      int pos = before, listed = 0;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        pos += w < wave ? cnt_s[w] : 0;
        listed += cnt_s[w];
      }
      if (used) {
        idx_s[pos] = c;
        w_s[pos] = exp2f((lc - M) * kLog2e);
      }
      __syncthreads();
#pragma unroll 4
      for (int k = sg; k < listed; k += kP) {
        const float w = w_s[k];
        const float4 v = op[static_cast<int64_t>(idx_s[k]) * kC + ch];
        den += w;
        acc.x += w * v.x;
        acc.y += w * v.y;
        acc.z += w * v.z;
        acc.w += w * v.w;
      }
      __syncthreads();  // the list is read before the next round writes it
    }
  }
  }
  acc_s[sg][ch] = acc;
  if (ch == 0) den_s[sg] = den;
  __syncthreads();

  float D = 0.0f;
#pragma unroll
  for (int g = 0; g < kP; ++g) D += den_s[g];
  for (int d = t; d < DV; d += 256) {
    float x = 0.0f;
#pragma unroll
    for (int g = 0; g < kP; ++g) x += reinterpret_cast<const float*>(acc_s[g])[d];
    x /= D;
    if (aborted || n == 0 || empty) x = 0.0f;
    if (overflow && !aborted) x = NAN;
    out[bh * DV + d] = pkv::f32_to_bf16_rne(x);
  }
  if (lse_out && t == 0) {
    float l = M + __log2f(D) * kLn2;
    if (aborted || n == 0 || empty) l = -INFINITY;
    if (overflow && !aborted) l = NAN;
    lse_out[bh] = l;
  }
}

template <int DV>
int launch(const float* o_part, const float* lse_part, const int32_t* seq_lens, int batch,
           int heads, int split_tokens, int max_splits, int max_seq_len,
           const uint8_t* abort_flags, uint16_t* out, float* lse_out, hipStream_t stream) {
  constexpr int kP = 256 / (DV / 4);
  if (max_splits <= kP * kDirectRows)
    combine_kernel<DV, true><<<dim3(heads, batch), 256, 0, stream>>>(
        o_part, lse_part, seq_lens, heads, split_tokens, max_splits, max_seq_len, abort_flags, out,
        lse_out);
  else
    combine_kernel<DV, false><<<dim3(heads, batch), 256, 0, stream>>>(
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
      return launch<64>(o_part, lse_part, seq_lens, batch, num_q_heads, split_tokens, max_splits,
                       max_seq_len, abort_flags, o, lse_out, stream);
    case 128:
      return launch<128>(o_part, lse_part, seq_lens, batch, num_q_heads, split_tokens, max_splits,
                       max_seq_len, abort_flags, o, lse_out, stream);
    case 256:
      return launch<256>(o_part, lse_part, seq_lens, batch, num_q_heads, split_tokens, max_splits,
                       max_seq_len, abort_flags, o, lse_out, stream);
    case 512:
      return launch<512>(o_part, lse_part, seq_lens, batch, num_q_heads, split_tokens, max_splits,
                       max_seq_len, abort_flags, o, lse_out, stream);
    default:
      return PKV_EUNSUPPORTED;
  }
}
