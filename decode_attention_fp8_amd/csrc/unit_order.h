// Work-unit order of the one-dimensional decode launches (internal).
#pragma once

#include "decode_params.h"

namespace pkv {

// Inclusive prefix sum over the wave.
__device__ __forceinline__ int wave_scan(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

// Sum over the wave, the same in every lane; the terms must keep the sum
// below 2^31.
__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return __builtin_amdgcn_readfirstlane(x);
}

// A request's length as it counts towards the launch's cache footprint:
// 0 without work units, at most 2^25 (the footprint is only compared with a
// threshold far below what one such request holds, and 64 capped terms
// still sum below 2^31).
__device__ __forceinline__ int footprint_len(int L) { return min(L, 1 << 25); }

// Length of request j if it has work units (not aborted, not empty, not
// over-long, j < batch), else 0.
// Both loads are issued before either value is tested, so they share one
// memory round trip.
__device__ __forceinline__ int unit_len(const DecodeParams& p, int j) {
  int L = 0, ab = 0;
  if (j < p.batch) {
    L = p.seq_lens[j];
    if (p.abort_flags) ab = p.abort_flags[j];
  }
  return (ab != 0 || L <= 0 || L > p.max_seq_len) ? 0 : L;
}

// Cache tokens the launch reads (each request capped as in footprint_len):
// the lengths of the requests that have work units, summed. Uniform.
__device__ __forceinline__ int64_t launch_tokens(const DecodeParams& p) {
  const int lane = threadIdx.x & 63;
  int64_t t = 0;
  for (int b0 = 0; b0 < p.batch; b0 += 64) t += wave_sum(footprint_len(unit_len(p, b0 + lane)));
  return t;
}

// Work unit u of the one-dimensional launch -> (request b, kv head g,
// split c). The hardware dispatcher hands out workgroups in index order, so
// the order is chosen for it: every full split first (request, split, kv
// head), then each request's last split, longest first (request order for
// batches above 64), so the launch ends on its shortest units; then indices
// with no unit (the launch is sized for max_seq_len), which exit at once.
// Aborted requests and empty or over-long contexts have no units.
//
// len_out receives footprint_len of lane's request (lanes 0..63 cover the
// first 64 requests), so that up to 64 requests launch_tokens(p) is
// wave_sum(len_out), without loads of its own.
__device__ __forceinline__ bool find_unit(const DecodeParams& p, int u, int& b_out, int& g_out, int& c_out,
                          int& L_out, int& len_out) {
  const int lane = threadIdx.x & 63;
  const int S = p.split_tokens, H = p.num_kv_heads;
  int L = 0;
  auto splits = [&](int j) __attribute__((always_inline)) {
    int n = 0;
    L = 0;
    if (j < p.batch) {
      L = p.seq_lens[j];
      const bool ab = p.abort_flags && p.abort_flags[j];
      if (!ab && L > 0 && L <= p.max_seq_len) n = (L + S - 1) / S;
    }
    return n;
  };
  int mine = 0;
  auto found = [&]() __attribute__((always_inline)) {
    len_out = mine;
    return true;
  };
  int base = 0;  // full units of the requests before this batch of 64
  for (int b0 = 0; b0 < p.batch; b0 += 64) {
    const int n = splits(b0 + lane);
    if (b0 == 0) mine = n > 0 ? footprint_len(L) : 0;
    const int full = n > 0 ? (n - 1) * H : 0;
    const int incl = wave_scan(full);
    const int total = __builtin_amdgcn_readlane(incl, 63);
    if (u < base + total) {
      const int bl = __popcll(__ballot(base + incl <= u));
      const int r = u - base - __builtin_amdgcn_readlane(incl - full, bl);
      b_out = b0 + bl;
      c_out = r / H;
      g_out = r - c_out * H;
      L_out = __builtin_amdgcn_readlane(L, bl);
      return found();
    }
    base += total;
  }
  int u2 = u - base;
  if (p.batch <= 64) {
    const int n = splits(lane);
    const int psz = n > 0 ? L - (n - 1) * S : -1;
    if (u2 >= __popcll(__ballot(n > 0)) * H) return false;
    int rank = 0;
    for (int k = 0; k < 64; ++k) {
      const int pk = __builtin_amdgcn_readlane(psz, k);
      rank += (pk > psz || (pk == psz && k < lane)) ? 1 : 0;
    }
    const int R = u2 / H;
    const uint64_t hit = __ballot(n > 0 && rank == R);
    const int bl = static_cast<int>(__builtin_ctzll(hit));
    b_out = bl;
    g_out = u2 - R * H;
    c_out = __builtin_amdgcn_readlane(n, bl) - 1;
    L_out = __builtin_amdgcn_readlane(L, bl);
    return found();
  }
  for (int b0 = 0; b0 < p.batch; b0 += 64) {
    const int n = splits(b0 + lane);
    const int part = n > 0 ? H : 0;
    const int incl = wave_scan(part);
    const int total = __builtin_amdgcn_readlane(incl, 63);
    if (u2 < total) {
      const int bl = __popcll(__ballot(incl <= u2));
      const int r = u2 - __builtin_amdgcn_readlane(incl - part, bl);
      b_out = b0 + bl;
      g_out = r;
      c_out = __builtin_amdgcn_readlane(n, bl) - 1;
      L_out = __builtin_amdgcn_readlane(L, bl);
      return found();
    }
    u2 -= total;
  }
  return false;
}

// Whether a launch that reads `bytes` of cache marks its cache loads
// non-temporal. A footprint that mostly fits in the 256 MB last-level cache
// (MALL) is read again from it by the next step when the loads keep their
// lines; above that, the lines would only be evicted unused, and the
// non-temporal form streams faster (random 2 KB blocks: about 6.7 against
// 6.0 TB/s). The threshold lies between the two footprints measured on the
// batch-8 and batch-16 grouped-query workloads (280 MB: plain loads 15%
// faster; 584 MB: non-temporal loads 8% faster).
constexpr int64_t kStreamAboveBytes = 384ll << 20;
__device__ __forceinline__ bool stream_cache(int64_t bytes) { return bytes > kStreamAboveBytes; }

}  // namespace pkv
