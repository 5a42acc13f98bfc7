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

// Work unit u of the one-dimensional launch -> (request b, kv head g,
// split c). The hardware dispatcher hands out workgroups in index order, so
// the order is chosen for it: every full split first (request, split, kv
// head), then each request's last split, longest first (request order for
// batches above 64), so the launch ends on its shortest units; then indices
// with no unit (the launch is sized for max_seq_len), which exit at once.
// Aborted requests and empty or over-long contexts have no units.
__device__ __forceinline__ bool find_unit(const DecodeParams& p, int u, int& b_out, int& g_out,
                                          int& c_out, int& L_out) {
  const int lane = threadIdx.x & 63;
  const int S = p.split_tokens, H = p.num_kv_heads;
  // request j's length and split count (0 for no units); the length and the
  // abort flag are loaded side by side, one memory latency
  auto fetch = [&](int j, int& L) __attribute__((always_inline)) {
    L = 0;
    int ab = 0;
    if (j < p.batch) {
      L = p.seq_lens[j];
      if (p.abort_flags) ab = p.abort_flags[j];
    }
    return (ab == 0 && L > 0 && L <= p.max_seq_len) ? (L + S - 1) / S : 0;
  };
  // the first 64 requests, fetched once for both passes below
  int L0;
  const int n0 = fetch(lane, L0);
  int base = 0;  // full units of the requests before this batch of 64
  for (int b0 = 0; b0 < p.batch; b0 += 64) {
    int L = L0;
    const int n = b0 == 0 ? n0 : fetch(b0 + lane, L);
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
      return true;
    }
    base += total;
  }
  int u2 = u - base;
  if (p.batch <= 64) {
    const int n = n0, L = L0;
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
    return true;
  }
  for (int b0 = 0; b0 < p.batch; b0 += 64) {
    int L = L0;
    const int n = b0 == 0 ? n0 : fetch(b0 + lane, L);
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
      return true;
    }
    u2 -= total;
  }
  return false;
}

}  // namespace pkv
