// pkv_combine: log-sum-exp merge of split-KV partials into the bf16 output.
//
// Not a step of the pages: splitting a long context into chunks and merging
// the chunk results (o_c, lse_c) by
//   M = max_c lse_c, w_c = exp(lse_c - M), o = sum w_c o_c / sum w_c
// is a reordering of the same softmax sum. exp runs as exp2 with log2(e)
// folded in.
//
// The step form (kStep, after the decode kernel's step form) also finishes
// what that launch could not ("Smaller, faster, safer", section "Protecting
// a shared KV cache": a request whose mapping fails the check is aborted and
// writes nothing): it ORs the request's per-split verdicts into its abort
// flag (a request with no units, its length past max_seq_len, is checked
// here in full), and appends the new token of every request that stands, as
// the append would have before the decode. Without recorded tags (no check)
// every request stands.
#include "common.h"
#include "step.h"

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// The step form's own work in a merge workgroup, after the request's verdict
// is known: the flag (workgroup `first`, thread 0) and, when the request
// stands, the append of its new token by threads ch < 16 of the first query
// head of each kv head (K chunks, then V), the row of position L - 1 of the
// block-table page pid, encoded as the append encodes it. A position past
// the block-table row, or a page outside the pool (both possible only
// without the check), appends nothing, as the append does not.
__device__ __forceinline__ void step_epilogue(const StepCombineArgs& sa, int b, int h, int ch,
                                              bool first, bool appender, bool aborted, int32_t L,
                                              int32_t pid, const uint4& nw0, const uint4& nw1) {
  if (first && threadIdx.x == 0) sa.abort_out[b] = aborted ? 1 : 0;
  if (!appender || aborted || (L - 1) / sa.page_size >= sa.max_pages || pid < 0 ||
      pid >= sa.num_pages)
    return;
  const int g = h / sa.group;
  const int64_t row =
      (static_cast<int64_t>(pid) * sa.kv_heads + g) * sa.page_size + (L - 1) % sa.page_size;
  const int64_t dst = row * sa.head_dim + 16 * (ch & 7);
  uint8_t* pool = ch < 8 ? sa.k_pool : sa.v_pool;
  if (sa.e4m3) {
    *reinterpret_cast<uint4*>(pool + dst) =
        pkv::encode16(nw0, nw1, (ch < 8 ? sa.k_scale : sa.v_scale)[g]);
  } else {
    uint4* d = reinterpret_cast<uint4*>(pool + 2 * dst);
    d[0] = nw0;
    d[1] = nw1;
  }
}

// More split rows than the register-held merges below take, or rows that
// may be empty (the latent kernel leaves most rows of a head empty: a run of
// splits it decoded together writes its partial in its first split's row):
// the merge lists the rows that hold a partial before reading any. One
// workgroup of 256 threads per (request, query head) reduces the maximum lse
// over the rows, then, 256 rows at a time, lists (in LDS, in split order)
// the rows whose lse is not -inf, with their weights; the threads form P =
// 256 / (Dv / 4) groups and group sg merges listed rows sg, sg + P, ...,
// each thread owning one 16-byte chunk of the head. The P partial sums meet
// in LDS. The order of every sum is fixed, so the result is the same bits on
// every run.
template <int DV, bool kStep>
__global__ void __launch_bounds__(256) combine_list_kernel(const float* __restrict__ o_part,
                                                           const float* __restrict__ lse_part,
                                                           const int32_t* __restrict__ seq_lens,
                                                           int heads, int split_tokens,
                                                           int max_splits, int max_seq_len,
                                                           const uint8_t* __restrict__ abort_flags,
                                                           uint16_t* __restrict__ out,
                                                           float* __restrict__ lse_out,
                                                           StepCombineArgs sa) {
  constexpr int kC = DV / 4;    // 16-byte chunks per split row
  constexpr int kP = 256 / kC;  // split rows merged side by side
  const int b = blockIdx.y;
  const int h = blockIdx.x;
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int sg = t / kC, ch = t % kC;
  const int64_t bh = static_cast<int64_t>(b) * heads + h;
  const int32_t L = seq_lens[b];
  // step form: the request's flag is the OR of its units' verdicts, known
  // after the first barrier
  bool aborted = !kStep && abort_flags && abort_flags[b];
  const bool overflow = L > max_seq_len;
  const int n = (overflow || aborted || L <= 0) ? 0 : (L + split_tokens - 1) / split_tokens;
  const float* lse = lse_part + bh * max_splits;
  const float4* op = reinterpret_cast<const float4*>(o_part + bh * max_splits * DV);
  const bool appender = kStep && t < 16 && h % sa.group == 0 && L >= 1;
  uint4 nw0 = make_uint4(0u, 0u, 0u, 0u), nw1 = nw0;
  int32_t pid = 0;
  bool ubad = false;
  if constexpr (kStep) {
    const int j = min(max(L - 1, 0) / sa.page_size, sa.max_pages - 1);
    pid = sa.block_table[static_cast<int64_t>(b) * sa.max_pages + j];
    if (appender) {
      const uint16_t* src = (t < 8 ? sa.k_new : sa.v_new) +
                            (static_cast<int64_t>(b) * sa.kv_heads + h / sa.group) * sa.head_dim +
                            16 * (t & 7);
      nw0 = *reinterpret_cast<const uint4*>(src);
      nw1 = *reinterpret_cast<const uint4*>(src + 8);
    }
    if (sa.expected_tags)
      for (int c = t; c < n; c += 256)
        ubad = ubad || sa.unit_flags[static_cast<int64_t>(b) * max_splits + c] != 0;
  }

  __shared__ float red[4];
  __shared__ int any_s[4];
  __shared__ int bad_s[4];
  __shared__ int cnt_s[4];
  __shared__ int idx_s[256];
  __shared__ float w_s[256];
  __shared__ float den_s[kP];
  __shared__ float4 acc_s[kP][kC];

  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  float den = 0.0f;
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
  const bool wave_bad = __ballot(ubad) != 0;
  if (lane == 0) {
    red[wave] = mx;
    any_s[wave] = wave_any;
    bad_s[wave] = wave_bad;
  }
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  // empty: no row holds a partial (a NaN lse is a partial: it makes the
  // output NaN, which fmaxf alone would hide)
  const bool empty = (any_s[0] | any_s[1] | any_s[2] | any_s[3]) == 0;
  if constexpr (kStep) {
    aborted = (bad_s[0] | bad_s[1] | bad_s[2] | bad_s[3]) != 0;
    // a request with no units (length past max_seq_len) is checked here in
    // full, by every workgroup of the request (the same verdict in each)
    if (overflow && sa.expected_tags)
      aborted = pkv::check_request(sa.page_tags, sa.num_pages, sa.page_size, sa.block_table,
                                   sa.expected_tags, seq_lens, sa.max_pages, b) != 0;
    step_epilogue(sa, b, h, t, h == 0, appender, aborted, L, pid, nw0, nw1);
  }
  if (!empty && !aborted) {
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

// The latent merge at head dim 512: rows mostly empty (a run of splits the
// latent kernel decoded together writes its partial in its first split's
// row), so the rows that hold a partial are listed before any is read. A
// 256-thread workgroup takes HW = 256 / (Dv / 4) heads (2 at 512), the
// Dv / 4 threads of a head one 16-byte chunk each. A thread loads the lse of
// rows ch, ch + Dv / 4, ... of its head at once, beside the request's length
// (rows past max_splits read the last row again; rows past the length are
// dropped after), so the lse and the length cost one memory latency; the
// head's maximum and its list of rows holding a partial (in split order)
// come from wave votes and LDS, and every thread then reads its chunk of the
// listed rows. The order of every sum is fixed, so the result is the same
// bits on every run.
template <int DV, int kL>
__global__ void __launch_bounds__(256) combine_sparse_kernel(const float* __restrict__ o_part,
                                                             const float* __restrict__ lse_part,
                                                             const int32_t* __restrict__ seq_lens,
                                                             int heads, int split_tokens,
                                                             int max_splits, int max_seq_len,
                                                             const uint8_t* __restrict__ abort_flags,
                                                             uint16_t* __restrict__ out,
                                                             float* __restrict__ lse_out) {
  constexpr int kC = DV / 4;    // threads per head
  constexpr int HW = 256 / kC;  // heads per workgroup
  constexpr int kWavesPerHead = kC / 64;
  static_assert(kC % 64 == 0 && kC <= 256, "a head's chunks fill whole waves");
  const int b = blockIdx.y;
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int hh = t / kC, ch = t % kC;
  const int hw = wave % kWavesPerHead;  // the wave's place within its head
  const int h = blockIdx.x * HW + hh;
  const bool head_ok = h < heads;
  const int64_t bh = static_cast<int64_t>(b) * heads + (head_ok ? h : 0);
  const float* lse = lse_part + bh * max_splits;
  const float4* op = reinterpret_cast<const float4*>(o_part + bh * max_splits * DV);

  // the lse of rows ch + kC j (kL of them cover max_splits), then the length
  float lr[kL];
#pragma unroll
  for (int j = 0; j < kL; ++j) lr[j] = lse[min(ch + kC * j, max_splits - 1)];
  const int32_t L = seq_lens[b];
  int abf = 0;
  if (abort_flags) abf = abort_flags[b];
#pragma unroll
  for (int j = 0; j < kL; ++j) asm volatile("" : : "v"(lr[j]));
  asm volatile("" : : "v"(abf));
  const bool aborted = abf != 0;
  const bool overflow = L > max_seq_len;
  const int n = (overflow || aborted || L <= 0) ? 0 : (L + split_tokens - 1) / split_tokens;

  __shared__ float red_s[HW][kWavesPerHead];
  __shared__ int any_s[HW][kWavesPerHead];
  __shared__ int cnt_s[HW][kWavesPerHead][kL];
  __shared__ int idx_s[HW][kL * kC];
  float mx = -INFINITY;
  bool any = false;
#pragma unroll
  for (int j = 0; j < kL; ++j) {
    if (ch + kC * j >= n) lr[j] = -INFINITY;
    mx = fmaxf(mx, lr[j]);
    any = any || lr[j] != -INFINITY;
  }
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  const bool wave_any = __ballot(any) != 0;
  // per row block j: this wave's rows holding a partial, in lane order
  uint64_t bal[kL];
#pragma unroll
  for (int j = 0; j < kL; ++j) bal[j] = __ballot(lr[j] != -INFINITY);
  if (lane == 0) {
    red_s[hh][hw] = mx;
    any_s[hh][hw] = wave_any;
#pragma unroll
    for (int j = 0; j < kL; ++j) cnt_s[hh][hw][j] = __popcll(bal[j]);
  }
  __syncthreads();
  float M = -INFINITY;
  bool hany = false;
#pragma unroll
  for (int w = 0; w < kWavesPerHead; ++w) {
    M = fmaxf(M, red_s[hh][w]);
    hany = hany || any_s[hh][w];
  }
  // list position of row ch + kC j: rows of earlier blocks, then of earlier
  // waves in this block, then of earlier lanes in this wave
  int listed = 0;
#pragma unroll
  for (int j = 0; j < kL; ++j) {
    int pos = listed;
#pragma unroll
    for (int w = 0; w < kWavesPerHead; ++w) pos += w < hw ? cnt_s[hh][w][j] : 0;
    pos += __popcll(bal[j] & ((1ull << lane) - 1ull));
    if (lr[j] != -INFINITY) idx_s[hh][pos] = ch + kC * j;
#pragma unroll
    for (int w = 0; w < kWavesPerHead; ++w) listed += cnt_s[hh][w][j];
  }
  __syncthreads();
  float den = 0.0f;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  if (hany) {
    for (int k = 0; k < listed; ++k) {
      const int c = idx_s[hh][k];
      const float w = exp2f((lse[c] - M) * kLog2e);
      const float4 v = op[static_cast<int64_t>(c) * kC + ch];
      den += w;
      acc.x += w * v.x;
      acc.y += w * v.y;
      acc.z += w * v.z;
      acc.w += w * v.w;
    }
  }
  if (!head_ok) return;
  const bool zero = aborted || n == 0 || !hany;
  const bool nan = overflow && !aborted;
  float x[4] = {acc.x / den, acc.y / den, acc.z / den, acc.w / den};
  uint32_t packed[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    float a0 = x[2 * k], a1 = x[2 * k + 1];
    if (zero) a0 = a1 = 0.0f;
    if (nan) a0 = a1 = NAN;
    packed[k] = static_cast<uint32_t>(pkv::f32_to_bf16_rne(a0)) |
                (static_cast<uint32_t>(pkv::f32_to_bf16_rne(a1)) << 16);
  }
  *reinterpret_cast<uint2*>(out + bh * DV + 4 * ch) = make_uint2(packed[0], packed[1]);
  if (lse_out && ch == 0) {
    float l = M + __log2f(den) * kLn2;
    if (zero) l = -INFINITY;
    if (nan) l = NAN;
    lse_out[bh] = l;
  }
}

// Up to P kR split rows per head, every one holding a partial (the
// grouped-query kernels write one per split), so nothing needs listing: one
// 256-thread workgroup per (request, query head), the threads in P = 256 /
// (Dv / 4) groups of one 16-byte chunk each; group sg takes rows sg, sg + P,
// ..., every load issued before any is waited for (one memory latency after
// the request's length), and sums them against its own maximum. The P groups
// meet in LDS in group order, each group's sums scaled to the common maximum.
// The order of every sum is fixed, so the result is the same bits on every
// run.
template <int DV, int kR, bool kStep>
__global__ void __launch_bounds__(256) combine_groups_kernel(const float* __restrict__ o_part,
                                                             const float* __restrict__ lse_part,
                                                             const int32_t* __restrict__ seq_lens,
                                                             int heads, int split_tokens,
                                                             int max_splits, int max_seq_len,
                                                             const uint8_t* __restrict__ abort_flags,
                                                             uint16_t* __restrict__ out,
                                                             float* __restrict__ lse_out,
                                                             StepCombineArgs sa) {
  constexpr int kC = DV / 4;    // 16-byte chunks per split row
  constexpr int kP = 256 / kC;  // row groups
  static_assert(kP >= 4, "the groups' meeting below takes at most 64 threads per chunk");
  const int b = blockIdx.y;
  const int h = blockIdx.x;
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int sg = t / kC, ch = t % kC;
  const int64_t bh = static_cast<int64_t>(b) * heads + h;
  const float* lse = lse_part + bh * max_splits;
  const float4* op = reinterpret_cast<const float4*>(o_part + bh * max_splits * DV);
  const int32_t L = seq_lens[b];
  const bool overflow = L > max_seq_len;
  // rows the length covers (a request the flags abort is dropped at the end)
  const int n = (overflow || L <= 0) ? 0 : min((L + split_tokens - 1) / split_tokens, max_splits);

  // step form: the new token's chunk (threads 0 .. 15 of the first query
  // head of each kv head), the page of the last position, and the verdicts
  // of the first 256 splits (thread t reads split t's; rows past the length
  // read the last row's and are dropped)
  const bool appender = kStep && t < 16 && h % sa.group == 0 && L >= 1;
  uint4 nw0 = make_uint4(0u, 0u, 0u, 0u), nw1 = nw0;
  int32_t pid = 0;
  uint32_t uflag = 0;
  if constexpr (kStep) {
    const int j = min(max(L - 1, 0) / sa.page_size, sa.max_pages - 1);
    pid = sa.block_table[static_cast<int64_t>(b) * sa.max_pages + j];
    if (appender) {
      const uint16_t* src = (t < 8 ? sa.k_new : sa.v_new) +
                            (static_cast<int64_t>(b) * sa.kv_heads + h / sa.group) * sa.head_dim +
                            16 * (t & 7);
      nw0 = *reinterpret_cast<const uint4*>(src);
      nw1 = *reinterpret_cast<const uint4*>(src + 8);
    }
    uflag = sa.unit_flags[static_cast<int64_t>(b) * max_splits + min(t, max(n, 1) - 1)];
  }
  int abf = 0;  // the abort flag, loaded behind the rows

  float m = -INFINITY, den = 0.0f;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  bool any = false;
  // the rows: every load issued before any is waited for, the rows a group
  // takes bounded by a workgroup-uniform count (a uniform branch per row; a
  // row past the length reads the last row again and is dropped)
  if (n > 0) {
    float lr[kR];
    float4 vr[kR];
    const int jn = min(kR, (n + kP - 1) / kP);
#pragma unroll
    for (int j = 0; j < kR; ++j) {
      lr[j] = -INFINITY;
      vr[j] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
#pragma unroll
    for (int j = 0; j < kR; ++j) {
      if (j < jn) {
        const int c = min(sg + kP * j, n - 1);
        lr[j] = lse[c];
        vr[j] = op[static_cast<int64_t>(c) * kC + ch];
      }
    }
    if (!kStep && abort_flags) abf = abort_flags[b];
#pragma unroll
    for (int j = 0; j < kR; ++j)
      asm volatile("" : : "v"(lr[j]), "v"(vr[j].x), "v"(vr[j].y), "v"(vr[j].z), "v"(vr[j].w));
#pragma unroll
    for (int j = 0; j < kR; ++j) {
      if (sg + kP * j >= n) lr[j] = -INFINITY;
      m = fmaxf(m, lr[j]);
      any = any || lr[j] != -INFINITY;
    }
#pragma unroll
    for (int j = 0; j < kR; ++j) {
      if (lr[j] != -INFINITY) {
        const float w = exp2f((lr[j] - m) * kLog2e);
        den += w;
        acc.x += w * vr[j].x;
        acc.y += w * vr[j].y;
        acc.z += w * vr[j].z;
        acc.w += w * vr[j].w;
      }
    }
  }
  bool ubad = kStep && sa.expected_tags && t < n && uflag != 0;
  if constexpr (kStep)
    if (sa.expected_tags)
      for (int c = t + 256; c < n; c += 256)
        ubad = ubad || sa.unit_flags[static_cast<int64_t>(b) * max_splits + c] != 0;

  __shared__ float m_s[kP];
  __shared__ float den_s[kP];
  __shared__ float4 acc_s[kP][kC];
  __shared__ int any_s[4];
  __shared__ int bad_s[4];
  acc_s[sg][ch] = acc;
  if (ch == 0) {
    m_s[sg] = m;
    den_s[sg] = den;
  }
  const bool wave_any = __ballot(any) != 0;
  const bool wave_bad = __ballot(ubad) != 0;
  if (lane == 0) {
    any_s[wave] = wave_any;
    bad_s[wave] = wave_bad;
  }
  __syncthreads();
  const bool empty = (any_s[0] | any_s[1] | any_s[2] | any_s[3]) == 0;
  bool aborted = abf != 0;
  if constexpr (kStep) {
    aborted = (bad_s[0] | bad_s[1] | bad_s[2] | bad_s[3]) != 0;
    // a request with no units (length past max_seq_len) is checked here in
    // full, by every workgroup of the request (the same verdict in each)
    if (overflow && sa.expected_tags)
      aborted = pkv::check_request(sa.page_tags, sa.num_pages, sa.page_size, sa.block_table,
                                   sa.expected_tags, seq_lens, sa.max_pages, b) != 0;
    step_epilogue(sa, b, h, t, h == 0, appender, aborted, L, pid, nw0, nw1);
  }
  // the groups meet: M over their maxima, each group's sums scaled to it
  float M = -INFINITY;
#pragma unroll
  for (int g = 0; g < kP; ++g) M = fmaxf(M, m_s[g]);
  float D = 0.0f;
  float fg[kP];
#pragma unroll
  for (int g = 0; g < kP; ++g) {
    fg[g] = m_s[g] == -INFINITY ? 0.0f : exp2f((m_s[g] - M) * kLog2e);
    D += den_s[g] * fg[g];
  }
  const bool zero = aborted || n == 0 || empty;
  const bool nan = overflow && !aborted;
  for (int d = t; d < DV; d += 256) {
    float x = 0.0f;
#pragma unroll
    for (int g = 0; g < kP; ++g) x += reinterpret_cast<const float*>(acc_s[g])[d] * fg[g];
    x /= D;
    if (zero) x = 0.0f;
    if (nan) x = NAN;
    out[bh * DV + d] = pkv::f32_to_bf16_rne(x);
  }
  if (lse_out && t == 0) {
    float l = M + __log2f(D) * kLn2;
    if (zero) l = -INFINITY;
    if (nan) l = NAN;
    lse_out[bh] = l;
  }
}

// When every split row of a request fits in registers (max_splits <= kMax):
// a workgroup takes HW = 256 / (Dv / 4) consecutive query heads of one
// request, thread (head hh, chunk ch) loads the lse values of its head's
// rows and its 16-byte chunk of each row at once, and merges them in split
// order by itself: no LDS and no barrier, one memory latency after the
// request's length. Every
// thread of a head sums the same rows in the same order, so the result is
// the same bits on every run. The step form's flags are per request: each
// wave ORs them with one vote.
template <int DV, int kMax, bool kStep>
__global__ void __launch_bounds__(256) combine_rows_kernel(const float* __restrict__ o_part,
                                                           const float* __restrict__ lse_part,
                                                           const int32_t* __restrict__ seq_lens,
                                                           int heads, int split_tokens,
                                                           int max_splits, int max_seq_len,
                                                           const uint8_t* __restrict__ abort_flags,
                                                           uint16_t* __restrict__ out,
                                                           float* __restrict__ lse_out,
                                                           StepCombineArgs sa) {
  constexpr int kC = DV / 4;    // 16-byte chunks per split row (threads per head)
  constexpr int HW = 256 / kC;  // heads per workgroup
  static_assert(kC <= 256 && 256 % kC == 0, "a head's chunks tile the workgroup");
  const int b = blockIdx.y;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int hh = t / kC, ch = t % kC;
  const int h = blockIdx.x * HW + hh;
  const bool head_ok = h < heads;
  const int64_t bh = static_cast<int64_t>(b) * heads + (head_ok ? h : 0);
  const float* lse = lse_part + bh * max_splits;
  const float4* op = reinterpret_cast<const float4*>(o_part + bh * max_splits * DV);

  // The length first (a scalar load), then every vector load is issued
  // before any is waited for, in one memory latency: the rows the length
  // covers (a uniform branch per row; the others are never read), the flags,
  // the new token and the page of the last position. The empty asm
  // statements below then take the values.
  const int32_t L = seq_lens[b];
  const int nl = (L > max_seq_len || L <= 0) ? 0 : min((L + split_tokens - 1) / split_tokens,
                                                        max_splits);
  float lr[kMax];
  float4 vr[kMax];
#pragma unroll
  for (int c = 0; c < kMax; ++c) {
    lr[c] = -INFINITY;
    vr[c] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  }
#pragma unroll
  for (int c = 0; c < kMax; ++c) {
    if (c < nl) {
      lr[c] = lse[c];
      vr[c] = op[static_cast<int64_t>(c) * kC + ch];
    }
  }
  int abf = 0;
  if (!kStep && abort_flags) abf = abort_flags[b];
  // step form: the units' verdicts (lane c of each wave reads split c's),
  // the new token's chunk (threads ch < 16 of the first query head of each
  // kv head: K chunks, then V) and the page of the last position
  const bool appender = kStep && head_ok && ch < 16 && h % sa.group == 0 && L >= 1;
  uint4 nw0 = make_uint4(0u, 0u, 0u, 0u), nw1 = nw0;
  uint32_t uflag = 0;
  int32_t pid = 0;
  if constexpr (kStep) {
    const int j = min(max(L - 1, 0) / sa.page_size, sa.max_pages - 1);
    pid = sa.block_table[static_cast<int64_t>(b) * sa.max_pages + j];
    uflag = sa.unit_flags[static_cast<int64_t>(b) * max_splits + min(lane, max_splits - 1)];
    if (appender) {
      const uint16_t* src = (ch < 8 ? sa.k_new : sa.v_new) +
                            (static_cast<int64_t>(b) * sa.kv_heads + h / sa.group) * sa.head_dim +
                            16 * (ch & 7);
      nw0 = *reinterpret_cast<const uint4*>(src);
      nw1 = *reinterpret_cast<const uint4*>(src + 8);
    }
  }
#pragma unroll
  for (int c = 0; c < kMax; ++c)
    asm volatile("" : : "v"(lr[c]), "v"(vr[c].x), "v"(vr[c].y), "v"(vr[c].z), "v"(vr[c].w));
  asm volatile("" : : "v"(abf), "v"(uflag), "v"(pid));
  asm volatile("" : : "v"(nw0.x), "v"(nw0.y), "v"(nw0.z), "v"(nw0.w));
  asm volatile("" : : "v"(nw1.x), "v"(nw1.y), "v"(nw1.z), "v"(nw1.w));

  bool aborted = abf != 0;
  const bool overflow = L > max_seq_len;
  const int n = (overflow || aborted || L <= 0) ? 0 : (L + split_tokens - 1) / split_tokens;
  if constexpr (kStep) {
    aborted = sa.expected_tags != nullptr && __any(uflag != 0 && lane < n);
    // a request with no units (length past max_seq_len) is checked here in
    // full, by every workgroup of the request (the same verdict in each)
    if (overflow && sa.expected_tags)
      aborted = pkv::check_request(sa.page_tags, sa.num_pages, sa.page_size, sa.block_table,
                                   sa.expected_tags, seq_lens, sa.max_pages, b) != 0;
    step_epilogue(sa, b, h, ch, blockIdx.x == 0, appender, aborted, L, pid, nw0, nw1);
  }

  // M = max lse over the rows that hold tokens; empty: no row holds a
  // partial (a NaN lse is a partial: it makes the output NaN)
  float M = -INFINITY;
  bool any = false;
#pragma unroll
  for (int c = 0; c < kMax; ++c) {
    if (c >= n) lr[c] = -INFINITY;
    M = fmaxf(M, lr[c]);
    any = any || lr[c] != -INFINITY;
  }
  float den = 0.0f;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  if (any && !aborted) {
#pragma unroll
    for (int c = 0; c < kMax; ++c) {
      if (lr[c] != -INFINITY) {
        const float w = exp2f((lr[c] - M) * kLog2e);
        den += w;
        acc.x += w * vr[c].x;
        acc.y += w * vr[c].y;
        acc.z += w * vr[c].z;
        acc.w += w * vr[c].w;
      }
    }
  }
  if (!head_ok) return;
  const bool zero = aborted || n == 0 || !any;
  const bool nan = overflow && !aborted;
  float x[4] = {acc.x / den, acc.y / den, acc.z / den, acc.w / den};
  uint32_t packed[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    float a0 = x[2 * k], a1 = x[2 * k + 1];
    if (zero) a0 = a1 = 0.0f;
    if (nan) a0 = a1 = NAN;
    packed[k] = static_cast<uint32_t>(pkv::f32_to_bf16_rne(a0)) |
                (static_cast<uint32_t>(pkv::f32_to_bf16_rne(a1)) << 16);
  }
  *reinterpret_cast<uint2*>(out + bh * DV + 4 * ch) = make_uint2(packed[0], packed[1]);
  if (lse_out && ch == 0) {
    float l = M + __log2f(den) * kLn2;
    if (zero) l = -INFINITY;
    if (nan) l = NAN;
    lse_out[bh] = l;
  }
}

// The merge kernels for head dim DV; kStep: the step form (head dim 128).
template <int DV, bool kStep>
int launch_form(const float* o_part, const float* lse_part, const int32_t* seq_lens, int batch,
                int heads, int split_tokens, int max_splits, int max_seq_len,
                const uint8_t* abort_flags, uint16_t* out, float* lse_out,
                const StepCombineArgs& a, hipStream_t stream) {
  constexpr int kP = 256 / (DV / 4);
  constexpr int kR = 24;  // rows per thread of the row-group merge
  const dim3 grid(heads, batch);
  // every row in registers: one workgroup per kP heads (up to 32 rows below
  // head dim 512, 16 at 512; the output written 8 bytes at a time)
  const dim3 rgrid((heads + kP - 1) / kP, batch);
  const bool out8 = (reinterpret_cast<uintptr_t>(out) & 7u) == 0;
  if (out8 && max_splits <= 16) {
    combine_rows_kernel<DV, 16, kStep><<<rgrid, 256, 0, stream>>>(
        o_part, lse_part, seq_lens, heads, split_tokens, max_splits, max_seq_len, abort_flags,
        out, lse_out, a);
  } else if constexpr (DV <= 256) {
    if (out8 && max_splits <= 32)
      combine_rows_kernel<DV, 32, kStep><<<rgrid, 256, 0, stream>>>(
          o_part, lse_part, seq_lens, heads, split_tokens, max_splits, max_seq_len, abort_flags,
          out, lse_out, a);
    else if (max_splits <= kP * kR)
      combine_groups_kernel<DV, kR, kStep><<<grid, 256, 0, stream>>>(
          o_part, lse_part, seq_lens, heads, split_tokens, max_splits, max_seq_len, abort_flags,
          out, lse_out, a);
    else
      combine_list_kernel<DV, kStep><<<grid, 256, 0, stream>>>(
          o_part, lse_part, seq_lens, heads, split_tokens, max_splits, max_seq_len, abort_flags,
          out, lse_out, a);
  } else if (!kStep && out8 && max_splits <= 2 * (DV / 4)) {
    // the latent merge: two heads per workgroup, rows listed per head
    combine_sparse_kernel<DV, 2><<<rgrid, 256, 0, stream>>>(
        o_part, lse_part, seq_lens, heads, split_tokens, max_splits, max_seq_len, abort_flags,
        out, lse_out);
  } else {
    combine_list_kernel<DV, kStep><<<grid, 256, 0, stream>>>(
        o_part, lse_part, seq_lens, heads, split_tokens, max_splits, max_seq_len, abort_flags,
        out, lse_out, a);
  }
  return pkv::launch_status();
}

template <int DV>
int launch(const float* o_part, const float* lse_part, const int32_t* seq_lens, int batch,
           int heads, int split_tokens, int max_splits, int max_seq_len,
           const uint8_t* abort_flags, uint16_t* out, float* lse_out, const StepCombineArgs* sa,
           hipStream_t stream) {
  if (sa) {
    if constexpr (DV == 128)
      return launch_form<DV, true>(o_part, lse_part, seq_lens, batch, heads, split_tokens,
                                   max_splits, max_seq_len, nullptr, out, lse_out, *sa, stream);
    return PKV_EUNSUPPORTED;
  }
  return launch_form<DV, false>(o_part, lse_part, seq_lens, batch, heads, split_tokens,
                                max_splits, max_seq_len, abort_flags, out, lse_out,
                                StepCombineArgs{}, stream);
}

}  // namespace

int combine_impl(const float* o_part, const float* lse_part, const int32_t* seq_lens,
                 int32_t batch, int32_t num_q_heads, int32_t head_dim_v, int32_t split_tokens,
                 int32_t max_splits, int32_t max_seq_len, const uint8_t* abort_flags, void* out,
                 float* lse_out, const StepCombineArgs* sa, hipStream_t stream) {
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
                        max_seq_len, abort_flags, o, lse_out, sa, stream);
    case 128:
      return launch<128>(o_part, lse_part, seq_lens, batch, num_q_heads, split_tokens,
                         max_splits, max_seq_len, abort_flags, o, lse_out, sa, stream);
    case 256:
      return launch<256>(o_part, lse_part, seq_lens, batch, num_q_heads, split_tokens,
                         max_splits, max_seq_len, abort_flags, o, lse_out, sa, stream);
    case 512:
      return launch<512>(o_part, lse_part, seq_lens, batch, num_q_heads, split_tokens,
                         max_splits, max_seq_len, abort_flags, o, lse_out, sa, stream);
    default:
      return PKV_EUNSUPPORTED;
  }
}

extern "C" int pkv_combine(const float* o_part, const float* lse_part, const int32_t* seq_lens,
                           int32_t batch, int32_t num_q_heads, int32_t head_dim_v,
                           int32_t split_tokens, int32_t max_splits, int32_t max_seq_len,
                           const uint8_t* abort_flags, void* out, float* lse_out,
                           hipStream_t stream) {
  return combine_impl(o_part, lse_part, seq_lens, batch, num_q_heads, head_dim_v, split_tokens,
                      max_splits, max_seq_len, abort_flags, out, lse_out, nullptr, stream);
}
