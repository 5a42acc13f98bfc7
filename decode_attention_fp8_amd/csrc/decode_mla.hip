// Wide-head decode kernel: many query heads over one latent kv head whose
// rows are 576 values, the first 512 of which are also V (the MLA-shaped
// layout), e4m3 or bf16 cache, page size 64.
//
// "Smaller, faster, safer", section "Quantizing the KV cache": the cache is
// e4m3 and the attention kernel converts values as it reads them. With 128
// query heads sharing every cached row, QK^T and PV are dense contractions
// (about 480 flop per cached byte), so they run on bf16 MFMA: e4m3 codes
// convert to bf16 exactly, q stays bf16, p is rounded to bf16, and all
// accumulation is fp32.
//
// Work unit = (request b, split c, group of 64 query heads): one workgroup
// of 4 waves, each wave owning 16 query heads (one MFMA block; q for them
// stays in 72 registers and the 16 x 512 accumulators in 128). The head
// groups of one (b, c) get block ids 8 apart, so they run on the same XCD
// and the second read of each tile hits that XCD's L2. The split is processed in tiles of 64 tokens (one
// page). Tiles travel HBM -> LDS by direct-to-LDS loads, kBufs - 1 tiles
// ahead of the one being computed; the first kIssuers waves each issue 9
// of a tile's 1 KB loads and wait for their own, then the workgroup
// barriers.
//
// Tile layout in LDS: row r (a token) holds its 16-byte chunks permuted
// within the row (chunk c at position c ^ swz(r) for the 512 value bytes)
// so that both the K fragment reads (8 consecutive rows, one chunk) and
// the transposing V reads (rows {4G..4G+3, 16+4G..16+4G+3}) hit distinct
// banks.
//
// QK^T is computed transposed, S^T = K Q^T (MFMA 16x16x32: M = 16 tokens,
// N = 16 heads, K = 32 dims); its accumulator layout then gives each lane
// the scores of one head for tokens {4G..4G+3} of every 16, which is
// exactly an A operand of PV (M = heads, K = 32 tokens) once the B operand
// (V, K = tokens, N = 16 dims) is read in the same token order. The V
// operand is read with ds_read_tr8_b64 (tr16 for bf16), which transposes an
// 8 x 16 byte block across 16 lanes: each lane receives one dim of 8
// tokens straight from the row-major tile.
//
// Softmax: as in the grouped-query kernel, log2 domain with a running max
// that only moves when a score exceeds it by kTau.
#include "common.h"
#include "decode_params.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef int v2i_t __attribute__((ext_vector_type(2)));
typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v2i_t lds_v2i_t;
typedef __attribute__((address_space(3))) v4s_t lds_v4s_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTau = 8.0f;
constexpr float kMInit = -1e30f;
constexpr int kDk = 576;
constexpr int kDv = 512;
constexpr int kTile = 64;          // tokens per tile (= page size)
constexpr int kHeadsPerWave = 16;
constexpr int kMaxUnitTiles = 512;

template <bool kE4M3>
struct Mla {
  static constexpr int kElem = kE4M3 ? 1 : 2;
  static constexpr int kRowBytes = kDk * kElem;         // 576 / 1152
  static constexpr int kRowChunks = kRowBytes / 16;     // 36 / 72
  static constexpr int kTileBytes = kTile * kRowBytes;  // 36 KB / 72 KB
  static constexpr int kTileDma = kTileBytes / 1024;    // 36 / 72 loads of 1 KB
  static constexpr int kBufs = kE4M3 ? 3 : 2;
};

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)p));
}

// 16 bytes per lane from base + voff into LDS at lds + 16 * lane (m0 is not
// otherwise used by this kernel; the immediate offset stays 0 because it
// would move both addresses). Marked non-temporal: a step reads each cache
// byte once, so its lines are not kept for reuse.
__device__ __forceinline__ void dma16(uint32_t lds, uint32_t voff, const uint8_t* base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
               :
               : "s"(lds), "v"(voff), "s"(base)
               : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// Workgroup barrier that neither waits for the loads in flight nor lets
// memory accesses move across it; LDS writes before it are complete.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
}

__device__ __forceinline__ int swz(int r) { return (r & 7) ^ (((r >> 4) & 1) << 2); }

// Position (in 16-byte chunks) of chunk c of tile row r.
template <bool kE4M3>
__device__ __forceinline__ int chunk_pos(int r, int c) {
  if constexpr (kE4M3) {
    const int cc = c < 32 ? (c ^ swz(r)) : (32 + ((c - 32) ^ (r & 3)));
    return r * 36 + cc;
  } else {
    return r * 72 + (c ^ swz(r));
  }
}

// Chunk stored at in-row position cc of row r (the inverse permutation).
template <bool kE4M3>
__device__ __forceinline__ int chunk_at(int r, int cc) {
  if constexpr (kE4M3) {
    return cc < 32 ? (cc ^ swz(r)) : (32 + ((cc - 32) ^ (r & 3)));
  } else {
    return cc ^ swz(r);
  }
}

__device__ __forceinline__ bf16x2_t cvt_lo(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
}
__device__ __forceinline__ bf16x2_t cvt_hi(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
}
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
  const bf16x2_t a = cvt_lo(w0), b = cvt_hi(w0), c = cvt_lo(w1), d = cvt_hi(w1);
  return bf16x8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}
__device__ __forceinline__ bf16x8_t as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const uint4 u = make_uint4(a, b, c, d);
  return __builtin_bit_cast(bf16x8_t, u);
}

template <bool kE4M3>
__global__ void __launch_bounds__(256) decode_mla_kernel(DecodeParams p, int n_splits,
                                                         int head_groups) {
  constexpr int W = 4;
  using M = Mla<kE4M3>;
  constexpr int kThreads = W * 64;
  constexpr int kIssuers = (W < M::kTileDma / 9) ? W : M::kTileDma / 9;
  constexpr int kMine = M::kTileDma / kIssuers;  // loads of each tile issued by an issuer
  static_assert(M::kTileDma % kIssuers == 0, "tile loads must split evenly");
  static_assert((M::kBufs - 1) * kMine <= 63, "vmcnt counts to 63");
  __shared__ __attribute__((aligned(16))) uint8_t tiles[M::kBufs * M::kTileBytes];
  __shared__ int32_t pages[kMaxUnitTiles];
  __shared__ float alpha_s[W][kHeadsPerWave];
  __shared__ float l_s[W][kHeadsPerWave];

  // blockIdx.x = (split / 8, head group, split % 8)
  const int x = blockIdx.x;
  const int hg = (x >> 3) % head_groups;
  const int c = (x / (8 * head_groups)) * 8 + (x & 7);
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  if (c >= n_splits) return;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int G = lane >> 4;
  const int lr = lane & 15;

  if (p.abort_flags && p.abort_flags[b]) return;
  const int L = p.seq_lens[b];
  if (L > p.max_seq_len) return;
  const int t_begin = c * p.split_tokens;
  if (t_begin >= L) return;
  const int t_end = min(L, t_begin + p.split_tokens);
  const int n_tiles = (t_end - t_begin + kTile - 1) / kTile;
  const int h_base = hg * (W * kHeadsPerWave) + wave * kHeadsPerWave;

  // q as B operands of S^T = K Q^T: head h_base + lr, and for k-step ks the
  // 8 dims this lane group G covers (e4m3: dims 64(ks/2) + 16G + 8(ks%2), so
  // one 16-byte K read serves two k-steps; bf16: 32ks + 8G).
  bf16x8_t qf[18];
  {
    const uint16_t* qrow = p.q + (static_cast<int64_t>(b) * p.num_q_heads + h_base + lr) * kDk;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      const int d0 = kE4M3 ? (64 * (ks >> 1) + 16 * G + 8 * (ks & 1)) : (32 * ks + 8 * G);
      qf[ks] = *reinterpret_cast<const bf16x8_t*>(qrow + d0);
    }
  }
  const float qk_scale = (kE4M3 ? p.k_scale[0] : 1.0f) * p.sm_scale_log2;
  const float o_scale = kE4M3 ? p.v_scale[0] : 1.0f;

  const int32_t* bt = p.block_table + static_cast<int64_t>(b) * p.max_pages;
  const int first_page = t_begin / kTile;
  for (int j = tid; j < n_tiles; j += kThreads) pages[j] = bt[first_page + j];
  // every compiler-issued load completes before the first tile load
#pragma unroll
  for (int ks = 0; ks < 18; ++ks) asm volatile("" : : "v"(qf[ks]));
  asm volatile("" : : "v"(qk_scale), "v"(o_scale));
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" : : : "memory");

  // per-lane sources of this wave's loads inside a tile
  uint32_t doff[kMine];
#pragma unroll
  for (int i = 0; i < kMine; ++i) {
    const int k = wave + kIssuers * i;
    const int pos = 64 * k + lane;
    const int r = pos / M::kRowChunks;
    const int cc = pos - r * M::kRowChunks;
    doff[i] = static_cast<uint32_t>(r * M::kRowBytes + chunk_at<kE4M3>(r, cc) * 16);
  }
  const uint8_t* kpool = static_cast<const uint8_t*>(p.k_pool);
  const uint32_t tiles0 = lds_addr(tiles);
  const int64_t page_bytes = static_cast<int64_t>(kTile) * M::kRowBytes;  // one kv head

  auto page_of = [&](int t) __attribute__((always_inline)) {
    return __builtin_amdgcn_readfirstlane(pages[t]);
  };
  auto issue = [&](int t) __attribute__((always_inline)) {
    int page = page_of(t);
    if (page < 0 || page >= p.num_pages) page = 0;  // loaded but never used
    const uint8_t* base = kpool + static_cast<int64_t>(page) * page_bytes;
    const uint32_t buf = tiles0 + (t % M::kBufs) * M::kTileBytes;
    if (wave < kIssuers) {
#pragma unroll
      for (int i = 0; i < kMine; ++i) dma16(buf + 1024 * (wave + kIssuers * i), doff[i], base);
    }
  };

  floatx4_t O[32];
#pragma unroll
  for (int dn = 0; dn < 32; ++dn) O[dn] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  float m = kMInit;
  float l = 0.f;

  auto compute = [&](int t, int nv) __attribute__((always_inline)) {
    const uint8_t* buf = tiles + (t % M::kBufs) * M::kTileBytes;

    // ---- S^T = K Q^T: 4 token blocks x this wave's 16 heads. The 36 (e4m3)
    // or 72 (bf16) K fragment reads run one step ahead of their MFMAs, and
    // the scheduling fences keep the compiler from hoisting all of them.
    floatx4_t st[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) st[mb] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    constexpr int kQkSteps = kE4M3 ? 36 : 72;  // (mb, 16-byte chunk) pairs
    constexpr int kPer = kQkSteps / 4;
    auto k_read = [&](int step) __attribute__((always_inline)) {
      const int mb = step / kPer, j = step % kPer;
      return *reinterpret_cast<const uint4*>(buf + chunk_pos<kE4M3>(16 * mb + lr, 4 * j + G) * 16);
    };
    uint4 raw = k_read(0);
#pragma unroll
    for (int step = 0; step < kQkSteps; ++step) {
      const int mb = step / kPer, j = step % kPer;
      const uint4 cur = raw;
      if (step + 1 < kQkSteps) raw = k_read(step + 1);
      if constexpr (kE4M3) {
        st[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16(cur.x, cur.y), qf[2 * j], st[mb], 0, 0, 0);
        st[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16(cur.z, cur.w), qf[2 * j + 1], st[mb], 0, 0, 0);
      } else {
        st[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(cur.x, cur.y, cur.z, cur.w), qf[j], st[mb], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- scores (log2 domain); token of st[mb][r] is 16mb + 4G + r, head lr
    bool over = false;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = st[mb][r] * qk_scale;
        st[mb][r] = (16 * mb + 4 * G + r < nv) ? v : -INFINITY;
        over |= st[mb][r] > m + kTau;
      }
    if (__any(over)) {  // rare: move the running max of this wave's heads
      float lm = -INFINITY;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) lm = fmaxf(lm, st[mb][r]);
      lm = fmaxf(lm, __shfl_xor(lm, 16));
      lm = fmaxf(lm, __shfl_xor(lm, 32));
      const float mn = fmaxf(m, lm);
      const float a = __builtin_amdgcn_exp2f(m - mn);
      m = mn;
      l *= a;
      if (G == 0) alpha_s[wave][lr] = a;
      __builtin_amdgcn_wave_barrier();
      floatx4_t f;
#pragma unroll
      for (int r = 0; r < 4; ++r) f[r] = alpha_s[wave][4 * G + r];
#pragma unroll
      for (int dn = 0; dn < 32; ++dn) O[dn] *= f;
      __builtin_amdgcn_wave_barrier();
    }

    // ---- P as A operands of PV: step s covers tokens 32s..32s+31 in the
    // order {4G..4G+3, 16+4G..16+4G+3} (rows of st[2s] then st[2s+1])
    bf16x8_t pf[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      __bf16 e[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float pr = __builtin_amdgcn_exp2f(st[2 * s + (k >> 2)][k & 3] - m);
        e[k] = static_cast<__bf16>(pr);
        l += static_cast<float>(e[k]);
      }
      pf[s] = bf16x8_t{e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]};
    }

    // ---- O += P V: 32 dim blocks x 2 token steps, the transposing V read
    // one step ahead of its MFMA
    const int e_row = lr >> 1;  // row of the transposed 8 x 16 block this lane addresses
    const int tok_in_step = (e_row < 4) ? (4 * G + e_row) : (16 + 4 * G + e_row - 4);
    auto v_read = [&](int step) __attribute__((always_inline)) {
      const int dn = step >> 1, s = step & 1;
      uint4 w;
      if constexpr (kE4M3) {
        const uint8_t* ad = buf + chunk_pos<true>(32 * s + tok_in_step, dn) * 16 + 8 * (lr & 1);
        const v2i_t r8 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_t*)ad);
        w = make_uint4(static_cast<uint32_t>(r8[0]), static_cast<uint32_t>(r8[1]), 0u, 0u);
      } else {
        // tr16: lanes 4e..4e+3 of a group address row e; two reads cover
        // the 8 tokens of the step
        const int e4 = lr >> 2, i4 = lr & 3;
        const int ch = 2 * dn + (i4 >> 1);
        const uint8_t* a0 = buf + chunk_pos<false>(32 * s + 4 * G + e4, ch) * 16 + 8 * (i4 & 1);
        const uint8_t* a1 = buf + chunk_pos<false>(32 * s + 16 + 4 * G + e4, ch) * 16 + 8 * (i4 & 1);
        const v4s_t r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t*)a0);
        const v4s_t r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t*)a1);
        w = make_uint4(__builtin_bit_cast(uint32_t, __builtin_shufflevector(r0, r0, 0, 1)),
                       __builtin_bit_cast(uint32_t, __builtin_shufflevector(r0, r0, 2, 3)),
                       __builtin_bit_cast(uint32_t, __builtin_shufflevector(r1, r1, 0, 1)),
                       __builtin_bit_cast(uint32_t, __builtin_shufflevector(r1, r1, 2, 3)));
      }
      return w;
    };
    uint4 vr = v_read(0);
#pragma unroll
    for (int step = 0; step < 64; ++step) {
      const int dn = step >> 1, s = step & 1;
      const uint4 cur = vr;
      if (step + 1 < 64) vr = v_read(step + 1);
      const bf16x8_t bv = kE4M3 ? fp8x8_to_bf16(cur.x, cur.y) : as_bf16x8(cur.x, cur.y, cur.z, cur.w);
      O[dn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf[s], bv, O[dn], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- tile pipeline
  constexpr int kAhead = M::kBufs - 1;
#pragma unroll
  for (int t = 0; t < kAhead; ++t)
    if (t < n_tiles) issue(t);
  for (int t = 0; t < n_tiles; ++t) {
    if (t + kAhead < n_tiles) issue(t + kAhead);
    const int after = min(kAhead, n_tiles - 1 - t);
    if constexpr (kAhead == 2) {
      if (after == 2) wait_vm<2 * kMine>();
      else if (after == 1) wait_vm<kMine>();
      else wait_vm<0>();
    } else {
      if (after == 1) wait_vm<kMine>();
      else wait_vm<0>();
    }
    wg_barrier();  // tile t is in LDS for every wave
    const int page = page_of(t);
    const int nv = min(kTile, t_end - (t_begin + kTile * t));
    if (page >= 0 && page < p.num_pages) {
      if (nv < kTile) {
        // rows past the context hold stale bytes; V must be finite there
        uint8_t* buf = tiles + (t % M::kBufs) * M::kTileBytes;
        const int n16 = (kTile - nv) * M::kRowChunks;
        for (int i = tid; i < n16; i += kThreads)
          *reinterpret_cast<uint4*>(buf + nv * M::kRowBytes + 16 * i) = make_uint4(0u, 0u, 0u, 0u);
        wg_barrier();
      }
      compute(t, nv);
    }
    wg_barrier();  // every wave is done with the buffer before it is reloaded
  }

  // ---- finish: denominators per head, then the normalised partial rows
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (G == 0) l_s[wave][lr] = l;
  __builtin_amdgcn_wave_barrier();
  const int64_t bh0 = static_cast<int64_t>(b) * p.num_q_heads + h_base;
  if (G == 0)
    p.lse_part[(bh0 + lr) * p.max_splits + c] = l > 0.0f ? (m + __log2f(l)) * kLn2 : -INFINITY;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int hl = 4 * G + r;
    const float lh = l_s[wave][hl];
    const float f = lh > 0.0f ? o_scale / lh : 0.0f;
    float* dst = p.o_part + ((bh0 + hl) * p.max_splits + c) * kDv + lr;
#pragma unroll
    for (int dn = 0; dn < 32; ++dn) dst[16 * dn] = O[dn][r] * f;
  }
}

// ---------------------------------------------------------------------------
// Wide variant for an e4m3 cache and query heads in multiples of 128: one
// workgroup of 4 waves takes all 128 heads of a (request, split), each wave
// 32 heads, so every cached byte is converted and read from LDS by 4 waves
// instead of 8. MFMA 32x32x16 (bf16 in, fp32 out):
//   A lane l: row l%32, k 8(l/32)..+7;  B lane l: column l%32, k 8(l/32)..+7;
//   D lane l, element i: row 8(i/4) + 4(l/32) + i%4, column l%32.
// S^T = K Q^T per 32-token block (M = tokens, N = the wave's 32 heads, 36
// k-steps of 16 dims), so a lane holds the scores of one head (l%32) for
// tokens {8u + 4(l/32) + r}; those are exactly the A operand of P V (M =
// heads, k = tokens) when the V operand is read in the same token order with
// ds_read_tr8_b64. The 32 x 512 accumulators of a wave live in the
// accumulation registers.
//
// Tile layout in LDS: 16-byte chunk c of row r at position c ^ ((r >> 2) & 3)
// of the row, which puts any 16 consecutive rows of one chunk (K operand
// reads) and the 8 rows x 2 half-chunks of a transposing V read on distinct
// bank groups. The ring holds 4 tiles; tile t + 3 is loaded into the buffer
// of tile t - 1 right after the barrier that opens tile t, so one barrier per
// tile suffices.
//
// Work unit order: blockIdx.y counts splits from the end of each request
// downwards (the first units dispatched are the ones far from the end,
// which are full), so the short last splits run last and fill the tail;
// the request index is rotated by blockIdx.y so that one request's units
// spread over all XCDs.
constexpr int kWideHeads = 32;
constexpr float kWideTau = 60.0f;  // log2 headroom of the reference max
constexpr int kWideBufs = 2;
constexpr int kWideTileBytes = kTile * kDk;          // 36 KB
constexpr int kWideDma = kWideTileBytes / 1024;      // 36 loads of 1 KB
constexpr int kWideMine = kWideDma / 4;              // 9 per wave

typedef float floatx16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int wide_pos(int r, int c) { return c ^ ((r >> 2) & 3); }

__global__ void __launch_bounds__(256, 1) decode_mla_wide_kernel(DecodeParams p, int n_splits,
                                                                 int head_groups) {
  static_assert((kWideBufs - 2) * kWideMine <= 63, "vmcnt counts to 63");
  __shared__ __attribute__((aligned(16))) uint8_t tiles[kWideBufs * kWideTileBytes];
  __shared__ int32_t pages[kMaxUnitTiles];
  __shared__ float l_s[4][kWideHeads];
  __shared__ int vote[2][4];

  // Consecutive workgroup ids go to the 8 XCDs in turn, so the (request,
  // head group) index is rotated by the split row: the units of one request
  // land on different XCDs instead of all on XCD (index mod 8).
  const int bx = static_cast<int>((blockIdx.x + blockIdx.y) % gridDim.x);
  const int b = bx / head_groups;
  const int hg = bx - b * head_groups;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5;     // which half of the k range this lane supplies
  const int col = lane & 31;    // head (QK, D of S^T) or dim (PV, D of O)

  if (p.abort_flags && p.abort_flags[b]) return;
  const int L = p.seq_lens[b];
  if (L > p.max_seq_len || L <= 0) return;
  const int n_b = (L + p.split_tokens - 1) / p.split_tokens;
  const int c = n_b - n_splits + static_cast<int>(blockIdx.y);
  if (c < 0) return;
  const int t_begin = c * p.split_tokens;
  const int t_end = min(L, t_begin + p.split_tokens);
  const int n_tiles = (t_end - t_begin + kTile - 1) / kTile;
  const int h_base = hg * 128 + wave * kWideHeads;

  // q as B operands: k-step ks covers dims 32(ks/2) + 16hh + 8(ks%2) .. +7 for
  // this lane's head, so one 16-byte K read serves two k-steps
  bf16x8_t qf[36];
  {
    const int qi = b * p.num_q_heads + h_base + col;  // < 2^31 (checked on the host)
    const uint16_t* qrow = p.q + static_cast<int64_t>(qi) * kDk;
#pragma unroll
    for (int ks = 0; ks < 36; ++ks)
      qf[ks] = *reinterpret_cast<const bf16x8_t*>(qrow + 32 * (ks >> 1) + 16 * hh + 8 * (ks & 1));
  }
  const float qk_scale = p.k_scale[0] * p.sm_scale_log2;
  const float o_scale = p.v_scale[0];

  const int32_t* bt = p.block_table + static_cast<int64_t>(b) * p.max_pages;
  const int first_page = t_begin / kTile;
  for (int j = tid; j < n_tiles; j += 256) pages[j] = bt[first_page + j];
#pragma unroll
  for (int ks = 0; ks < 36; ++ks) asm volatile("" : : "v"(qf[ks]));
  asm volatile("" : : "s"(qk_scale), "s"(o_scale));
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" : : : "memory");

  // per-lane source of this wave's load i of a tile: load k = wave + 4i fills
  // LDS chunks 64k .. 64k+63, chunk q = row q/36, position q%36
  auto doff = [&](int i) __attribute__((always_inline)) {
    const int q = 64 * (wave + 4 * i) + lane;
    const int r = q / 36;
    const int pp = q - 36 * r;
    return static_cast<uint32_t>(r * kDk + wide_pos(r, pp) * 16);
  };
  const uint8_t* kpool = static_cast<const uint8_t*>(p.k_pool);
  const uint32_t tiles0 = lds_addr(tiles);
  auto page_of = [&](int t) __attribute__((always_inline)) {
    return __builtin_amdgcn_readfirstlane(pages[t]);
  };
  auto issue = [&](int t) __attribute__((always_inline)) {
    int page = page_of(t);
    if (page < 0 || page >= p.num_pages) page = 0;  // loaded but never used
    const uint8_t* base = kpool + static_cast<int64_t>(page) * kWideTileBytes;
    const uint32_t buf = tiles0 + (t % kWideBufs) * kWideTileBytes;
#pragma unroll
    for (int i = 0; i < kWideMine; ++i) dma16(buf + 1024 * (wave + 4 * i), doff(i), base);
  };

  floatx16_t O[16];
#pragma unroll
  for (int nb = 0; nb < 16; ++nb)
#pragma unroll
    for (int i = 0; i < 16; ++i) O[nb][i] = 0.f;
  // Scores are taken relative to a reference max m (log2 domain) that is set
  // by the first tile and never moves by less than kWideTau: p = 2^(s - m)
  // stays below 2^kWideTau, far inside bf16 and fp32 range, so O never has to
  // be rescaled inside the loop. A score above m + kWideTau (not reachable by
  // attention scores in practice) restarts the unit with the larger m.
  float m = kMInit;
  float l = 0.f;
  const int a16 = (lane >> 4) & 1;
  const int jj = lane & 15;
  const int kk = jj >> 1;

  // Per-lane LDS offsets. The swizzle term (r >> 2) & 3 of every row a lane
  // reads is the same in both halves and both k-steps of a half (row offsets
  // 32mb + 16u are multiples of 16), so four bases cover all reads:
  // K operand, chunk 2j + hh of row 32mb + col, sits at position
  // 4(j/2) + ((2(j%2) + hh) ^ sw): base koff[j%2] + 64(j/2) + 32mb rows;
  // V operand of k-step (mb, u): the 16 lanes of a group address rows
  // T[jj/2] of the step, half-chunk jj%2 of chunk 2nb + a16, at position
  // 4(nb/2) + ((2(nb%2) + a16) ^ sw): base voff[nb%2] + 64(nb/2) + (32mb + 16u) rows.
  // Lane i of a group then holds dim 32nb + 16a16 + i of the step's 8 tokens
  // in P's order.
  uint32_t koff[2], voff[2];
  {
    const int rk = col;
    const int rv = 8 * (kk >> 2) + 4 * hh + (kk & 3);
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      koff[x] = static_cast<uint32_t>(rk * kDk + wide_pos(rk, 2 * x + hh) * 16);
      voff[x] = static_cast<uint32_t>(rv * kDk + wide_pos(rv, 2 * x + a16) * 16 + 8 * (jj & 1));
    }
  }
  bool jump = false;  // a score went above the reference max by more than kWideTau

  // One 32-token half (mb) of a tile: S^T, numerators, O += P V.
  auto half_tile = [&](const uint8_t* buf, int mb, int nv) __attribute__((always_inline)) {
    floatx16_t st;
#pragma unroll
    for (int i = 0; i < 16; ++i) st[i] = 0.f;
    const uint8_t* kb0 = buf + 32 * mb * kDk + koff[0];
    const uint8_t* kb1 = buf + 32 * mb * kDk + koff[1];
    auto k_read = [&](int j) __attribute__((always_inline)) {
      return *reinterpret_cast<const uint4*>(((j & 1) ? kb1 : kb0) + 64 * (j >> 1));
    };
    constexpr int kKAhead = 3;  // 16-byte K reads in flight ahead of their MFMAs
    uint4 kq[kKAhead];
#pragma unroll
    for (int a = 0; a < kKAhead; ++a) kq[a] = k_read(a);
#pragma unroll
    for (int j = 0; j < 18; ++j) {
      const uint4 cur = kq[j % kKAhead];
      if (j + kKAhead < 18) kq[j % kKAhead] = k_read(j + kKAhead);
      st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fp8x8_to_bf16(cur.x, cur.y), qf[2 * j], st, 0, 0, 0);
      st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fp8x8_to_bf16(cur.z, cur.w), qf[2 * j + 1], st, 0, 0, 0);
    }
    // scores: st[i] is token 32mb + 8(i/4) + 4hh + i%4 of head h_base + col
    float lm = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float v = st[i] * qk_scale;
      st[i] = (32 * mb + 8 * (i >> 2) + 4 * hh + (i & 3) < nv) ? v : -INFINITY;
      lm = fmaxf(lm, st[i]);
    }
    // the lanes col and col + 32 hold the two token halves of one head and
    // feed the same A row of PV: both take the head's maximum, so their m
    // (and the numerators summed into one l) always agree
    lm = fmaxf(lm, __shfl_xor(lm, 32));
    if (m == kMInit) {  // first scores of the unit set the reference max
      m = lm > -INFINITY ? lm : kMInit;
    } else if (lm > m + kWideTau) {
      jump = true;
      m = lm;  // raised; the unit is redone with it (see the pipeline)
    }
    // numerators as A operands of the two PV k-steps of this half:
    // k-step u takes st[8u .. 8u+7] (tokens 32mb + 16u + {0..3, 8..11} + 4hh)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float pr[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        pr[k] = __builtin_amdgcn_exp2f(st[8 * u + k] - m);
        l += pr[k];
      }
      bf16x8_t pf;
#pragma unroll
      for (int k = 0; k < 8; ++k) pf[k] = static_cast<__bf16>(pr[k]);
      const uint8_t* vb0 = buf + (32 * mb + 16 * u) * kDk + voff[0];
      const uint8_t* vb1 = buf + (32 * mb + 16 * u) * kDk + voff[1];
      auto v_read = [&](int nb) __attribute__((always_inline)) {
        const uint8_t* ad = ((nb & 1) ? vb1 : vb0) + 64 * (nb >> 1);
        const v2i_t r8 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_t*)ad);
        return make_uint2(static_cast<uint32_t>(r8[0]), static_cast<uint32_t>(r8[1]));
      };
      constexpr int kVAhead = 6;  // tr8 reads in flight ahead of their MFMA
      uint2 vq[kVAhead];
#pragma unroll
      for (int a = 0; a < kVAhead; ++a) vq[a] = v_read(a);
#pragma unroll
      for (int nb = 0; nb < 16; ++nb) {
        const uint2 cur = vq[nb % kVAhead];
        if (nb + kVAhead < 16) vq[nb % kVAhead] = v_read(nb + kVAhead);
        O[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pf, fp8x8_to_bf16(cur.x, cur.y), O[nb], 0, 0, 0);
      }
    }
  };

  // ---- tile pipeline: kWideBufs - 1 tiles loaded ahead. A unit in which
  // some score jumped (see above) is redone from tile 0 with the raised
  // reference maxima once every wave has voted.
  bool done = false;
  while (!done) {
#pragma unroll
    for (int t = 0; t < kWideBufs - 1; ++t)
      if (t < n_tiles) issue(t);
    for (int t = 0; t < n_tiles; ++t) {
      const int after = min(kWideBufs - 2, n_tiles - 1 - t);
      if (after >= 2) wait_vm<2 * kWideMine>();
      else if (after == 1) wait_vm<kWideMine>();
      else wait_vm<0>();
      wg_barrier();  // tile t is in LDS for every wave; every wave is done with tile t - 1
      if (t + kWideBufs - 1 < n_tiles) issue(t + kWideBufs - 1);
      const int page = page_of(t);
      const int nv = min(kTile, t_end - (t_begin + kTile * t));
      if (page >= 0 && page < p.num_pages) {
        uint8_t* buf = tiles + (t % kWideBufs) * kWideTileBytes;
        if (nv < kTile) {
          // rows past the context hold stale bytes; their V part must be finite
          const int n16 = (kTile - nv) * (kDk / 16);
          for (int i = tid; i < n16; i += 256)
            *reinterpret_cast<uint4*>(buf + nv * kDk + 16 * i) = make_uint4(0u, 0u, 0u, 0u);
          wg_barrier();
        }
#pragma unroll 1
        for (int mb = 0; mb < 2; ++mb) half_tile(buf, mb, nv);
      }
    }
    if (lane == 0) vote[0][wave] = jump ? 1 : 0;
    wg_barrier();
    done = (vote[0][0] | vote[0][1] | vote[0][2] | vote[0][3]) == 0;
    if (!done) {
      // drain the loads in flight (none: the last tile waited for all) and
      // start over; each head keeps its raised reference max
      wait_vm<0>();
      jump = false;
      l = 0.f;
#pragma unroll
      for (int nb = 0; nb < 16; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) O[nb][i] = 0.f;
    }
    wg_barrier();  // the vote has been read before it is written again
  }

  // ---- finish: denominators per head, then the normalised partial rows.
  // Lane indices and output addresses are formed afresh here (mbcnt gives
  // the lane) so that nothing from the prologue stays alive through the loop.
  const int lane_e = static_cast<int>(__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)));
  const int col_e = lane_e & 31, hh_e = lane_e >> 5;
  l += __shfl_xor(l, 32);
  if (hh_e == 0) l_s[wave][col_e] = l;
  __builtin_amdgcn_wave_barrier();
  int b_out = b, h_out = h_base, c_out = c;
  asm volatile("" : "+s"(b_out), "+s"(h_out), "+s"(c_out));
  const int bh0 = b_out * p.num_q_heads + h_out;
  if (hh_e == 0)
    p.lse_part[static_cast<int64_t>(bh0 + col_e) * p.max_splits + c_out] =
        l > 0.0f ? (m + __log2f(l)) * kLn2 : -INFINITY;
  float f[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float lh = l_s[wave][8 * (i >> 2) + 4 * hh_e + (i & 3)];
    f[i] = lh > 0.0f ? o_scale / lh : 0.0f;
  }
  float* dst0 = p.o_part + (static_cast<int64_t>(bh0 + 4 * hh_e) * p.max_splits + c_out) * kDv + col_e;
  const int64_t head_stride = static_cast<int64_t>(p.max_splits) * kDv;
#pragma unroll
  for (int nb = 0; nb < 16; ++nb)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      dst0[(8 * (i >> 2) + (i & 3)) * head_stride + 32 * nb] = O[nb][i] * f[i];
}

}  // namespace

bool mla_fast_path_supported(int dk, int dv, int num_kv_heads, int num_q_heads, int page_size,
                             int split_tokens) {
  return dk == kDk && dv == kDv && num_kv_heads == 1 && page_size == kTile &&
         num_q_heads % 64 == 0 && num_q_heads <= 1024 && split_tokens <= kMaxUnitTiles * kTile;
}

int launch_decode_mla(const DecodeParams& p, bool e4m3, int n_split_blocks, int batch,
                      hipStream_t stream) {
  if (e4m3 && p.num_q_heads % 128 == 0 && n_split_blocks <= 65535) {
    const int head_groups = p.num_q_heads / 128;
    const dim3 grid(batch * head_groups, n_split_blocks);
    decode_mla_wide_kernel<<<grid, 256, 0, stream>>>(p, n_split_blocks, head_groups);
    return pkv::launch_status();
  }
  const int head_groups = p.num_q_heads / 64;
  const int n_x = (n_split_blocks + 7) / 8 * 8 * head_groups;
  const dim3 grid(n_x, batch);
  if (e4m3) {
    decode_mla_kernel<true><<<grid, 256, 0, stream>>>(p, n_split_blocks, head_groups);
  } else {
    decode_mla_kernel<false><<<grid, 256, 0, stream>>>(p, n_split_blocks, head_groups);
  }
  return pkv::launch_status();
}
