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
    p.lse_part[(bh0 + lr) * p.max_splits + c] = !(l <= 0.0f) ? (m + __log2f(l)) * kLn2 : -INFINITY;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int hl = 4 * G + r;
    const float lh = l_s[wave][hl];
    const float f = !(lh <= 0.0f) ? o_scale / lh : 0.0f;
    float* dst = p.o_part + ((bh0 + hl) * p.max_splits + c) * kDv + lr;
#pragma unroll
    for (int dn = 0; dn < 32; ++dn) dst[16 * dn] = O[dn][r] * f;
  }
}

// ---------------------------------------------------------------------------
// Wide variant for query heads in multiples of 128, bf16 cache (the e4m3
// cache has its own kernel below): one workgroup of 4 waves takes all 128
// heads of a range of splits. MFMA
// 32x32x16 (bf16 in, fp32 out):
//   A lane l: row l%32, k 8(l/32)..+7;  B lane l: column l%32, k 8(l/32)..+7;
//   D lane l, element i: row 8(i/4) + 4(l/32) + i%4, column l%32.
// The cache is taken 32 tokens (half a tile) at a time. QK^T: wave w holds
// q of heads 32 w .. 32 w + 31 in registers and forms S^T = K Q^T for them
// (M = tokens, N = heads, 36 k-steps of 16 dims); its softmax numerators go
// to LDS as bf16 (row = head, 32 tokens). P V: after a barrier, wave w
// multiplies all 128 heads' numerators (A, read back from LDS) by dims 128 w
// .. 128 w + 127 of V (B, read with ds_read_b64_tr_b16), so every V byte in
// LDS is read once per workgroup instead of once per wave; its 128 x 128
// accumulators live in the accumulation registers. One accumulator per
// 32-token block of S^T suffices: dependent MFMAs issue back to back.
//
// The cache arrives by direct-to-LDS loads in a four-slot ring of 32-row
// halves (three halves load while one is used), already in the layout the
// operands are read in. The loads of a later half are spread over the MFMAs
// of a QK^T.
//
// bf16 half layout (32 rows of 72 chunks of 16 bytes): nine 4 KB groups,
// group g holding chunks 8 g .. 8 g + 7 of every row, row r at 128 r of the
// group and chunk c at position (c % 8) ^ swz(r) of those 128 bytes, swz(r)
// = bit 1 | bit 2 << 1 | (bit 1 ^ bit 3) << 2 of r. The bank group (of 16
// four-bank groups) of position p in row r is then 8 (r & 1) + p; with this
// swizzle the 16 rows of one pass of a K operand read (16 consecutive rows,
// one chunk) and the 4 rows x 4 chunks of one pass of a transposing V read
// fall on distinct bank groups (checked exhaustively). Every lane's offsets are a
// fixed base plus immediates: a cache load fills 1 KB of a group (8 rows x
// 128 bytes of the page), an operand read steps 4 KB per 8 chunks.
//
// Work split: one workgroup per compute unit (per 128-head group), each
// taking an equal share of the launch's tiles. The tiles of the requests
// with work (not aborted, not empty) are laid end to end; range i is
// [i T / R, (i + 1) T / R) of the T tiles, each end moved to the nearest
// split boundary of the request it falls in, so a range is a run of whole
// splits of one or more requests (a segment per request). A segment is
// decoded as one unit (its softmax state carried across its splits) and
// writes its partial in the row of its first split; the rows of its other
// splits get lse = -inf and no o_part (pkv_combine skips them). Shares of
// equal size keep every compute unit busy to the end whatever the length
// mix; the split only sets the granularity of the cuts.
constexpr int kWideHeads = 32;
constexpr float kWideTau = 60.0f;            // log2 headroom of the reference max
constexpr int kRow16 = kDk * 2;              // bf16 row: 1152 bytes, 72 chunks
constexpr int kHalf16 = 32 * kRow16;         // 36 KB: 32 bf16 rows
constexpr int kGroup16 = 32 * 128;           // 4 KB: 8 chunks of each of 32 rows
constexpr int kVmcnt0 = 0x0F70;              // s_waitcnt vmcnt(0), other counters free
constexpr int kTile16 = kTile * kRow16;      // 72 KB: a bf16 page
constexpr int kTile8 = kTile * kDk;          // 36 KB of codes
constexpr int kDma = 9;                      // loads per wave per code tile or bf16 half
constexpr int kSlots16 = 4;                  // bf16 halves in the ring

typedef float floatx16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int wswz(int r) {
  return ((r >> 1) & 1) | (((r >> 2) & 1) << 1) | ((((r >> 1) ^ (r >> 3)) & 1) << 2);
}

// max(x, x of lane l ^ 32) in every lane: a copy of x and x swap their
// halves of the wave (v_permlane32_swap), so every lane holds both values.
// Written out (the swap, and the wait state its read of the copy needs):
// the compiler builtin for it lets the max be folded away.
__device__ __forceinline__ float max_across_halves(float x) {
  float a = x, b;
  asm volatile("v_mov_b32 %1, %0\n\ts_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "=&v"(b));
  return fmaxf(a, b);
}

// Inclusive prefix sum over the wave.
__device__ __forceinline__ int wave_scan_i(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

// Tiles request j contributes to the launch (0 if it has no work).
__device__ __forceinline__ int req_tiles(const DecodeParams& p, int j) {
  if (j >= p.batch) return 0;
  const int L = p.seq_lens[j];
  const bool ab = p.abort_flags && p.abort_flags[j];
  return (ab || L <= 0 || L > p.max_seq_len) ? 0 : (L + kTile - 1) / kTile;
}

// Total tiles of the launch (uniform).
__device__ __forceinline__ int64_t launch_tiles(const DecodeParams& p) {
  const int lane = threadIdx.x & 63;
  int64_t t = 0;
  for (int b0 = 0; b0 < p.batch; b0 += 64)
    t += __builtin_amdgcn_readlane(wave_scan_i(req_tiles(p, b0 + lane)), 63);
  return t;
}

// The request holding flattened tile x (x < total): its index, its first
// flattened tile and its tile count (uniform).
__device__ __forceinline__ void locate(const DecodeParams& p, int64_t x, int& b_out,
                                       int64_t& start_out, int& n_out) {
  const int lane = threadIdx.x & 63;
  int64_t base = 0;
  for (int b0 = 0; b0 < p.batch; b0 += 64) {
    const int n = req_tiles(p, b0 + lane);
    const int incl = wave_scan_i(n);
    const int tot = __builtin_amdgcn_readlane(incl, 63);
    if (x < base + tot) {
      const int bl = __popcll(__ballot(base + incl <= x));
      b_out = b0 + bl;
      start_out = base + __builtin_amdgcn_readlane(incl - n, bl);
      n_out = __builtin_amdgcn_readlane(n, bl);
      return;
    }
    base += tot;
  }
  b_out = p.batch;
  start_out = base;
  n_out = 0;
}

// Flattened tile x moved to the nearest split boundary of its request (or
// the request's end); the same x gives the same boundary in every workgroup.
__device__ __forceinline__ int64_t snap(const DecodeParams& p, int64_t x, int64_t total,
                                        int tps) {
  if (x >= total) return total;
  int b, n;
  int64_t start;
  locate(p, x, b, start, n);
  const int j = static_cast<int>(x - start);
  const int jj = min(n, (j + tps / 2) / tps * tps);
  return start + jj;
}

__global__ void __launch_bounds__(256, 1) decode_mla_wide_kernel(DecodeParams p, int head_groups,
                                                                 int n_ranges) {
  // [ring of 4 bf16 halves: 4 x 36 KB], then the half's numerators P: 128
  // heads x 32 tokens of bf16, rows padded to 80 bytes
  constexpr int kTiles = kSlots16 * kHalf16;
  constexpr int kPRow = 80;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kTiles + 128 * kPRow];
  __shared__ int32_t pages[kMaxUnitTiles];
  __shared__ float l_all[128];
  __shared__ int vote[4];

  const int hg = static_cast<int>(blockIdx.x) % head_groups;
  const int ri = static_cast<int>(blockIdx.x) / head_groups;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5;     // which half of the k range this lane supplies
  const int col = lane & 31;    // head (QK, D of S^T) or dim (PV, D of O)
  const int tps = p.split_tokens / kTile;  // tiles per split

  // this workgroup's range [s0, s1) of the launch's flattened tiles
  const int64_t total = launch_tiles(p);
  const int64_t s0 = snap(p, ri * total / n_ranges, total, tps);
  const int64_t s1 = snap(p, (ri + 1) * total / n_ranges, total, tps);
  if (s0 >= s1) return;

  const float qk_scale = p.sm_scale_log2;
  const uint8_t* kpool = static_cast<const uint8_t*>(p.k_pool);
  const uint32_t lds0 = lds_addr(lds);
  uint8_t* pbuf = lds + kTiles;
  // QK: this wave's 32 heads; PV: this wave's 128 dims, all 128 heads
  const int h_base = hg * 128 + wave * kWideHeads;

  // Per-lane LDS byte offsets in a bf16 half (the swizzle only touches the
  // low three bits of a chunk index, so the rest is an immediate or a
  // wave-uniform add):
  // K operand of k-step ks: row col, chunk 2 ks + hh in group ks / 4 at
  // position (2 (ks % 4) + hh) ^ swz(col);
  // V operand of dim block nb, token step u: the 16 lanes of group gq =
  // lane / 16 read rows 8 hh + e and 8 hh + 4 + e of the step (e = (lane %
  // 16) / 4), the 8 bytes (lane % 2) of chunk 16 wave + 4 nb + 2 a +
  // (lane % 4) / 2 (a = gq % 2): dims 128 wave + 32 nb + 16 a .. + 15;
  // P operand of head block hb, token step u: head 32 hb + col, tokens
  // 16 u + 8 hh .. + 7.
  uint32_t koff[4], voff[2][2];
  {
    const int fr = wswz(col);
#pragma unroll
    for (int j = 0; j < 4; ++j) koff[j] = static_cast<uint32_t>(col * 128 + (((2 * j + hh) ^ fr) << 4));
    const int e = (lane & 15) >> 2, a = (lane >> 4) & 1, i4 = lane & 3;
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int rv = 8 * hh + 4 * x + e;
#pragma unroll
      for (int par = 0; par < 2; ++par)  // parity of nb
        voff[x][par] = static_cast<uint32_t>(
            rv * 128 + ((((4 * par + 2 * a + (i4 >> 1)) ^ wswz(rv))) << 4) + 8 * (i4 & 1));
    }
  }
  const uint32_t vwave = static_cast<uint32_t>(wave) * 2 * kGroup16;  // chunk 16 wave
  const uint32_t poff = static_cast<uint32_t>(col * kPRow + 16 * hh);
  // bf16 cache loads: lane l of wave w takes row 8 w + l / 8 of a half, the
  // chunk that lands at position l % 8 of that row's group
  const int dma_row = 8 * wave + (lane >> 3);
  const uint32_t dma_off = static_cast<uint32_t>(dma_row * kRow16 + (((lane & 7) ^ wswz(dma_row)) << 4));

  int64_t x = s0;
  while (x < s1) {
    // ---- the segment of request b in this range: its tiles [j0, j1)
    int b, nt;
    int64_t start;
    locate(p, x, b, start, nt);
    const int j0 = static_cast<int>(x - start);
    const int j1 = static_cast<int>(min<int64_t>(nt, s1 - start));
    x = start + j1;
    const int L = p.seq_lens[b];
    const int t_begin = j0 * kTile;
    const int t_end = min(L, j1 * kTile);
    const int n_tiles = j1 - j0;
    const int c0 = j0 / tps;  // the split whose row takes the partial

    // q as B operands: k-step ks covers dims 16 ks + 8 hh .. +7 of head h_base + col
    bf16x8_t qf[36];
    {
      const int qi = b * p.num_q_heads + h_base + col;  // < 2^31 (checked on the host)
      const uint16_t* qrow = p.q + static_cast<int64_t>(qi) * kDk + 8 * hh;
#pragma unroll
      for (int ks = 0; ks < 36; ++ks) qf[ks] = *reinterpret_cast<const bf16x8_t*>(qrow + 16 * ks);
      // wait for q here, with a wait the compiler accounts for: it does not
      // see the cache loads (inline asm), and a wait it placed for q inside
      // the tile loop would also wait for every tile load in flight
      __builtin_amdgcn_s_waitcnt(kVmcnt0);
    }
    const int32_t* bt = p.block_table + static_cast<int64_t>(b) * p.max_pages;

    // O[hb][nb]: heads 32 hb + .., dims 128 wave + 32 nb + .. (D layout)
    floatx16_t O[4][4];
#pragma unroll
    for (int hb = 0; hb < 4; ++hb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) O[hb][nb][i] = 0.f;
    // Scores are taken relative to a reference max m (log2 domain) that is
    // set by the first tile and never moves by less than kWideTau: p = 2^(s
    // - m) stays below 2^kWideTau, far inside bf16 and fp32 range, so O never
    // has to be rescaled inside the loop (which is what lets the waves that
    // own a head's scores and the waves that own its output rows differ). A
    // score above m + kWideTau (not reachable by attention scores in
    // practice) restarts the segment with the larger m.
    float m = kMInit;
    float l = 0.f;
    bool jump = false;

    // QK^T of a 32-token half (rows of buf; row r is token 32 mb + r of the
    // tile, of which nv are valid) for this wave's 32 heads; the numerators
    // go to pbuf as bf16 (row = head, natural token order).
    // `after(ks)` runs after the MFMA of k-step ks (the cache loads are
    // spread over the chain there, so their issue overlaps the MFMAs).
    auto qk_half = [&](const uint8_t* buf, int mb, int nv, auto&& after) __attribute__((always_inline)) {
      floatx16_t st;
#pragma unroll
      for (int i = 0; i < 16; ++i) st[i] = 0.f;
      auto k_read = [&](int ks) __attribute__((always_inline)) {
        return *reinterpret_cast<const uint4*>(buf + koff[ks & 3] + kGroup16 * (ks >> 2));
      };
      constexpr int kKAhead = 4;  // K reads in flight ahead of their MFMAs
      uint4 kq[kKAhead];
#pragma unroll
      for (int a = 0; a < kKAhead; ++a) kq[a] = k_read(a);
#pragma unroll
      for (int ks = 0; ks < 36; ++ks) {
        const uint4 cur = kq[ks % kKAhead];
        if (ks + kKAhead < 36) kq[ks % kKAhead] = k_read(ks + kKAhead);
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(cur.x, cur.y, cur.z, cur.w),
                                                     qf[ks], st, 0, 0, 0);
        after(ks);
      }
      // scores: st[i] is token 32mb + 8(i/4) + 4hh + i%4 of head h_base + col;
      // the exponent of token i is st[i] * qk_scale - m (one fused step
      // where every token of the half is in the context)
      const bool full = 32 * mb + 32 <= nv;
      float lm = -INFINITY;
      if (full) {
        // the largest scaled score, from the largest (or, for a negative
        // scale, smallest) raw one: rounding is monotonic
        if (qk_scale >= 0.0f) {
#pragma unroll
          for (int i = 0; i < 16; ++i) lm = fmaxf(lm, st[i]);
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) lm = fmaxf(lm, -st[i]);
        }
        lm *= fabsf(qk_scale);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float v = st[i] * qk_scale;
          st[i] = (32 * mb + 8 * (i >> 2) + 4 * hh + (i & 3) < nv) ? v : -INFINITY;
          lm = fmaxf(lm, st[i]);
        }
      }
      // the lanes col and col + 32 hold the two token halves of one head:
      // both take the head's maximum (the two halves of the wave swap
      // values), so their m (and the numerators summed into one l) always
      // agree
      lm = max_across_halves(lm);
      // the first scores of the segment set the reference max; a score
      // above it by more than kWideTau raises it, and the segment is redone
      const bool first = m == kMInit;
      const bool raise = !first && lm > m + kWideTau;
      jump = jump || raise;
      m = first ? (lm > -INFINITY ? lm : kMInit) : (raise ? lm : m);
      auto store = [&](int q, const float (&pr)[4]) __attribute__((always_inline)) {
        const bf16x2_t lo = {static_cast<__bf16>(pr[0]), static_cast<__bf16>(pr[1])};
        const bf16x2_t hi = {static_cast<__bf16>(pr[2]), static_cast<__bf16>(pr[3])};
        *reinterpret_cast<uint2*>(pbuf + (wave * kWideHeads + col) * kPRow + 16 * q + 8 * hh) =
            make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
      };
      if (full) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float pr[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            pr[k] = __builtin_amdgcn_exp2f(__builtin_fmaf(st[4 * q + k], qk_scale, -m));
            l += pr[k];
          }
          store(q, pr);
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float pr[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            pr[k] = __builtin_amdgcn_exp2f(st[4 * q + k] - m);
            l += pr[k];
          }
          store(q, pr);
        }
      }
    };

    // O += P V of a half for this wave's 128 dims and all 128 heads;
    // `after(j)` runs after MFMA j of 32 (work that interleaves with them)
    auto pv_half = [&](const uint8_t* buf, auto&& after) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        bf16x8_t pa[4], vb[4];
#pragma unroll
        for (int hb = 0; hb < 4; ++hb)
          pa[hb] = *reinterpret_cast<const bf16x8_t*>(pbuf + poff + hb * 32 * kPRow + 32 * u);
        const uint8_t* vrow = buf + 16 * u * 128 + vwave;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const uint32_t o = kGroup16 * (nb >> 1);
          const v4s_t r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t*)(vrow + voff[0][nb & 1] + o));
          const v4s_t r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t*)(vrow + voff[1][nb & 1] + o));
          vb[nb] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
        }
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
          for (int hb = 0; hb < 4; ++hb) {
            O[hb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[hb], vb[nb], O[hb][nb], 0, 0, 0);
            after(16 * u + 4 * nb + hb);
          }
      }
    };

    // ---- the segment's tiles, in chunks of at most kMaxUnitTiles (their
    // page ids in LDS). A segment in which some score jumped (see above) is
    // redone from its first tile with the raised reference maxima once every
    // wave has voted.
    bool done = false;
    while (!done) {
      for (int k0 = 0; k0 < n_tiles; k0 += kMaxUnitTiles) {
        const int kn = min(kMaxUnitTiles, n_tiles - k0);
        for (int j = tid; j < kn; j += 256) pages[j] = bt[j0 + k0 + j];
        // every load so far (q, page ids) completes before the first tile
        // load, so the vmcnt waits below count tile loads only
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" : : : "memory");
        auto page_of = [&](int t) __attribute__((always_inline)) {
          return __builtin_amdgcn_readfirstlane(pages[t]);
        };
        auto base_of = [&](int page) __attribute__((always_inline)) {
          if (page < 0 || page >= p.num_pages) page = 0;  // loaded but never used
          return kpool + static_cast<int64_t>(page) * kTile16;
        };
        auto page_base = [&](int t) __attribute__((always_inline)) { return base_of(page_of(t)); };
        // a page id read ahead (kept in a vector register until it is used,
        // so the read's latency passes during the MFMAs in between)
        auto page_ahead = [&](int t) __attribute__((always_inline)) { return pages[min(t, kn - 1)]; };
        auto nv_of = [&](int t) __attribute__((always_inline)) {
          return min(kTile, t_end - (t_begin + kTile * (k0 + t)));
        };
        // one half: QK^T, its numerators in LDS for every wave, then PV
        auto half = [&](const uint8_t* buf, int mb, int nv, auto&& after) __attribute__((always_inline)) {
          qk_half(buf, mb, nv, after);
          wg_barrier();  // every head's numerators are in pbuf
          pv_half(buf, [](int) {});
        };
        // ---- bf16: halves of a page, three ahead, straight into the
        // layout the operands are read in: load i of wave w fills group i,
        // rows 8 w .. 8 w + 7 (1 KB of LDS), each lane one chunk, reading
        // 128 bytes of each of 8 rows of the page
        const int nh = 2 * kn;
        auto half_base = [&](int h) __attribute__((always_inline)) {
          return page_base(h >> 1) + (h & 1) * kHalf16;
        };
        auto issue_one = [&](int h, const uint8_t* base, int i) __attribute__((always_inline)) {
          dma16(lds0 + (h % kSlots16) * kHalf16 + 1024 * wave + kGroup16 * i, dma_off, base + 128 * i);
        };
        auto issue = [&](int h) __attribute__((always_inline)) {
          const uint8_t* base = half_base(h);
#pragma unroll
          for (int i = 0; i < kDma; ++i) issue_one(h, base, i);
        };
        for (int h = 0; h < 3 && h < nh; ++h) issue(h);
        int pv_cur = page_ahead(0);  // page ids of tiles h / 2 and (h + 3) / 2
        int pv_far = page_ahead(1);
        for (int h = 0; h < nh; ++h) {
          const int later = min(2, nh - 1 - h);  // halves loading behind half h
          if (later == 2) wait_vm<2 * kDma>();
          else if (later == 1) wait_vm<kDma>();
          else wait_vm<0>();
          wg_barrier();  // half h is in LDS; every wave is done with half h - 1 and pbuf
          const int page = __builtin_amdgcn_readfirstlane(pv_cur);
          const int page_far = __builtin_amdgcn_readfirstlane(pv_far);
          pv_cur = page_ahead((h + 1) >> 1);
          pv_far = page_ahead((h + 4) >> 1);
          // half h + 3 goes to the slot of half h - 1, during half h's QK^T
          const bool more = h + 3 < nh;
          const uint8_t* nbase = more ? base_of(page_far) + ((h + 3) & 1) * kHalf16 : nullptr;
          const int t = h >> 1, xh = h & 1;
          const int nv = nv_of(t);
          if (!(page >= 0 && page < p.num_pages && 32 * xh < nv)) {
            if (more) {
#pragma unroll
              for (int i = 0; i < kDma; ++i) issue_one(h + 3, nbase, i);
            }
          } else {
            uint8_t* buf = lds + (h % kSlots16) * kHalf16;
            if (nv < 32 * xh + 32) {
              // rows past the context hold stale bytes; V must be finite there
              const int r0 = nv - 32 * xh;
              const int per_group = (32 - r0) * 8;  // chunks of those rows in a group
              for (int i = tid; i < 9 * per_group; i += 256) {
                const int g = i / per_group, rem = i - g * per_group;
                *reinterpret_cast<uint4*>(buf + g * kGroup16 + (r0 + (rem >> 3)) * 128 + 16 * (rem & 7)) =
                    make_uint4(0u, 0u, 0u, 0u);
              }
              wg_barrier();
            }
            half(buf, xh, nv, [&](int ks) __attribute__((always_inline)) {
              if (more && (ks & 3) == 3) issue_one(h + 3, nbase, ks >> 2);
            });
          }
        }
        wg_barrier();  // every wave is done with the slots and the page ids
      }
      // a jump in any lane of the wave (any of its heads) counts
      const bool wave_jump = __builtin_amdgcn_ballot_w64(jump) != 0;
      if (lane == 0) vote[wave] = wave_jump ? 1 : 0;
      wg_barrier();
      done = (vote[0] | vote[1] | vote[2] | vote[3]) == 0;
      if (!done) {
        // nothing is in flight (the last tile waited for all); start over,
        // each head keeping its raised reference max
        jump = false;
        l = 0.f;
#pragma unroll
        for (int hb = 0; hb < 4; ++hb)
#pragma unroll
          for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int i = 0; i < 16; ++i) O[hb][nb][i] = 0.f;
      }
      wg_barrier();  // the vote has been read before it is written again
    }

    // ---- the segment's partial: denominators per head (from the waves
    // that own the heads' scores), then the normalised rows (from the waves
    // that own the dims) in split c0's row; the rows of its other splits get
    // lse = -inf
    l += __shfl_xor(l, 32);
    const int64_t bh0 = static_cast<int64_t>(b) * p.num_q_heads + hg * 128;
    if (hh == 0) {
      l_all[wave * kWideHeads + col] = l;
      const int64_t row = (bh0 + wave * kWideHeads + col) * p.max_splits;
      p.lse_part[row + c0] = !(l <= 0.0f) ? (m + __log2f(l)) * kLn2 : -INFINITY;
      const int c_last = (j1 - 1) / tps;
      for (int cx = c0 + 1; cx <= c_last; ++cx) p.lse_part[row + cx] = -INFINITY;
    }
    wg_barrier();  // every head's denominator is in l_all
    // the stride is made opaque here so that the 64 row addresses are formed
    // per segment instead of being kept live (and spilled) across segments
    int64_t head_stride = static_cast<int64_t>(p.max_splits) * kDv;
    asm volatile("" : "+s"(head_stride));
    float* dst0 = p.o_part + (bh0 * p.max_splits + c0) * kDv + 128 * wave + col;
    int hq = 4 * hh;  // opaque for the same reason
    asm volatile("" : "+v"(hq));
#pragma unroll
    for (int hb = 0; hb < 4; ++hb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int hl = 32 * hb + 8 * (i >> 2) + hq + (i & 3);
        const float lh = l_all[hl];
        const float f = !(lh <= 0.0f) ? 1.0f / lh : 0.0f;
        float* dst = dst0 + hl * head_stride;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) dst[32 * nb] = O[hb][nb][i] * f;
      }
    wg_barrier();  // l_all is read before the next segment writes it
  }
}

// ---------------------------------------------------------------------------
// e4m3 cache, 128-head groups. Every wave owns 32 heads end to end: their q,
// scores, numerators and all 512 dims of their output rows (256
// accumulation registers), so scores never leave the lane that computed
// them. The waves share only the code tiles: a ring of three 36 KB tiles,
// two loading while one is used, and one barrier per 64-token tile. The
// work split is the bf16 wide kernel's (one workgroup per compute unit and
// 128-head group, balanced ranges of whole splits).
//  - QK^T: S^T = K Q^T on the bf16 MFMA 32x32x16, K's codes converted
//    (exactly) in registers as each wave reads them, q bf16: exact products
//    and fp32 accumulation. A 64-dim step reads a lane's 32 codes (dims 64 s
//    + 32 (l / 32) .. + 31 of its token) and runs four k-steps of 16; k-step
//    (s, j) pairs A's and B's dims 64 s + 32 (l / 32) + 8 j .. + 7.
//  - P V on gfx950's scaled fp8 MFMA 32x32x64
//    (v_mfma_scale_f32_32x32x64_f8f6f4: e4m3 operands, each 32-value block
//    of a row or column times a power of two given per lane, fp32
//    accumulation), V being the codes read with ds_read_b64_tr_b8. A head's
//    numerators over a 32-token half are scaled by 2^-e, e = the floor of the
//    half's largest exponent, so they lie in [0, 2), and split into two e4m3
//    parts, hi and lo = the remainder times 16 (eight significant bits in
//    all, as a bf16 numerator has); two MFMAs per 32 dims. The MFMA's adder
//    sums each run of eight k-values aligned to the run's largest product,
//    keeping about 13 bits below it (measured), so a weight's error stays
//    within the bf16 rounding the other kernels give it.
//
// MFMA 32x32x64 operand layout (measured): lane l supplies row (A) or
// column (B) l % 32 and 32 bytes; byte j < 16 of lane l is k-value 16 (l /
// 32) + j, byte j >= 16 is k-value 32 + 16 (l / 32) + j - 16; the scale of
// lane l % 32 multiplies k-values 0..31, that of lane l % 32 + 32 k-values
// 32..63. D as for the bf16 MFMA: lane l, element i is row 8 (i / 4) + 4 (l
// / 32) + i % 4, column l % 32. Only the pairing of A's and B's bytes
// matters: in P V (M = 32 heads, N = 32 dims, K = the 64 tokens of a tile)
// byte j of lane l is token 8 (j' / 4) + 4 (l / 32) + j' % 4 of the tile's
// first half for j < 16 (j' = j) and of its second half for j >= 16 (j' = j
// - 16) -- exactly the tokens whose scores QK^T leaves in lane l's
// accumulators (element i = j'), so the numerators go from the QK^T
// accumulators to the A operand without leaving the lane, and the scales of
// lane l % 32 (first half) and of lane l % 32 + 32 (second half) are the two
// halves' own.
//
// Code tile layout in LDS (64 rows, one per token): dims 0..511 in four 8 KB
// groups, group G holding 16-byte chunks 8 G .. 8 G + 7 of every row, row r
// at 128 r, chunk c at position (c % 8) ^ f8swz(r); the 64 rope dims in a 4
// KB group after them, row r at 64 r, chunk c at (c - 32) ^ f8swz4(r). K
// operand reads (16 rows, one chunk per pass) and the transposing V reads
// (8 rows, two chunks per pass) hit distinct banks (checked exhaustively).
// A direct-to-LDS load fills 1 KB of one group (8 rows, or 16 rope rows) and
// each lane fetches the global chunk its LDS position holds.
constexpr int kF8Slots = 3;             // code tiles in the ring
constexpr int kF8Ahead = kF8Slots - 1;  // tiles loading while one is used
constexpr int kQLds = 1;                // trailing 64-dim steps whose q lives in LDS
constexpr int kQReg = 9 - kQLds;        // 64-dim steps whose q lives in registers
constexpr int kF8Group = 8192;   // 64 rows x 128 bytes
constexpr int kF8Rope = 32768;   // the rope group: 64 rows x 64 bytes
constexpr float kF8MinExp = -100.0f;  // lowest numerator scale exponent

typedef int v8i_t __attribute__((ext_vector_type(8)));

// compile-time choice between two straight-line bodies
template <bool B>
struct FullTag {
  static constexpr bool value = B;
};

__device__ __forceinline__ int f8swz(int r) {
  return (((r >> 1) & 1) << 1) | (((r >> 3) & 1) << 2) | ((r >> 2) & 1);
}
__device__ __forceinline__ int f8swz4(int r) { return (r >> 2) & 3; }

__device__ __forceinline__ floatx16_t mfma_f8(const v8i_t& a, const v8i_t& b, const floatx16_t& c,
                                              int scale_a, int scale_b) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, scale_a, 0, scale_b);
}

__device__ __forceinline__ float pow2f(int e) { return __uint_as_float(static_cast<uint32_t>(127 + e) << 23); }

// Four floats x (already times 2^-e) -> their e4m3 codes hi (one word) and
// the codes lo of the remainders times 16 (one word).
__device__ __forceinline__ void split4(float x0, float x1, float x2, float x3, uint32_t& hi, uint32_t& lo) {
  int h = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
  h = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, h, true);
  const auto d0 = __builtin_amdgcn_cvt_pk_f32_fp8(h, false);
  const auto d1 = __builtin_amdgcn_cvt_pk_f32_fp8(h, true);
  int o = __builtin_amdgcn_cvt_pk_fp8_f32((x0 - d0[0]) * 16.0f, (x1 - d0[1]) * 16.0f, 0, false);
  o = __builtin_amdgcn_cvt_pk_fp8_f32((x2 - d1[0]) * 16.0f, (x3 - d1[1]) * 16.0f, o, true);
  hi = static_cast<uint32_t>(h);
  lo = static_cast<uint32_t>(o);
}

__global__ void __launch_bounds__(256, 1) decode_mla_f8_kernel(DecodeParams p, int head_groups,
                                                               int n_ranges) {
  // code tiles, then per wave q of the last kQLds 64-dim steps (4 KB each:
  // its four 8-dim k-steps, each 64 lanes x 16 bytes)
  __shared__ __attribute__((aligned(16))) uint8_t lds[kF8Slots * kTile8 + 4 * kQLds * 4096];
  __shared__ int32_t pages[kMaxUnitTiles];
  __shared__ int vote[4];

  const int hg = static_cast<int>(blockIdx.x) % head_groups;
  const int ri = static_cast<int>(blockIdx.x) / head_groups;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5;   // which 32-byte half of a k-step (QK), which token quads (P V)
  const int col = lane & 31;  // head (QK^T, A of P V) or dim (B and D of P V)
  const int tps = p.split_tokens / kTile;

  const int64_t total = launch_tiles(p);
  const int64_t s0 = snap(p, ri * total / n_ranges, total, tps);
  const int64_t s1 = snap(p, (ri + 1) * total / n_ranges, total, tps);
  if (s0 >= s1) return;

  const float qk_scale = p.k_scale[0] * p.sm_scale_log2;
  const float o_scale = p.v_scale[0];
  const uint8_t* kpool = static_cast<const uint8_t*>(p.k_pool);
  const uint32_t lds0 = lds_addr(lds);
  const int h_base = hg * 128 + wave * 32;

  // Per-lane LDS offsets in a tile (the swizzles depend on the row modulo
  // 16, so a row 16 or 32 further is a plain add):
  // K of k-step ks < 8, 16-byte half x: row col (+ 32 for the second token
  // half), chunk 4 ks + 2 hh + x, in group ks / 2 at position (4 (ks % 2) +
  // 2 hh + x) ^ f8swz(col); the rope k-step: chunks 32 + 2 hh + x.
  uint32_t koff[2][2], kro[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int x = 0; x < 2; ++x)
      koff[j][x] = static_cast<uint32_t>(128 * col + 16 * ((4 * j + 2 * hh + x) ^ f8swz(col)));
#pragma unroll
  for (int x = 0; x < 2; ++x)
    kro[x] = static_cast<uint32_t>(kF8Rope + 64 * col + 16 * ((2 * hh + x) ^ f8swz4(col)));
  // V of dim block nb (dims 32 nb + col), read x (bytes 8 x .. 8 x + 7 of the
  // operand): the lane pair 2 e, 2 e + 1 of each 16-lane group addresses row
  // 32 (x / 2) + 16 (x % 2) + rv, rv = 8 (e / 4) + 4 hh + e % 4, at chunk 2 nb
  // + a (a = the group's parity: its 16 dims), byte 8 (lane % 2).
  uint32_t voff[4];
  {
    const int e = (lane & 15) >> 1, a = (lane >> 4) & 1;
    const int rv = 8 * (e >> 2) + 4 * hh + (e & 3);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      voff[j] = static_cast<uint32_t>(128 * rv + 16 * ((2 * j + a) ^ f8swz(rv)) + 8 * (lane & 1));
  }
  // Cache loads: wave w fills blocks w + 4 i of a tile, i < 8 the 1 KB
  // block (i % 2) (rows 8 (w + 4 (i % 2)) ..) of group i / 2, i = 8 the rope
  // block w (rows 16 w ..); each lane fetches the chunk its LDS position holds.
  uint32_t goff, groff;
  {
    const int r8 = 8 * (wave & 1) + (lane >> 3);  // the row modulo 16 of a block's lane
    goff = static_cast<uint32_t>((lane >> 3) * kDk + 16 * ((lane & 7) ^ f8swz(r8)));
    groff = static_cast<uint32_t>((16 * wave + (lane >> 2)) * kDk + 16 * (32 + ((lane & 3) ^ ((lane >> 4) & 3))));
  }

  int64_t x = s0;
  while (x < s1) {
    int b, nt;
    int64_t start;
    locate(p, x, b, start, nt);
    const int j0 = static_cast<int>(x - start);
    const int j1 = static_cast<int>(min<int64_t>(nt, s1 - start));
    x = start + j1;
    const int L = p.seq_lens[b];
    const int t_begin = j0 * kTile;
    const int t_end = min(L, j1 * kTile);
    const int n_tiles = j1 - j0;
    const int c0 = j0 / tps;

    // ---- q of this lane's head (dims 64 ks + 32 hh .. + 31 of each k-step),
    // loaded with the first chunk's page ids, so that one wait covers both;
    // it is split into B operands (below) while the first tiles load
    const int32_t* bt = p.block_table + static_cast<int64_t>(b) * p.max_pages;
    uint4 qraw[36];
    {
      const int qi = b * p.num_q_heads + h_base + col;  // < 2^31 (checked on the host)
      const uint16_t* qrow = p.q + static_cast<int64_t>(qi) * kDk + 32 * hh;
#pragma unroll
      for (int ks = 0; ks < 9; ++ks)
#pragma unroll
        for (int c = 0; c < 4; ++c) qraw[4 * ks + c] = *reinterpret_cast<const uint4*>(qrow + 64 * ks + 8 * c);
    }
    auto base_of = [&](int page) __attribute__((always_inline)) {
      if (page < 0 || page >= p.num_pages) page = 0;  // loaded but never used
      return kpool + static_cast<int64_t>(page) * kTile8;
    };
    // the cache loads of tile t (slot t % 4) of `page`: this wave's nine
    auto issue = [&](int t, int page) __attribute__((always_inline)) {
      const uint8_t* base = base_of(page);
      const uint32_t slot = lds0 + (t % kF8Slots) * kTile8;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int kb = wave + 4 * (i & 1);  // block of the group: rows 8 kb ..
        dma16(slot + kF8Group * (i >> 1) + 1024 * kb, goff, base + 8 * kb * kDk + 128 * (i >> 1));
      }
      dma16(slot + kF8Rope + 1024 * wave, groff, base);
    };
    // page ids of a chunk of at most kMaxUnitTiles tiles into LDS, then its
    // first three tiles' loads (every earlier load, q's included, has
    // landed when they are issued, so the waits below count tile loads only)
    auto open_chunk = [&](int k0, int kn) __attribute__((always_inline)) {
      for (int j = tid; j < kn; j += 256) pages[j] = bt[j0 + k0 + j];
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" : : : "memory");
      for (int t = 0; t < kF8Ahead && t < kn; ++t) issue(t, __builtin_amdgcn_readfirstlane(pages[t]));
    };
    open_chunk(0, min(kMaxUnitTiles, n_tiles));

    // q as B operands of the bf16 MFMA: k-step (s, j) takes dims 64 s + 32 hh
    // + 8 j .. + 7, which is qraw[4 s + j]; the last kQLds 64-dim steps go to
    // this lane's slots in LDS (read back only by this lane, after the
    // wave's own writes)
    uint8_t* const qlds = lds + kF8Slots * kTile8 + wave * kQLds * 4096 + 16 * lane;
#pragma unroll
    for (int s = kQReg; s < 9; ++s)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<uint4*>(qlds + (s - kQReg) * 4096 + 1024 * j) = qraw[4 * s + j];

    // O[nb]: rows = this wave's 32 heads (D layout), columns = dims 32 nb + ..
    floatx16_t O[16];
#pragma unroll
    for (int nb = 0; nb < 16; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) O[nb][i] = 0.f;
    // reference max (log2 domain) as in the bf16 wide kernel: set by the
    // segment's first scores, raised (with a redo of the segment) only by a
    // score more than kWideTau above it
    float m = kMInit;
    float l = 0.f;
    bool jump = false;

    bool done = false;
    bool opened = true;  // the first chunk of the first pass is open
    while (!done) {
      for (int k0 = 0; k0 < n_tiles; k0 += kMaxUnitTiles) {
        const int kn = min(kMaxUnitTiles, n_tiles - k0);
        if (!opened) open_chunk(k0, kn);
        opened = false;
        auto page_ahead = [&](int t) __attribute__((always_inline)) { return pages[min(t, kn - 1)]; };
        auto nv_of = [&](int t) __attribute__((always_inline)) {
          return min(kTile, t_end - (t_begin + kTile * (k0 + t)));
        };
        int pv_cur = page_ahead(0);
        int pv_far = page_ahead(kF8Ahead);
        for (int t = 0; t < kn; ++t) {
          const int later = min(kF8Ahead - 1, kn - 1 - t);  // tiles loading behind tile t
          if (later == 2) wait_vm<2 * kDma>();
          else if (later == 1) wait_vm<kDma>();
          else wait_vm<0>();
          const int page = __builtin_amdgcn_readfirstlane(pv_cur);
          const int page_far = __builtin_amdgcn_readfirstlane(pv_far);
          pv_cur = page_ahead(t + 1);
          pv_far = page_ahead(t + 1 + kF8Ahead);
          const int nv = nv_of(t);
          const bool valid = page >= 0 && page < p.num_pages;
          uint8_t* const buf = lds + (t % kF8Slots) * kTile8;
          if (valid && nv < kTile) {
            // rows past the context hold stale codes; V must be finite there
            wg_barrier();
            for (int i = tid; i < 32 * (kTile - nv); i += 256) {
              const int g = i & 3, rem = i >> 2;
              *reinterpret_cast<uint4*>(buf + kF8Group * g + (nv + (rem >> 3)) * 128 + 16 * (rem & 7)) =
                  make_uint4(0u, 0u, 0u, 0u);
            }
          }
          wg_barrier();  // tile t is in LDS; every wave is done with tile t - 1
          if (t + kF8Ahead < kn) issue(t + kF8Ahead, page_far);
          if (!valid) continue;

          // ---- QK^T of token half mb: S = scores of tokens 32 mb .. 32 mb + 31,
          // on the bf16 MFMA with the codes converted (exactly) in registers
          // as they are read: 64-dim step s reads the lane's 32 codes (dims
          // 64 s + 32 hh .. + 31 of its token) and runs four k-steps of 16
          auto qk = [&](int mb) __attribute__((always_inline)) {
            floatx16_t S;
#pragma unroll
            for (int i = 0; i < 16; ++i) S[i] = 0.f;
            auto kread = [&](int s) __attribute__((always_inline)) {
              uint4 k0v, k1v;
              if (s < 8) {
                const uint8_t* gp = buf + kF8Group * (s >> 1) + 4096 * mb;
                k0v = *reinterpret_cast<const uint4*>(gp + koff[s & 1][0]);
                k1v = *reinterpret_cast<const uint4*>(gp + koff[s & 1][1]);
              } else {
                const uint8_t* gp = buf + 2048 * mb;
                k0v = *reinterpret_cast<const uint4*>(gp + kro[0]);
                k1v = *reinterpret_cast<const uint4*>(gp + kro[1]);
              }
              return v8i_t{static_cast<int>(k0v.x), static_cast<int>(k0v.y), static_cast<int>(k0v.z),
                           static_cast<int>(k0v.w), static_cast<int>(k1v.x), static_cast<int>(k1v.y),
                           static_cast<int>(k1v.z), static_cast<int>(k1v.w)};
            };
            v8i_t kq[2] = {kread(0), kread(1)};
#pragma unroll
            for (int s = 0; s < 9; ++s) {
              const v8i_t ka = kq[s & 1];
              if (s + 2 < 9) kq[s & 1] = kread(s + 2);
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const bf16x8_t kb = fp8x8_to_bf16(static_cast<uint32_t>(ka[2 * j]),
                                                  static_cast<uint32_t>(ka[2 * j + 1]));
                const uint4 qw = s < kQReg ? qraw[4 * s + j]
                                           : *reinterpret_cast<const uint4*>(qlds + (s - kQReg) * 4096 + 1024 * j);
                S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb, as_bf16x8(qw.x, qw.y, qw.z, qw.w), S, 0, 0, 0);
              }
            }
            // order: the first two steps' code reads and the LDS q reads, then
            // per step its four MFMAs followed by the code reads of the step
            // two ahead
            __builtin_amdgcn_sched_group_barrier(0x100, 4 + 4 * kQLds, 0);
#pragma unroll
            for (int s = 0; s < 9; ++s) {
              __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
              if (s + 2 < 9) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            return S;
          };

          // ---- numerators of token half mb: 2^(s - m) = p 2^e with p in [0,
          // 2), split into hi and lo codes (words 4 mb .. 4 mb + 3 of the A
          // operands of P V); l += the p times 2^e. Straight-line code (the
          // masking is compiled in or out), so it can interleave with the
          // MFMAs of the other half.
          v8i_t pa_hi, pa_lo;
          int e_half[2];
          auto numerators = [&](floatx16_t S, int mb, auto full_tag) __attribute__((always_inline)) {
            constexpr bool kFull = decltype(full_tag)::value;
            float lm;
            if constexpr (kFull) {
              // the largest scaled score, from the largest (or, for a negative
              // scale, smallest) raw one: rounding is monotonic
              float hi = -INFINITY, lo = INFINITY;
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                hi = fmaxf(hi, S[i]);
                lo = fminf(lo, S[i]);
              }
              lm = (qk_scale >= 0.0f ? hi : lo) * qk_scale;
            } else {
              lm = -INFINITY;
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                const float v = S[i] * qk_scale;
                S[i] = (32 * mb + 8 * (i >> 2) + 4 * hh + (i & 3) < nv) ? v : -INFINITY;
                lm = fmaxf(lm, S[i]);
              }
            }
            lm = max_across_halves(lm);
            const bool first = m == kMInit;
            const bool raise = !first && lm > m + kWideTau;
            jump = jump || raise;
            const float m_first = lm > -INFINITY ? lm : kMInit;
            const float m_next = raise ? lm : m;
            m = first ? m_first : m_next;
            const int e = static_cast<int>(floorf(fmaxf(lm - m, kF8MinExp)));
            e_half[mb] = e;
            const float mm = m + static_cast<float>(e);
            float pr[16];
            float ps = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              pr[i] = __builtin_amdgcn_exp2f(kFull ? __builtin_fmaf(S[i], qk_scale, -mm) : S[i] - mm);
              ps += pr[i];
            }
            l = __builtin_fmaf(ps, pow2f(e), l);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              uint32_t h, o;
              split4(pr[4 * w], pr[4 * w + 1], pr[4 * w + 2], pr[4 * w + 3], h, o);
              pa_hi[4 * mb + w] = static_cast<int>(h);
              pa_lo[4 * mb + w] = static_cast<int>(o);
            }
          };
#pragma unroll
          for (int mb = 0; mb < 2; ++mb) {
            const floatx16_t S = qk(mb);
            if (nv >= kTile) numerators(S, mb, FullTag<true>{});
            else numerators(S, mb, FullTag<false>{});
          }
          // lane col supplies the first half's scale, lane col + 32 the second's
          const int e_mine = hh ? e_half[1] : e_half[0];
          const int sph = 127 + e_mine, spl = 127 + e_mine - 4;

          // ---- O += P V over the tile's 64 tokens, 16 blocks of 32 dims
          auto vread = [&](int nb) __attribute__((always_inline)) {
            const uint8_t* vp = buf + kF8Group * (nb >> 2) + voff[nb & 3];
            v8i_t vb;
#pragma unroll
            for (int xr = 0; xr < 4; ++xr) {
              const v2i_t r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                  (lds_v2i_t*)(vp + 128 * (32 * (xr >> 1) + 16 * (xr & 1))));
              vb[2 * xr] = r[0];
              vb[2 * xr + 1] = r[1];
            }
            return vb;
          };
          v8i_t vq[2] = {vread(0), vread(1)};
#pragma unroll
          for (int nb = 0; nb < 16; ++nb) {
            const v8i_t vb = vq[nb & 1];
            if (nb + 2 < 16) vq[nb & 1] = vread(nb + 2);
            O[nb] = mfma_f8(pa_hi, vb, O[nb], sph, 127);
            O[nb] = mfma_f8(pa_lo, vb, O[nb], spl, 127);
          }
          // order: the first two blocks' V reads, then per block its two
          // MFMAs followed by the reads of the block two ahead
          __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
          for (int nb = 0; nb < 16; ++nb) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            if (nb + 2 < 16) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
          }
        }
        wg_barrier();  // every wave is done with the slots and the page ids
      }
      const bool wave_jump = __builtin_amdgcn_ballot_w64(jump) != 0;
      if (lane == 0) vote[wave] = wave_jump ? 1 : 0;
      wg_barrier();
      done = (vote[0] | vote[1] | vote[2] | vote[3]) == 0;
      if (!done) {
        jump = false;
        l = 0.f;
#pragma unroll
        for (int nb = 0; nb < 16; ++nb)
#pragma unroll
          for (int i = 0; i < 16; ++i) O[nb][i] = 0.f;
      }
      wg_barrier();  // the vote has been read before it is written again
    }

    // ---- the segment's partial in split c0's row (its other splits' rows
    // get lse = -inf): head col's denominator is the sum of lanes col and
    // col + 32; lane (dim col, hh) holds output rows 8 (i / 4) + 4 hh + i % 4
    l += __shfl_xor(l, 32);
    const int64_t bh0 = static_cast<int64_t>(b) * p.num_q_heads + h_base;
    if (hh == 0) {
      const int64_t row = (bh0 + col) * p.max_splits;
      p.lse_part[row + c0] = !(l <= 0.0f) ? (m + __log2f(l)) * kLn2 : -INFINITY;
      const int c_last = (j1 - 1) / tps;
      for (int cx = c0 + 1; cx <= c_last; ++cx) p.lse_part[row + cx] = -INFINITY;
    }
    int64_t head_stride = static_cast<int64_t>(p.max_splits) * kDv;
    asm volatile("" : "+s"(head_stride));
    float* dst0 = p.o_part + (bh0 * p.max_splits + c0) * kDv + col;
    int hq = 4 * hh;
    asm volatile("" : "+v"(hq));
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int hl = 8 * (i >> 2) + hq + (i & 3);
      const float lh = __shfl(l, hl);
      const float f = !(lh <= 0.0f) ? o_scale / lh : 0.0f;
      float* dst = dst0 + hl * head_stride;
#pragma unroll
      for (int nb = 0; nb < 16; ++nb) dst[32 * nb] = O[nb][i] * f;
    }
  }
}

}  // namespace

bool mla_fast_path_supported(int dk, int dv, int num_kv_heads, int num_q_heads, int page_size,
                             int split_tokens) {
  return dk == kDk && dv == kDv && num_kv_heads == 1 && page_size == kTile &&
         num_q_heads % 64 == 0 && num_q_heads <= 1024 && split_tokens <= kMaxUnitTiles * kTile;
}

// Compute units of the current device (looked up once per device).
int cu_count() {
  static int counts[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (counts[dev] <= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    counts[dev] = n;
  }
  return counts[dev];
}

int launch_decode_mla(const DecodeParams& p, bool e4m3, int n_split_blocks, int batch,
                      hipStream_t stream) {
  if (p.num_q_heads % 128 == 0) {
    // one workgroup per compute unit and 128-head group, each an equal share
    // of the launch's tiles
    const int head_groups = p.num_q_heads / 128;
    const int n_ranges = std::max(1, cu_count() / head_groups);
    const dim3 grid(n_ranges * head_groups);
    if (e4m3) {
      decode_mla_f8_kernel<<<grid, 256, 0, stream>>>(p, head_groups, n_ranges);
    } else {
      decode_mla_wide_kernel<<<grid, 256, 0, stream>>>(p, head_groups, n_ranges);
    }
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
