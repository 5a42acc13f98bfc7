// Grouped-query decode over an e4m3 cache with head dim 128, on MFMA.
//
// "Smaller, faster, safer: running Kimi and GLM at scale" (Cloudflare blog),
// section "Quantizing the KV cache": K and V are held as e4m3 and the
// attention kernel converts codes as it reads them.
//
// The G <= 16 query heads of a kv head share every cached K and V row, so
// for 32 cached tokens QK^T is a [32 x 128] x [128 x G] product and PV a
// [G x 32] x [32 x 128] one. Both run on MFMA 16x16x32 with fp32
// accumulation, the G heads padded to 16 rows: QK^T in bf16 (the query is
// bf16; K codes convert exactly), PV in f16 (V codes convert exactly;
// numerators rounded to f16). The VALU keeps only the exact converts and the
// softmax, a fifth of the instructions of a dot-product design.
//
// One wave per work unit (request, kv head, split), in the one-dimensional
// longest-first order of find_unit. A split runs in tiles of 32 tokens whose
// K and V bytes (4 KB each) travel HBM -> LDS by direct-to-LDS loads into a
// ring of kSlots tiles.
//
// MFMA 16x16x32 operand layouts (lane l, c = l % 16, q = l / 16):
//   A: row c, k 8q .. 8q+7;  B: column c, k 8q .. 8q+7;
//   D element i: row 4q + i, column c.
// QK^T runs transposed, S^T = K Q^T (M = 16 tokens, N = 16 heads), with the
// contraction order permuted so that a lane's K operand is one 32-byte run
// of its token row: in k-step s, slot 8q + j is dim 32q + 8s + j. A lane then
// holds head c's scores for tokens 4q .. 4q+3 of each 16-token half of the
// tile, which is already the A operand of O += P V (M = heads, 32 tokens of
// contraction; slot 8q + e is token 4q + e of the first half for e < 4 and
// token 4q + e - 4 of the second half otherwise) once V is read in that
// token order with ds_read_tr8_b64: lane i of a 16-lane group gets byte i of
// the 8 rows the group's lane pairs address.
//
// Softmax: log2 domain, per head a reference max set by the first tile with
// a valid token, so the accumulators never need a rescale and stay in the
// MFMA's own registers. A later score more than kTau above it raises it and
// restarts the unit from its first tile (a uniform branch real scores
// almost never take); the f16 numerators thus stay at most 2^kTau.
#include "common.h"
#include "decode_params.h"
#include "mfma_tile.h"
#include "unit_order.h"

namespace {

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTau = 15.0f;      // f16 numerators stay at most 2^kTau
constexpr float kMUnset = -1e30f;  // reference max before the first valid score
constexpr int kD = 128;
constexpr int kRows = 16;              // query heads per MFMA tile (G padded)
constexpr int kTile = 32;              // tokens per tile
constexpr int kHalf = kTile * kD;      // K (or V) bytes of a tile
constexpr int kTileBytes = 2 * kHalf;  // K then V: 8 KB
constexpr int kPageVecs = 4;                  // page offsets per lane
constexpr int kMaxUnitPages = 64 * kPageVecs;

// LDS layouts, 64 banks of 4 bytes (bank = 32 (row & 1) + 4 chunk position
// for 128-byte rows). K chunk c of tile row t sits at c ^ kswz(t): the 16
// rows one 16-lane phase of a K read touches at one chunk fall on distinct
// banks. V chunk c of row t sits at c ^ vswz(t), vswz(t) = bits 1, 2 and 4
// of t: the 16 rows of a half-wave's transposing read at one chunk, likewise.
__device__ __forceinline__ uint32_t kswz(uint32_t t) { return (t >> 1) & 7u; }
__device__ __forceinline__ uint32_t vswz(uint32_t t) {
  return ((t >> 1) & 3u) | (((t >> 4) & 1u) << 2);
}

// one of four values by a wave-uniform index (values, not addresses, so the
// four stay in registers)
template <typename T>
__device__ __forceinline__ T pick4(int h, T a, T b, T c, T d) {
  return h == 0 ? a : h == 1 ? b : h == 2 ? c : d;
}

template <int N>
__device__ __forceinline__ void wait_tiles(int ahead) {
  // every tile is 8 loads; wait until only the `ahead` younger tiles remain
  if (N >= 3 && ahead >= 3) {
    wait_vm<24>();
  } else if (N >= 2 && ahead >= 2) {
    wait_vm<16>();
  } else if (ahead >= 1) {
    wait_vm<8>();
  } else {
    wait_vm<0>();
  }
}

template <int kSlots>
__global__ void __launch_bounds__(64) decode_gqa_mfma_kernel(DecodeParams p) {
  static_assert(kSlots >= 2 && kSlots <= 4, "ring of 2 to 4 tiles");
  __shared__ __attribute__((aligned(16))) uint8_t ring[kSlots * kTileBytes];
  __shared__ float rowbuf[kRows];
  const int lane = threadIdx.x;
  const int col = lane & 15, qg = lane >> 4;
  int b, g, c, L;
  if (!pkv::find_unit(p, static_cast<int>(blockIdx.x), b, g, c, L)) return;
  const int G = p.num_q_heads / p.num_kv_heads;
  const int t_begin = c * p.split_tokens;
  const int t_end = min(L, t_begin + p.split_tokens);
  const int n_tiles = (t_end - t_begin + kTile - 1) / kTile;
  const int P = p.page_size;
  const int log2P = P == 16 ? 4 : (P == 32 ? 5 : 6);

  // query head col as B operands (heads G .. 15 are zero rows): k-step s,
  // slot 8 qg + j <-> dim 32 qg + 8 s + j
  const bool head_ok = col < G;
  bf16x8_t qf[4];
  {
    const uint16_t* qrow =
        p.q + (static_cast<int64_t>(b) * p.num_q_heads + g * G + (head_ok ? col : 0)) * kD +
        32 * qg;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (head_ok) {
        qf[s] = *reinterpret_cast<const bf16x8_t*>(qrow + 8 * s);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[s][e] = static_cast<__bf16>(0.0f);
      }
    }
  }
  const float qk_scale = p.k_scale[g] * p.sm_scale_log2;
  const float o_scale = p.v_scale[g];

  // the unit's pages: lane j holds the byte offsets of (page 64 h + j, kv
  // head g) in vector h < kPageVecs (named variables, so that selecting one
  // by a uniform index stays in registers)
  const int32_t* bt = p.block_table + static_cast<int64_t>(b) * p.max_pages;
  const int first_page = t_begin >> log2P;
  const int n_pages = (t_end - t_begin + P - 1) >> log2P;
  auto load_page = [&](int h) __attribute__((always_inline)) {
    return 64 * h + lane < n_pages ? bt[first_page + 64 * h + lane] : -1;
  };
  const int pg0 = load_page(0), pg1 = load_page(1), pg2 = load_page(2), pg3 = load_page(3);
#pragma unroll
  for (int s = 0; s < 4; ++s) asm volatile("" : : "v"(qf[s]));
  asm volatile("" : : "v"(pg0), "v"(pg1), "v"(pg2), "v"(pg3));
  asm volatile("" : : "v"(qk_scale), "v"(o_scale));
  // from here on the only vector memory loads in flight are the ring's
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" : : : "memory");
  auto page_ok_lane = [&](int pg) __attribute__((always_inline)) {
    return pg >= 0 && pg < p.num_pages;
  };
  auto page_off = [&](int pg) __attribute__((always_inline)) {
    return (static_cast<int64_t>(page_ok_lane(pg) ? pg : 0) * p.num_kv_heads + g) *
           (static_cast<int64_t>(P) * kD);
  };
  const uint64_t valid0 = __ballot(page_ok_lane(pg0)), valid1 = __ballot(page_ok_lane(pg1)),
                 valid2 = __ballot(page_ok_lane(pg2)), valid3 = __ballot(page_ok_lane(pg3));
  const int64_t off0 = page_off(pg0), off1 = page_off(pg1), off2 = page_off(pg2),
                off3 = page_off(pg3);
  static_assert(kPageVecs == 4, "four named page vectors");
  auto page_ok = [&](int j) __attribute__((always_inline)) {
    const int h = j >> 6;
    const uint64_t v = pick4(h, valid0, valid1, valid2, valid3);
    return ((v >> (j & 63)) & 1u) != 0;
  };

  // DMA source offsets inside a 16-token group block: lane L fills LDS chunk
  // position L & 7 of group row L >> 3 (first 1 KB) and of row 8 + (L >> 3)
  // (second 1 KB); position pos of tile row t holds chunk pos ^ swz(t)
  const uint32_t dr0 = lane >> 3, dr1 = 8 + (lane >> 3), dpos = lane & 7;
  const uint32_t koff0 = dr0 * kD + ((dpos ^ kswz(dr0)) << 4);
  const uint32_t koff1 = dr1 * kD + ((dpos ^ kswz(dr1)) << 4);
  uint32_t voffd[2][2];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    voffd[x][0] = dr0 * kD + ((dpos ^ vswz(16 * x + dr0)) << 4);
    voffd[x][1] = dr1 * kD + ((dpos ^ vswz(16 * x + dr1)) << 4);
  }
  const uint8_t* kpool = static_cast<const uint8_t*>(p.k_pool);
  const uint8_t* vpool = static_cast<const uint8_t*>(p.v_pool);
  const uint32_t ring0 = lds_addr(ring);

  auto group_base = [&](int gg) __attribute__((always_inline)) {
    const int j = (gg << 4) >> log2P;
    const int h = j >> 6, jl = j & 63;
    const int64_t o = pick4(h, off0, off1, off2, off3);
    const uint64_t off =
        (static_cast<uint64_t>(static_cast<uint32_t>(
             __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint64_t>(o) >> 32), jl)))
         << 32) |
        static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(o), jl));
    return off + static_cast<uint32_t>(((gg << 4) & (P - 1)) * kD);
  };
  // 8 loads per tile, always: a 16-token group past the unit's end loads the
  // tile's first group again (its scores are masked and its V rows zeroed)
  auto issue = [&](int t) __attribute__((always_inline)) {
    const uint32_t slot = ring0 + (t % kSlots) * kTileBytes;
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int gg = (t_begin + kTile * t + 16 * x < t_end) ? 2 * t + x : 2 * t;
      const uint64_t off = group_base(gg);
      dma16(slot + 2048 * x, koff0, kpool + off);
      dma16(slot + 2048 * x + 1024, koff1, kpool + off);
      dma16(slot + kHalf + 2048 * x, voffd[x][0], vpool + off);
      dma16(slot + kHalf + 2048 * x + 1024, voffd[x][1], vpool + off);
    }
  };

  // LDS read offsets. K operand of half x, read r: chunk 2 qg + r (dims
  // 32 qg + 16 r ..) of tile row 16 x + col. V operand of dim block nb: lane
  // pair 2e, 2e+1 of a 16-lane group addresses the halves of chunk nb of row
  // tv(e), the e-th token of the group's contraction slots.
  uint32_t koffr[2][2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const uint32_t row = 16 * x + col;
      koffr[x][r] = row * kD + ((static_cast<uint32_t>(2 * qg + r) ^ kswz(row)) << 4);
    }
  const int e_row = (lane & 15) >> 1;
  const uint32_t tv = e_row < 4 ? 4 * qg + e_row : 16 + 4 * qg + (e_row - 4);
  uint32_t voffr[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb)
    voffr[nb] = kHalf + tv * kD + ((static_cast<uint32_t>(nb) ^ vswz(tv)) << 4) + 8 * (lane & 1);

  floatx4_t O[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i) O[nb][i] = 0.0f;
  float m = kMUnset;  // reference max of head col (its four lanes agree)
  float l = 0.0f;     // this lane's part of head col's denominator

  auto prime = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < kSlots - 1; ++k)
      if (k < n_tiles) issue(k);
  };
  prime();
  for (int t = 0; t < n_tiles; ++t) {
    if (t + kSlots - 1 < n_tiles) issue(t + kSlots - 1);
    wait_tiles<kSlots - 1>(min(kSlots - 1, n_tiles - 1 - t));
    uint8_t* buf = ring + (t % kSlots) * kTileBytes;
    const int tile0 = t_begin + kTile * t;
    // rows past the unit or of a page outside the pool: V to zero (their
    // scores are masked, and 0 * NaN must not reach the accumulators)
    const bool g0_ok = page_ok(((2 * t) << 4) >> log2P);
    const bool g1_ok = tile0 + 16 < t_end && page_ok(((2 * t + 1) << 4) >> log2P);
    const int nv = min(kTile, t_end - tile0);
    const bool full = g0_ok && g1_ok && nv == kTile;
    if (!full) {
      for (int q = lane; q < kTile * (kD / 16); q += 64) {
        const int row = q >> 3;
        const bool keep = row < nv && (row < 16 ? g0_ok : g1_ok);
        if (!keep) *reinterpret_cast<uint4*>(buf + kHalf + 16 * q) = make_uint4(0u, 0u, 0u, 0u);
      }
      __builtin_amdgcn_wave_barrier();
    }

    // ---- S^T = K Q^T, one 16-token half at a time
    floatx4_t s[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
#pragma unroll
      for (int i = 0; i < 4; ++i) s[x][i] = 0.0f;
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const uint4 kq = *reinterpret_cast<const uint4*>(buf + koffr[x][r]);
        s[x] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16(kq.x, kq.y), qf[2 * r],
                                                       s[x], 0, 0, 0);
        s[x] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16(kq.z, kq.w), qf[2 * r + 1],
                                                       s[x], 0, 0, 0);
      }
    }
    // s[x][i]: head col, token tile0 + 16 x + 4 qg + i
    float tmax = -INFINITY;
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = s[x][i] * qk_scale;
        if (!full) {
          const int tt = 16 * x + 4 * qg + i;
          v = (tt < nv && (x == 0 ? g0_ok : g1_ok)) ? v : -INFINITY;
        }
        s[x][i] = v;
        tmax = fmaxf(tmax, v);
      }
    // every head has its first valid score in the same tile, so m is unset
    // in all lanes or in none
    if (m == kMUnset) {
      float hm = fmaxf(tmax, __shfl_xor(tmax, 16));
      hm = fmaxf(hm, __shfl_xor(hm, 32));
      if (hm > -INFINITY) m = hm;
    }
    if (__any(tmax > m + kTau)) {
      // rare: raise the reference max of the heads that need it and start
      // the unit again (m only grows, each time to a score of the unit, so
      // this ends); the ring is drained and primed afresh
      float hm = fmaxf(tmax, __shfl_xor(tmax, 16));
      hm = fmaxf(hm, __shfl_xor(hm, 32));
      m = hm > m + kTau ? hm : m;
      wait_vm<0>();
#pragma unroll
      for (int nb = 0; nb < 8; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) O[nb][i] = 0.0f;
      l = 0.0f;
      __builtin_amdgcn_wave_barrier();
      prime();
      t = -1;
      continue;
    }

    // ---- O += P V over the 32 tokens, 8 blocks of 16 dims
    f16x8_t pf;
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pr = __builtin_amdgcn_exp2f(s[x][i] - m);
        l += pr;
        pf[4 * x + i] = static_cast<_Float16>(pr);
      }
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const v2i_t r8 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_t*)(buf + voffr[nb]));
      O[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
          pf, fp8x8_to_f16(static_cast<uint32_t>(r8[0]), static_cast<uint32_t>(r8[1])), O[nb], 0,
          0, 0);
    }
    __builtin_amdgcn_wave_barrier();
  }

  // ---- finish: per head, o / l and lse = m + log2 l (natural-log units)
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (qg == 0) rowbuf[col] = l;
  __builtin_amdgcn_wave_barrier();
  const int64_t head0 = static_cast<int64_t>(b) * p.num_q_heads + g * G;
  if (qg == 0 && head_ok)
    p.lse_part[(head0 + col) * p.max_splits + c] = l > 0.0f ? (m + __log2f(l)) * kLn2 : -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * qg + i;
    if (h >= G) continue;
    const float lr = rowbuf[h];
    const float f = lr > 0.0f ? o_scale / lr : 0.0f;
    float* dst = p.o_part + ((head0 + h) * p.max_splits + c) * kD + col;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) dst[16 * nb] = O[nb][i] * f;
  }
}

}  // namespace

bool gqa_mfma_path_supported(int dk, int dv, int group, bool latent, int split_tokens,
                             int page_size) {
  return !latent && dk == kD && dv == kD && group >= 1 && group <= kRows &&
         split_tokens <= kMaxUnitPages * page_size;
}

int launch_decode_gqa_mfma(const DecodeParams& p, int n_split_blocks, int batch,
                           hipStream_t stream) {
  const int64_t units = static_cast<int64_t>(n_split_blocks) * p.num_kv_heads * batch;
  if (units > 0x7FFFFFFF) return PKV_EUNSUPPORTED;
  decode_gqa_mfma_kernel<2><<<dim3(static_cast<uint32_t>(units)), 64, 0, stream>>>(p);
  return pkv::launch_status();
}
