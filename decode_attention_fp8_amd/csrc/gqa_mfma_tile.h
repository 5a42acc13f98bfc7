// One 32-token tile of grouped-query decode on MFMA 16x16x32 (internal),
// the tile math of the e4m3 grouped-query kernel.
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
// softmax.
//
// A tile's K and V bytes (4 KB each, two 16-token groups of each) sit in an
// 8 KB LDS slot, written by direct-to-LDS loads.
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
// a valid token; a later score more than kTau above it raises it and
// rescales the head's accumulators (a uniform branch real scores almost
// never take), so the f16 numerators stay at most 2^kTau.
#pragma once

#include "decode_params.h"
#include "mfma_tile.h"

namespace gqa_mfma {

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTau = 15.0f;      // f16 numerators stay at most 2^kTau
constexpr float kMUnset = -1e30f;  // reference max before the first valid score
constexpr int kD = 128;
constexpr int kRows = 16;              // query heads per MFMA tile (G padded)
constexpr int kTile = 32;              // tokens per tile
constexpr int kHalf = kTile * kD;      // K (or V) bytes of a tile
constexpr int kTileBytes = 2 * kHalf;  // K then V: 8 KB

// LDS layouts, 64 banks of 4 bytes (bank = 32 (row & 1) + 4 chunk position
// for 128-byte rows). K chunk c of tile row t sits at c ^ kswz(t): the 16
// rows one 16-lane phase of a K read touches at one chunk fall on distinct
// banks. V chunk c of row t sits at c ^ vswz(t), vswz(t) = bits 1, 2 and 4
// of t: the 16 rows of a half-wave's transposing read at one chunk, likewise.
__device__ __forceinline__ uint32_t kswz(uint32_t t) { return (t >> 1) & 7u; }
__device__ __forceinline__ uint32_t vswz(uint32_t t) {
  return ((t >> 1) & 3u) | (((t >> 4) & 1u) << 2);
}

// Per-lane byte offsets, fixed for the whole kernel.
struct LaneOffsets {
  // DMA sources inside a 16-token group block: lane L fills LDS chunk
  // position L & 7 of group row L >> 3 (first 1 KB) and of row 8 + (L >> 3)
  // (second 1 KB); position pos of tile row t holds chunk pos ^ swz(t)
  uint32_t kdma0, kdma1;
  uint32_t vdma[2][2];  // [half of the tile][first / second 1 KB]
  // LDS reads: K operand of half x, read r = chunk 2 qg + r (dims
  // 32 qg + 16 r ..) of tile row 16 x + col; V operand of dim block nb =
  // halves of chunk nb of row tv(e) for lane pair 2e, 2e+1 of a group
  uint32_t kread[2][2];
  uint32_t vread[8];
};

__device__ __forceinline__ LaneOffsets lane_offsets(int lane) {
  LaneOffsets o;
  const int col = lane & 15, qg = lane >> 4;
  const uint32_t dr0 = lane >> 3, dr1 = 8 + (lane >> 3), dpos = lane & 7;
  o.kdma0 = dr0 * kD + ((dpos ^ kswz(dr0)) << 4);
  o.kdma1 = dr1 * kD + ((dpos ^ kswz(dr1)) << 4);
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    o.vdma[x][0] = dr0 * kD + ((dpos ^ vswz(16 * x + dr0)) << 4);
    o.vdma[x][1] = dr1 * kD + ((dpos ^ vswz(16 * x + dr1)) << 4);
  }
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const uint32_t row = 16 * x + col;
      o.kread[x][r] = row * kD + ((static_cast<uint32_t>(2 * qg + r) ^ kswz(row)) << 4);
    }
  const int e_row = (lane & 15) >> 1;
  const uint32_t tv = e_row < 4 ? 4 * qg + e_row : 16 + 4 * qg + (e_row - 4);
#pragma unroll
  for (int nb = 0; nb < 8; ++nb)
    o.vread[nb] =
        kHalf + tv * kD + ((static_cast<uint32_t>(nb) ^ vswz(tv)) << 4) + 8 * (lane & 1);
  return o;
}

// DMA of one 16-token group (K and V, 2 KB each) into half x of a slot, in
// the non-temporal form: a step reads each cache byte once, and the next
// step of the same layer comes after the model's other layers, so keeping
// the lines would only evict others.
__device__ __forceinline__ void dma_group(uint32_t slot, int x, const LaneOffsets& o,
                                          const uint8_t* kgroup, const uint8_t* vgroup) {
  dma16_stream(slot + 2048 * x, o.kdma0, kgroup);
  dma16_stream(slot + 2048 * x + 1024, o.kdma1, kgroup);
  dma16_stream(slot + kHalf + 2048 * x, o.vdma[x][0], vgroup);
  dma16_stream(slot + kHalf + 2048 * x + 1024, o.vdma[x][1], vgroup);
}

struct Acc {
  floatx4_t O[8];  // head 4 qg + i, dim 16 nb + col
  float m;         // reference max of head col (its four lanes agree)
  float l;         // this lane's part of head col's denominator
  // scales set at append: O holds sum p * code * (v_scale / vref), vref a
  // power of two at or above every V row scale seen so far (0 = none yet),
  // so that f16 numerators p * v_scale / vref stay at most 2^kTau
  float vref;
};

__device__ __forceinline__ void acc_init(Acc& a) {
#pragma unroll
  for (int nb = 0; nb < 8; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i) a.O[nb][i] = 0.0f;
  a.m = kMUnset;
  a.l = 0.0f;
  a.vref = 0.0f;
}

// Smallest power of two at or above a positive float (2^-126 for any
// subnormal; infinity above 2^127).
__device__ __forceinline__ float pow2_at_or_above(float x) {
  return __uint_as_float((__float_as_uint(x) + 0x7FFFFFu) & 0xFF800000u);
}

// QK^T, softmax and PV of the tile in buf. Group x of the tile holds valid
// rows only if gx_ok (its page is in the pool); of the tile's 32 rows the
// first nv are in the unit. kRowScales: the tile's
// rows carry their own scales (set at append), in LDS at rs[t] (K) and
// rs[64 + t] (V) for tile row t; a score is multiplied by its row's K scale
// and a numerator by its row's V scale over the unit's V reference a.vref
// before PV (the denominator takes the unscaled numerator), masked rows
// contributing nothing.
template <bool kRowScales>
__device__ __forceinline__ void tile_math(uint8_t* buf, const LaneOffsets& o,
                                          const bf16x8_t (&qf)[4], float qk_scale, bool g0_ok,
                                          bool g1_ok, int nv, Acc& a,
                                          const float* rs = nullptr) {
  const int lane = threadIdx.x;
  const int qg = lane >> 4;
  const bool full = g0_ok && g1_ok && nv == kTile;
  if (!full) {
    // rows past the unit or of a page outside the pool: V to zero (their
    // scores are masked, and 0 * NaN must not reach the accumulators)
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
      const uint4 kq = *reinterpret_cast<const uint4*>(buf + o.kread[x][r]);
      s[x] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16(kq.x, kq.y), qf[2 * r], s[x],
                                                     0, 0, 0);
      s[x] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16(kq.z, kq.w), qf[2 * r + 1],
                                                     s[x], 0, 0, 0);
    }
  }
  // s[x][i]: head col, tile row 16 x + 4 qg + i
  float4 ks[2], vs[2];
  if constexpr (kRowScales) {
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      ks[x] = *reinterpret_cast<const float4*>(rs + 16 * x + 4 * qg);
      vs[x] = *reinterpret_cast<const float4*>(rs + 64 + 16 * x + 4 * qg);
    }
  }
  float tmax = -INFINITY;
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = s[x][i] * qk_scale;
      if constexpr (kRowScales) v *= (&ks[x].x)[i];
      if (!full) {
        const int tt = 16 * x + 4 * qg + i;
        v = (tt < nv && (x == 0 ? g0_ok : g1_ok)) ? v : -INFINITY;
      }
      s[x][i] = v;
      tmax = fmaxf(tmax, v);
    }
  // every head has its first valid score in the same tile, so m is unset
  // in all lanes or in none
  if (a.m == kMUnset) {
    float hm = fmaxf(tmax, __shfl_xor(tmax, 16));
    hm = fmaxf(hm, __shfl_xor(hm, 32));
    if (hm > -INFINITY) a.m = hm;
  }
  if (__any(tmax > a.m + kTau)) {
    // rare: raise the reference max of the heads that need it, rescale
    float hm = fmaxf(tmax, __shfl_xor(tmax, 16));
    hm = fmaxf(hm, __shfl_xor(hm, 32));
    const float mn = hm > a.m + kTau ? hm : a.m;
    const float al = __builtin_amdgcn_exp2f(a.m - mn);
    a.m = mn;
    a.l *= al;
    // the four lanes of a head hold the same factor; lane h (< 16) holds
    // head h's
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float f = __shfl(al, 4 * qg + i);
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) a.O[nb][i] *= f;
    }
  }

  float vinv = 1.0f;
  if constexpr (kRowScales) {
    // V row scales relative to vref: a tile with a larger scale (always the
    // unit's first valid tile) raises vref and rescales O in a uniform
    // branch. A masked row's scale may be unwritten and takes no part.
    bool up = false;
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int i = 0; i < 4; ++i) up |= s[x][i] != -INFINITY && (&vs[x].x)[i] > a.vref;
    if (__any(up)) {
      float vm = 0.0f;
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (s[x][i] != -INFINITY) vm = fmaxf(vm, (&vs[x].x)[i]);
      vm = fmaxf(vm, __shfl_xor(vm, 16));
      vm = fmaxf(vm, __shfl_xor(vm, 32));
      const float nref = pow2_at_or_above(vm);
      const float f = a.vref / nref;  // 0 before the first valid tile: O is 0
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) a.O[nb] *= f;
      a.vref = nref;
    }
    // 1 / vref, exact for a power of two in [2^-126, 2^126]
    vinv = __uint_as_float(0x7F000000u - __float_as_uint(a.vref));
  }

  // ---- O += P V over the 32 tokens, 8 blocks of 16 dims
  f16x8_t pf;
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pr = __builtin_amdgcn_exp2f(s[x][i] - a.m);
      a.l += pr;
      if constexpr (kRowScales) {
        // a masked row's scale may be unwritten: its numerator stays 0
        pf[4 * x + i] = static_cast<_Float16>(
            s[x][i] == -INFINITY ? 0.0f : pr * ((&vs[x].x)[i] * vinv));
      } else {
        pf[4 * x + i] = static_cast<_Float16>(pr);
      }
    }
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
    const v2i_t r8 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_t*)(buf + o.vread[nb]));
    a.O[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
        pf, fp8x8_to_f16(static_cast<uint32_t>(r8[0]), static_cast<uint32_t>(r8[1])), a.O[nb], 0,
        0, 0);
  }
  __builtin_amdgcn_wave_barrier();
}

// ---------------------------------------------------------------------------
// bf16 cache: the same tile and operand layouts with two bytes per value, no
// conversion. A tile's K and V are 8 KB each (16 KB per slot); a 16-token
// group is 4 KB of K and 4 KB of V, four direct-to-LDS loads each.
//
// LDS rows are 256 bytes, 16 chunks of 16 bytes; 64 banks of 4 bytes cover
// one row, chunk position p taking banks 4p .. 4p+3. K chunk c of tile row t
// sits at c ^ (t & 15): the 8 rows of one pass of a 16-byte read (lanes
// 8k .. 8k+7, rows 8(k%2) .. +7 at one chunk) fall on distinct banks. V
// chunk c of row t sits at c ^ 2(t & 3): one pass of a transposing read
// (16 lanes: 4 rows x the two chunks of 16 dims) covers 8 distinct
// positions.
namespace bf16c {

constexpr int kHalf = kTile * kD * 2;  // K (or V) bytes of a tile
constexpr int kTileBytes = 2 * kHalf;  // K then V: 16 KB

__device__ __forceinline__ uint32_t kswz(uint32_t t) { return t & 15u; }
__device__ __forceinline__ uint32_t vswz(uint32_t t) { return (t & 3u) << 1; }

struct LaneOffsets {
  // DMA sources inside a 16-token group block: load i fills group rows
  // 4i + (lane >> 4), chunk position lane & 15 (the swizzles depend only on
  // the row within its group, so both halves of a tile share them)
  uint32_t kdma[4], vdma[4];
  // K operand of half x, k-step s: chunk 4 qg + s (dims 32 qg + 8 s ..) of
  // tile row 16 x + col
  uint32_t kread[2][4];
  // V operand of dim block nb: transposing reads of rows 4 qg + e and
  // 16 + 4 qg + e (e = (lane & 15) >> 2), 8 bytes at chunk 2 nb + (i >> 1),
  // byte 8 (i & 1) (i = lane & 3): the 16 dims 16 nb .. 16 nb + 15
  uint32_t vread[8][2];
};

__device__ __forceinline__ LaneOffsets lane_offsets(int lane) {
  LaneOffsets o;
  const int col = lane & 15, qg = lane >> 4;
  const uint32_t pos = lane & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t r = 4 * i + (lane >> 4);
    o.kdma[i] = r * 2 * kD + ((pos ^ kswz(r)) << 4);
    o.vdma[i] = r * 2 * kD + ((pos ^ vswz(r)) << 4);
  }
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const uint32_t row = 16 * x + col;
      o.kread[x][st] = row * 2 * kD + ((static_cast<uint32_t>(4 * qg + st) ^ kswz(row)) << 4);
    }
  const uint32_t e = (lane & 15) >> 2, i = lane & 3;
#pragma unroll
  for (int nb = 0; nb < 8; ++nb)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t row = 16 * h + 4 * qg + e;
      const uint32_t c = 2 * nb + (i >> 1);
      o.vread[nb][h] = kHalf + row * 2 * kD + ((c ^ vswz(row)) << 4) + 8 * (i & 1);
    }
  return o;
}

// DMA of one 16-token group (K and V, 4 KB each) into half x of a slot
// (non-temporal, as above)
__device__ __forceinline__ void dma_group(uint32_t slot, int x, const LaneOffsets& o,
                                          const uint8_t* kgroup, const uint8_t* vgroup) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    dma16_stream(slot + 4096 * x + 1024 * i, o.kdma[i], kgroup);
    dma16_stream(slot + kHalf + 4096 * x + 1024 * i, o.vdma[i], vgroup);
  }
}

// QK^T, softmax and PV of the tile in buf (as tile_math, bf16 values): the
// numerators are rounded to bf16 for PV, and the rounded values are what the
// denominator sums, so the weights are normalised exactly as used.
__device__ __forceinline__ void tile_math(uint8_t* buf, const LaneOffsets& o,
                                          const bf16x8_t (&qf)[4], float qk_scale, bool g0_ok,
                                          bool g1_ok, int nv, Acc& a) {
  const int lane = threadIdx.x;
  const int qg = lane >> 4;
  const bool full = g0_ok && g1_ok && nv == kTile;
  if (!full) {
    // V rows past the unit or of a page outside the pool: zero (their
    // scores are masked, and 0 * NaN must not reach the accumulators)
    for (int q = lane; q < kTile * 16; q += 64) {
      const int row = q >> 4;
      const bool keep = row < nv && (row < 16 ? g0_ok : g1_ok);
      if (!keep) *reinterpret_cast<uint4*>(buf + kHalf + 16 * q) = make_uint4(0u, 0u, 0u, 0u);
    }
    __builtin_amdgcn_wave_barrier();
  }

  floatx4_t s[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
#pragma unroll
    for (int i = 0; i < 4; ++i) s[x][i] = 0.0f;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const uint4 kq = *reinterpret_cast<const uint4*>(buf + o.kread[x][st]);
      s[x] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kq), qf[st], s[x], 0, 0, 0);
    }
  }
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
  if (a.m == kMUnset) {
    float hm = fmaxf(tmax, __shfl_xor(tmax, 16));
    hm = fmaxf(hm, __shfl_xor(hm, 32));
    if (hm > -INFINITY) a.m = hm;
  }
  if (__any(tmax > a.m + kTau)) {
    float hm = fmaxf(tmax, __shfl_xor(tmax, 16));
    hm = fmaxf(hm, __shfl_xor(hm, 32));
    const float mn = hm > a.m + kTau ? hm : a.m;
    const float al = __builtin_amdgcn_exp2f(a.m - mn);
    a.m = mn;
    a.l *= al;
    // the four lanes of a head hold the same factor; lane h (< 16) holds
    // head h's
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float f = __shfl(al, 4 * qg + i);
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) a.O[nb][i] *= f;
    }
  }

  bf16x8_t pf;
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const __bf16 pb = static_cast<__bf16>(__builtin_amdgcn_exp2f(s[x][i] - a.m));
      pf[4 * x + i] = pb;
      a.l += static_cast<float>(pb);
    }
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
    const v4s_t r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t*)(buf + o.vread[nb][0]));
    const v4s_t r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t*)(buf + o.vread[nb][1]));
    a.O[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf, join_bf16x4(r0, r1), a.O[nb], 0, 0, 0);
  }
  __builtin_amdgcn_wave_barrier();
}

}  // namespace bf16c

// The unit's partials: per query head g G + h (h < G) of request b, split c,
// o = v_scale O / l and lse = (m + log2 l) ln 2 (o = 0, lse = -inf where no
// token was valid).
__device__ __forceinline__ void finish(const DecodeParams& p, int b, int g, int c, int G,
                                       float o_scale, Acc& a) {
  const int lane = threadIdx.x;
  const int col = lane & 15, qg = lane >> 4;
  float l = a.l;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  const int64_t head0 = static_cast<int64_t>(b) * p.num_q_heads + g * G;
  if (qg == 0 && col < G)
    p.lse_part[(head0 + col) * p.max_splits + c] =
        !(l <= 0.0f) ? (a.m + __log2f(l)) * kLn2 : -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * qg + i;
    const float lr = __shfl(l, h);  // lane h (< 16) holds head h's
    if (h >= G) continue;
    const float f = !(lr <= 0.0f) ? o_scale / lr : 0.0f;
    float* dst = p.o_part + ((head0 + h) * p.max_splits + c) * kD + col;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) dst[16 * nb] = a.O[nb][i] * f;
  }
  __builtin_amdgcn_wave_barrier();
}

// one of four values by a wave-uniform index (values, not addresses, so the
// four stay in registers)
template <typename T>
__device__ __forceinline__ T pick4(int h, T a, T b, T c, T d) {
  return h == 0 ? a : h == 1 ? b : h == 2 ? c : d;
}

}  // namespace gqa_mfma
