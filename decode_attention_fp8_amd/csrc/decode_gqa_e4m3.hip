// Grouped-query decode kernel for an e4m3 cache, head dim 128, 8 query heads
// per kv head (the production shape).
//
// "Smaller, faster, safer", section "Quantizing the KV cache": the FP8
// kernel converts cached values as it reads them. Here the conversion is
// gfx950's packed e4m3 -> bf16 / f16 convert (two exact codes per
// instruction) and the arithmetic is packed two-term dot products with fp32
// accumulation. Decode at 8 query heads per kv head does 16 flop per cached
// byte, so the vector ALU, not HBM, is what this kernel has to economise.
//
// One wave per work unit (request b, kv head g, split c), processed in groups
// of 16 tokens. A group's K and V bytes (2 KB each) travel HBM -> LDS by
// direct-to-LDS loads into a ring of kSlots group buffers; a group's bytes
// are copied into registers as soon as they land, so its slot is refilled at
// once and kSlots groups stay in flight while one is computed.
//
// Lane (r = lane >> 4, i = lane & 15). The four 16-lane rows split the head
// dimension: row r owns dims [32r, 32r + 32) in QK^T and dims 32r + i and
// 32r + 16 + i in PV.
//
// QK^T. Lane i of a row takes token tok(i) = 2(i & 7) + (i >> 3) of the group
// and reads its 32 dims of that token's K row. The query is not replicated:
// register qd[h] of lane i holds the bf16 pair (32r + 2i, 32r + 2i + 1) of
// head h, and every dot product takes its query operand through the DPP
// row_newbcast modifier, which hands lane m's value to the whole row at no
// extra cost. The four row partials are summed by a reduce-scatter with
// permlane32 / permlane16 swaps, after which row r holds the scores of heads
// 2r and 2r + 1 for the 16 tokens.
//
// Softmax. Scores are kept in the log2 domain relative to a reference max
// m per head, the largest score of the first group that has a valid token.
// The accumulators are rescaled only when a later score exceeds m by more
// than kTau (a uniform branch that real attention scores almost never take);
// so numerators are at most 2^kTau and are rounded to f16 for the PV
// products, while the denominator sums them unrounded.
//
// PV. The numerators of a row's two heads are packed into f16 token pairs
// (tokens 2k, 2k + 1), exchanged through 256 bytes of LDS so every lane holds
// all four rows' packs, and again enter the dot products as row_newbcast
// operands. V is read with ds_read_tr8_b64, which gives lane i one dim of 8
// consecutive tokens, so token pairs come out of the converts already paired
// and each lane accumulates 8 heads x 2 dims over all 16 tokens.
//
// Launch: one workgroup (one wave) per work unit, in a one-dimensional grid
// whose order is chosen for the hardware dispatcher (see find_unit). With
// two ring slots a wave holds 8.6 KB of LDS and ~85 VGPRs, so 18 waves share
// a compute unit; a wave waiting for its first bytes (a unit's start costs
// three dependent memory round trips under load) leaves the others running.
#include <utility>

#include "common.h"
#include "decode_params.h"
#include "unit_order.h"

namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef int v2i_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i_t lds_v2i_t;

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTau = 15.0f;  // numerators stay at most 2^kTau (f16 range)
constexpr int kD = 128;
constexpr int kG = 8;
constexpr int kGroupBytes = 4096;  // K 16 x 128 B, then V 16 x 128 B
constexpr int kMaxUnitPages = 64;  // pages per work unit (one per lane)

__device__ __forceinline__ float u2f(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t f2u(float f) { return __float_as_uint(f); }

template <typename F, int... I>
__device__ __forceinline__ void unroll_seq(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
// f(std::integral_constant<int, 0>) ... f(std::integral_constant<int, N - 1>)
template <int N, typename F>
__device__ __forceinline__ void unroll(F&& f) {
  unroll_seq(f, std::make_integer_sequence<int, N>{});
}

// acc += dot(a of lane M of this 16-lane row, b), bf16 pairs, fp32 accumulate.
template <int M>
__device__ __forceinline__ float dot2_bf16_bcast(float acc, uint32_t a, uint32_t b) {
  asm("v_dot2c_f32_bf16_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
      : "+v"(acc)
      : "v"(a), "v"(b), "n"(M));
  return acc;
}
// dot(a, b) of bf16 pairs into a fresh fp32 register (no accumulator to zero).
__device__ __forceinline__ float dot2_bf16_first(uint32_t a, uint32_t b) {
  float r;
  asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
// The same with f16 pairs.
template <int M>
__device__ __forceinline__ float dot2_f16_bcast(float acc, uint32_t a, uint32_t b) {
  asm("v_dot2c_f32_f16_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
      : "+v"(acc)
      : "v"(a), "v"(b), "n"(M));
  return acc;
}

template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
  return u2f(static_cast<uint32_t>(
      __builtin_amdgcn_mov_dpp(static_cast<int>(f2u(v)), kCtrl, 0xf, 0xf, false)));
}
// max without the NaN-quieting canonicalisation fmaxf brings (NaN inputs
// do not reach it: masked scores are -inf, never NaN, for finite caches).
__device__ __forceinline__ float fmax_nc(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
// Maximum / sum over the 16 lanes of a row, returned to every lane of it
// (xor 1, xor 2 within quads, then the half-row and row mirrors).
__device__ __forceinline__ float row_max(float v) {
  v = fmax_nc(v, dpp<0xB1>(v));
  v = fmax_nc(v, dpp<0x4E>(v));
  v = fmax_nc(v, dpp<0x141>(v));
  return fmax_nc(v, dpp<0x140>(v));
}
__device__ __forceinline__ float row_sum(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x141>(v);
  return v + dpp<0x140>(v);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)p));
}

// 16 bytes per lane from base + voff into LDS at lds + 16 * lane. m0 is not
// otherwise used by this kernel.
__device__ __forceinline__ void dma16(uint32_t lds, uint32_t voff, const uint8_t* base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds), "v"(voff), "s"(base)
               : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
// Wait until at most n vector-memory loads are outstanding (n is uniform; a
// smaller count than n only waits longer).
__device__ __forceinline__ void wait_vm_le(int n) {
  switch (n < 0 ? 0 : n) {
    case 0: wait_vm<0>(); break;
    case 1: wait_vm<1>(); break;
    case 2: wait_vm<2>(); break;
    case 3: wait_vm<3>(); break;
    case 4: wait_vm<4>(); break;
    case 5: wait_vm<5>(); break;
    case 6: wait_vm<6>(); break;
    case 7: wait_vm<7>(); break;
    case 8: wait_vm<8>(); break;
    case 9: wait_vm<9>(); break;
    case 10: wait_vm<10>(); break;
    case 11: wait_vm<11>(); break;
    case 12: wait_vm<12>(); break;
    case 13: wait_vm<13>(); break;
    case 14: wait_vm<14>(); break;
    default: wait_vm<15>(); break;
  }
}

// Ring layouts. K: 16-byte chunk c of token row t sits at chunk position
// c ^ ((t >> 1) & 7), so the 8 even (or 8 odd) token rows a QK read touches
// land on distinct bank groups. V: chunk c of row t sits at
// c ^ vswz(t), vswz(t) = bits 0 and 2 taken from bits 1 and 2 of t, so the
// 8 rows x 2 chunks of one transposing read of a half-wave do too.
__device__ __forceinline__ uint32_t kswz(uint32_t t) { return (t >> 1) & 7u; }
__device__ __forceinline__ uint32_t vswz(uint32_t t) {
  const uint32_t j = (t >> 1) & 3u;
  return (j & 1u) | ((j & 2u) << 1);
}

// Per-lane constants of the lane layout above.
struct LaneMap {
  int r, i, tok;
  bool lo8;
  uint32_t pack_sel;                    // v_perm selector of the numerator pack
  uint32_t kr0, kr1;                    // K read offsets in a ring slot
  uint32_t vr[2][2];                    // V transposing-read offsets in a slot
  uint32_t koff0, koff1, voff0, voff1;  // DMA source offsets in a group's K / V block
};

__device__ __forceinline__ LaneMap lane_map(int lane) {
  LaneMap m;
  m.r = lane >> 4;
  m.i = lane & 15;
  m.tok = 2 * (m.i & 7) + (m.i >> 3);
  m.lo8 = m.i < 8;
  // lane i < 8 packs (own head-2r value, partner's), lane i >= 8 (partner's
  // head-2r+1 value, own): bytes of {partner, own} for v_perm
  m.pack_sel = m.lo8 ? 0x05040100u : 0x03020706u;
  m.kr0 = m.tok * kD + (((2 * m.r) ^ kswz(m.tok)) << 4);
  m.kr1 = m.tok * kD + (((2 * m.r + 1) ^ kswz(m.tok)) << 4);
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int o = 0; o < 2; ++o) {
      const uint32_t t = 8 * o + (m.i >> 1);
      m.vr[s][o] = 2048 + t * kD + (((2 * m.r + s) ^ vswz(t)) << 4) + 8 * (m.i & 1);
    }
  // lane L fills LDS chunk position L & 7 of row L >> 3 (first 1 KB of a
  // block) and of row 8 + (L >> 3) (second)
  const uint32_t dr0 = lane >> 3, dr1 = 8 + (lane >> 3), dpos = lane & 7;
  m.koff0 = dr0 * kD + ((dpos ^ kswz(dr0)) << 4);
  m.koff1 = dr1 * kD + ((dpos ^ kswz(dr1)) << 4);
  m.voff0 = dr0 * kD + ((dpos ^ vswz(dr0)) << 4);
  m.voff1 = dr1 * kD + ((dpos ^ vswz(dr1)) << 4);
  return m;
}

// A work unit: request b, kv head g, split c (tokens [t_begin, t_end)).
struct Unit {
  int b, g, c, t_begin, t_end, n_groups, first_page, n_pages;
};

__device__ __forceinline__ Unit make_unit(int b, int g, int c, int L, int S, int log2P) {
  Unit u;
  u.b = b;
  u.g = g;
  u.c = c;
  u.t_begin = c * S;
  u.t_end = min(L, u.t_begin + S);
  u.n_groups = (u.t_end - u.t_begin + 15) >> 4;
  u.first_page = u.t_begin >> log2P;
  u.n_pages = (u.t_end - u.t_begin + (1 << log2P) - 1) >> log2P;
  return u;
}

// The unit's pages (at most 64): lane j holds the byte offset of the
// (page j, kv head g) block, read back per group with readlane; bit j of
// valid says whether page id j is inside the pool (an invalid page is
// replaced by page 0 for the loads and its tokens are masked).
struct Pages {
  uint64_t valid;
  int lo, hi;
};

__device__ __forceinline__ Pages page_offsets(const DecodeParams& p, int pg, int g) {
  Pages pgs;
  const bool ok = pg >= 0 && pg < p.num_pages;
  pgs.valid = __ballot(ok);
  const int64_t off =
      (static_cast<int64_t>(ok ? pg : 0) * p.num_kv_heads + g) * (static_cast<int64_t>(p.page_size) * kD);
  pgs.lo = static_cast<int>(static_cast<uint32_t>(off));
  pgs.hi = static_cast<int>(static_cast<uint32_t>(static_cast<uint64_t>(off) >> 32));
  return pgs;
}

__device__ __forceinline__ int group_tokens(const Unit& u, const Pages& pgs, int gi, int log2P) {
  const bool ok = ((pgs.valid >> ((gi << 4) >> log2P)) & 1u) != 0;
  return ok ? min(16, u.t_end - (u.t_begin + (gi << 4))) : 0;
}

// DMA of group gi of a unit into the ring slot at LDS address slot.
__device__ __forceinline__ void issue_group(uint32_t slot, const LaneMap& lm, const DecodeParams& p,
                                            const Pages& pgs, int gi, int log2P) {
  const int j = (gi << 4) >> log2P;
  const uint64_t off =
      (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(pgs.hi, j))) << 32) |
      static_cast<uint32_t>(__builtin_amdgcn_readlane(pgs.lo, j));
  const uint32_t row_off = static_cast<uint32_t>(((gi << 4) & (p.page_size - 1)) * kD);
  const uint8_t* kb = static_cast<const uint8_t*>(p.k_pool) + off + row_off;
  const uint8_t* vb = static_cast<const uint8_t*>(p.v_pool) + off + row_off;
  dma16(slot, lm.koff0, kb);
  dma16(slot + 1024, lm.koff1, kb);
  dma16(slot + 2048, lm.voff0, vb);
  dma16(slot + 3072, lm.voff1, vb);
}

// Running softmax state of a lane (heads 2r, 2r + 1).
struct Softmax {
  float m[2];  // reference max (log2 domain), once set
  float l[2];  // denominators over this lane's tokens
  bool set;    // (wave-uniform) a valid token has been seen
};

// The query operands of a unit.
struct Query {
  uint32_t qd[kG];   // bf16 pair (32r + 2i, 32r + 2i + 1) of head h
  uint32_t qb0[kG];  // pair 0 of the row, in every lane of the row
  float qk_scale;    // k_scale * sm_scale * log2(e)
  float o_scale;     // v_scale
};

__device__ __forceinline__ void finish_query(Query& q) {
#pragma unroll
  for (int h = 0; h < kG; ++h)
    q.qb0[h] = static_cast<uint32_t>(
        __builtin_amdgcn_mov_dpp(static_cast<int>(q.qd[h]), 0x150, 0xf, 0xf, false));
}

// One 16-token group: K words kw0/kw1 and V words vw (already in registers)
// into the softmax state and the accumulators o[h][s] (head h, dim
// 32r + 16s + i). pbuf: 256 B of LDS for the numerator exchange; abuf: 8
// floats for the rare rescale.
__device__ __forceinline__ void group_math(const LaneMap& lm, const uint4& kw0, const uint4& kw1,
                                           uint32_t (&vw)[2][2][2], int nv, const Query& q,
                                           Softmax& st, float (&o)[kG][2], uint32_t* pbuf,
                                           float* abuf) {
  if (nv < 16) {
    // tokens past the context or of an invalid page: V bytes to 0
#pragma unroll
    for (int o2 = 0; o2 < 2; ++o2) {
      const int vo = min(8, max(0, nv - 8 * o2));
      const uint64_t m64 = vo >= 8 ? ~0ull : ((1ull << (8 * vo)) - 1ull);
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        vw[s2][o2][0] &= static_cast<uint32_t>(m64);
        vw[s2][o2][1] &= static_cast<uint32_t>(m64 >> 32);
      }
    }
  }

  // ---- QK^T: row partial dots of token tok for the 8 heads
  float a[kG];
  const uint32_t kw[8] = {kw0.x, kw0.y, kw0.z, kw0.w, kw1.x, kw1.y, kw1.z, kw1.w};
  unroll<8>([&](auto wc) {
    constexpr int w = decltype(wc)::value;
    const uint32_t x0 = __builtin_bit_cast(
        uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(kw[w], 1.0f, false));
    const uint32_t x1 = __builtin_bit_cast(
        uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(kw[w], 1.0f, true));
    unroll<kG>([&](auto hc) {
      constexpr int h = decltype(hc)::value;
      if constexpr (w == 0)
        a[h] = dot2_bf16_first(q.qb0[h], x0);
      else
        a[h] = dot2_bf16_bcast<2 * w>(a[h], q.qd[h], x0);
    });
    unroll<kG>([&](auto hc) {
      constexpr int h = decltype(hc)::value;
      a[h] = dot2_bf16_bcast<2 * w + 1>(a[h], q.qd[h], x1);
    });
  });
  // reduce-scatter over the four rows: row r keeps heads 2r, 2r + 1
  float u[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const auto rr = __builtin_amdgcn_permlane32_swap(f2u(a[h]), f2u(a[h + 4]), false, false);
    u[h] = u2f(rr[0]) + u2f(rr[1]);
  }
  float sc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const auto rr = __builtin_amdgcn_permlane16_swap(f2u(u[j]), f2u(u[j + 2]), false, false);
    sc[j] = u2f(rr[0]) + u2f(rr[1]);
  }

  // ---- scores relative to the reference max (log2 domain)
  const bool tv = lm.tok < nv;
  float d[2];
  if (!st.set) {
    // the first group with a valid token sets the reference max
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float raw = tv ? sc[j] * q.qk_scale : -INFINITY;
      if (nv > 0) st.m[j] = row_max(raw);
      d[j] = nv > 0 ? raw - st.m[j] : -INFINITY;
    }
    st.set = nv > 0;
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j) d[j] = tv ? __builtin_fmaf(sc[j], q.qk_scale, -st.m[j]) : -INFINITY;
    if (__any(d[0] > kTau || d[1] > kTau)) {
      // rare: raise the reference max of the heads that need it, rescale
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float mx = row_max(d[j]);
        const float sh = mx > 0.0f ? mx : 0.0f;
        st.m[j] += sh;
        d[j] -= sh;
        const float al = __builtin_amdgcn_exp2f(-sh);
        st.l[j] *= al;
        if (lm.i == 0) abuf[2 * lm.r + j] = al;
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int h = 0; h < kG; ++h) {
        const float al = abuf[h];
        o[h][0] *= al;
        o[h][1] *= al;
      }
      __builtin_amdgcn_wave_barrier();
    }
  }

  // ---- numerators, packed into f16 token pairs and shared with all rows
  float pr[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    pr[j] = __builtin_amdgcn_exp2f(d[j]);
    st.l[j] += pr[j];
  }
  // lanes i and i ^ 8 hold tokens 2(i & 7) and 2(i & 7) + 1 (row_ror:8
  // swaps them): lane i < 8 packs head 2r, lane i >= 8 head 2r + 1, both
  // for token pair k = i & 7
  const half2_t own = {static_cast<_Float16>(pr[0]), static_cast<_Float16>(pr[1])};
  const uint32_t ownu = __builtin_bit_cast(uint32_t, own);
  const uint32_t other = static_cast<uint32_t>(
      __builtin_amdgcn_mov_dpp(static_cast<int>(ownu), 0x128, 0xf, 0xf, false));
  pbuf[lm.i * 4 + lm.r] = __builtin_amdgcn_perm(other, ownu, lm.pack_sel);
  __builtin_amdgcn_wave_barrier();
  const uint4 G4 = *reinterpret_cast<const uint4*>(&pbuf[lm.i * 4]);
  const uint32_t Gp[4] = {G4.x, G4.y, G4.z, G4.w};  // Gp[j]: heads 2j (lanes 0-7), 2j+1 (8-15)
  __builtin_amdgcn_wave_barrier();

  // ---- PV: o[h][s] += sum over token pairs k of p[h][2k..2k+1] . v
  unroll<2>([&](auto sc_) {
    constexpr int s2 = decltype(sc_)::value;
    unroll<4>([&](auto wc) {
      constexpr int ow = decltype(wc)::value;  // octet ow >> 1, word ow & 1
      const uint32_t word = vw[s2][ow >> 1][ow & 1];
      const uint32_t v0 = __builtin_bit_cast(
          uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word, 1.0f, false));
      const uint32_t v1 = __builtin_bit_cast(
          uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word, 1.0f, true));
      constexpr int k0 = 2 * ow;  // pair index of v0 (tokens 4ow, 4ow + 1)
      unroll<kG>([&](auto hc) {
        constexpr int h = decltype(hc)::value;
        o[h][s2] = dot2_f16_bcast<8 * (h & 1) + k0>(o[h][s2], Gp[h >> 1], v0);
      });
      unroll<kG>([&](auto hc) {
        constexpr int h = decltype(hc)::value;
        o[h][s2] = dot2_f16_bcast<8 * (h & 1) + k0 + 1>(o[h][s2], Gp[h >> 1], v1);
      });
    });
  });
}

// K and V words of the group in the ring slot at LDS pointer slot.
__device__ __forceinline__ void read_group(const uint8_t* slot, const LaneMap& lm, uint4& kw0,
                                           uint4& kw1, uint32_t (&vw)[2][2][2]) {
  kw0 = *reinterpret_cast<const uint4*>(slot + lm.kr0);
  kw1 = *reinterpret_cast<const uint4*>(slot + lm.kr1);
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
    for (int o2 = 0; o2 < 2; ++o2) {
      const v2i_t x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_t*)(slot + lm.vr[s2][o2]));
      vw[s2][o2][0] = static_cast<uint32_t>(x[0]);
      vw[s2][o2][1] = static_cast<uint32_t>(x[1]);
    }
  // the slot may be refilled once its bytes are in registers
  asm volatile("" : : "v"(kw0.x), "v"(kw0.y), "v"(kw0.z), "v"(kw0.w), "v"(kw1.x), "v"(kw1.y),
               "v"(kw1.z), "v"(kw1.w));
  asm volatile("" : : "v"(vw[0][0][0]), "v"(vw[0][0][1]), "v"(vw[0][1][0]), "v"(vw[0][1][1]),
               "v"(vw[1][0][0]), "v"(vw[1][0][1]), "v"(vw[1][1][0]), "v"(vw[1][1][1]));
}

// Partial output of a finished unit: o / l per head and lse = m + log2 l
// (natural-log units). fin: 16 floats of LDS.
__device__ __forceinline__ void finish_unit(const DecodeParams& p, const LaneMap& lm, const Unit& u,
                                            const Softmax& st, const float (&o)[kG][2],
                                            float o_scale, float* fin) {
  float ls[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) ls[j] = row_sum(st.l[j]);
  if (lm.i == 0) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      fin[2 * lm.r + j] = ls[j];
      fin[kG + 2 * lm.r + j] = st.set ? st.m[j] : 0.0f;
    }
  }
  __builtin_amdgcn_wave_barrier();
  const int64_t bh0 = static_cast<int64_t>(u.b) * p.num_q_heads + u.g * kG;
#pragma unroll
  for (int h = 0; h < kG; ++h) {
    const float lh = fin[h];
    const float f = lh > 0.0f ? o_scale / lh : 0.0f;
    float* dst = p.o_part + ((bh0 + h) * p.max_splits + u.c) * kD + 32 * lm.r + lm.i;
    dst[0] = o[h][0] * f;
    dst[16] = o[h][1] * f;
  }
  const int lane = threadIdx.x;
  if (lane < kG) {
    const float lh = fin[lane];
    p.lse_part[(bh0 + lane) * p.max_splits + u.c] =
        lh > 0.0f ? (fin[kG + lane] + __log2f(lh)) * kLn2 : -INFINITY;
  }
  __builtin_amdgcn_wave_barrier();
}

// ------------------------------------------------------------ dispatched
template <int kSlots>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(3)))
decode_gqa_e4m3_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[kSlots * kGroupBytes];
  __shared__ __attribute__((aligned(16))) uint32_t pbuf[16 * 4];  // [lane in row][row]
  __shared__ float fin[2 * kG];
  __shared__ float abuf[kG];
  const int lane = threadIdx.x;
  int b, g, c, L;
  if (!pkv::find_unit(p, static_cast<int>(blockIdx.x), b, g, c, L)) return;
  const int log2P = p.page_size == 16 ? 4 : (p.page_size == 32 ? 5 : 6);
  const Unit u = make_unit(b, g, c, L, p.split_tokens, log2P);
  const LaneMap lm = lane_map(lane);

  Query q;
  {
    const uint32_t* qw = reinterpret_cast<const uint32_t*>(
        p.q + (static_cast<int64_t>(b) * p.num_q_heads + g * kG) * kD);
#pragma unroll
    for (int h = 0; h < kG; ++h) q.qd[h] = qw[h * (kD / 2) + lane];
  }
  q.qk_scale = p.k_scale[g] * p.sm_scale_log2;
  q.o_scale = p.v_scale[g];
  const int32_t* bt = p.block_table + static_cast<int64_t>(b) * p.max_pages;
  int pg = -1;
  if (lane < u.n_pages) pg = bt[u.first_page + lane];
  // Every compiler-issued load must be complete before the first DMA, or its
  // own wait for them would also wait for the ring.
  asm volatile("" : : "v"(q.qd[0]), "v"(q.qd[1]), "v"(q.qd[2]), "v"(q.qd[3]), "v"(q.qd[4]),
               "v"(q.qd[5]), "v"(q.qd[6]), "v"(q.qd[7]));
  asm volatile("" : : "v"(q.qk_scale), "v"(q.o_scale), "v"(pg));
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" : : : "memory");
  finish_query(q);
  const Pages pgs = page_offsets(p, pg, g);
  const uint32_t ring0 = lds_addr(ring);

  Softmax st;
  st.set = false;
  st.m[0] = st.m[1] = 0.0f;
  st.l[0] = st.l[1] = 0.0f;
  float o[kG][2];
#pragma unroll
  for (int h = 0; h < kG; ++h) o[h][0] = o[h][1] = 0.0f;

  const int n_groups = u.n_groups;
  unroll<kSlots>([&](auto kc) {
    constexpr int k = decltype(kc)::value;
    if (k < n_groups) issue_group(ring0 + k * kGroupBytes, lm, p, pgs, k, log2P);
  });
  for (int g0 = 0; g0 < n_groups; g0 += kSlots) {
    unroll<kSlots>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      const int gi = g0 + k;
      if (gi >= n_groups) return;
      // groups gi + 1 .. gi + kSlots - 1 may still be in flight
      wait_vm_le(4 * min(kSlots - 1, n_groups - 1 - gi));
      uint4 kw0, kw1;
      uint32_t vw[2][2][2];
      read_group(ring + k * kGroupBytes, lm, kw0, kw1, vw);
      if (gi + kSlots < n_groups) issue_group(ring0 + k * kGroupBytes, lm, p, pgs, gi + kSlots, log2P);
      group_math(lm, kw0, kw1, vw, group_tokens(u, pgs, gi, log2P), q, st, o, pbuf, abuf);
    });
  }
  finish_unit(p, lm, u, st, o, q.o_scale, fin);
}

}  // namespace

bool gqa_e4m3_path_supported(int dk, int dv, int group, bool latent, int split_tokens,
                             int page_size) {
  return !latent && dk == kD && dv == kD && group == kG &&
         split_tokens <= kMaxUnitPages * page_size;
}

int launch_decode_gqa_e4m3(const DecodeParams& p, int n_split_blocks, int batch,
                           hipStream_t stream) {
  const int64_t units = static_cast<int64_t>(n_split_blocks) * p.num_kv_heads * batch;
  if (units > 0x7FFFFFFF) return launch_decode_gqa(p, true, n_split_blocks, batch, stream);
  decode_gqa_e4m3_kernel<2><<<dim3(static_cast<uint32_t>(units)), 64, 0, stream>>>(p);
  return pkv::launch_status();
}
