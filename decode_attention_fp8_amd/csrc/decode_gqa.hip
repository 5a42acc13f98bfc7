// Grouped-query decode kernel for head dim 128 and 8 query heads per kv head
// (the production shape), e4m3 or bf16 cache.
//
// "Smaller, faster, safer", section "Quantizing the KV cache": the FP8
// kernel converts cached values as it reads them, a little extra work per
// token. Here that conversion is gfx950's packed e4m3 -> bf16 / f16 convert
// (two codes per instruction, exact), and the arithmetic it feeds is packed
// two-term dot products, so the per-byte VALU cost stays under the HBM time.
//
// One wave per work unit (request b, kv head g, split c). The split is
// processed in groups of 16 tokens (one page of 16, or a quarter of a page
// of 64). Each group's K and V bytes travel HBM -> LDS by direct-to-LDS
// loads (global_load_lds_dwordx4) into a ring of kSlots group buffers, so
// kSlots - 1 groups are in flight while one is computed without holding any
// registers; the loads and their vmcnt waits are issued by hand because the
// compiler cannot tell the ring slots apart and would wait for all of them.
//
// QK^T. Lane (cq = lane >> 4, tq = lane & 15) holds dims [32cq, 32cq+32) of
// the 8 query heads (128 registers of bf16 pairs) and reads those dims of
// row tq from LDS (the DMA lane order stores 16-byte chunk c of row r at
// chunk position c ^ (r & 7), so these reads are bank-conflict free). The
// 8 partial dot products are reduce-scattered over the 4 chunk lanes
// (permlane32 swap, permlane16 swap), leaving each lane the full scores of
// its token for two heads.
//
// Softmax. Scores are kept in the log2 domain. Each head's running maximum
// m only moves when a score exceeds it by more than kTau (and on the first
// group), so exp2(s - m) <= 2^kTau and the rescale of the accumulators is
// rare. p is rounded to f16 (bf16 for a bf16 cache) and the rounded value is
// what both the numerator and the denominator use.
//
// PV. Lane (tg = lane >> 4, dg = lane & 15) owns dims [8dg, 8dg+8) of all 8
// heads (64 fp32 accumulators) for tokens tg, tg+4, tg+8, tg+12. Token pairs
// (t, t+4) are interleaved with a byte permute so one packed dot product
// takes p and v of both tokens. p reaches these lanes through 256 bytes of
// LDS.
#include <type_traits>

#include "common.h"
#include "decode_params.h"
#include "unit_order.h"

namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTau = 8.0f;      // log2 headroom before a rescale
constexpr float kMInit = -1e30f;  // running max before any token
constexpr int kD = 128;
constexpr int kG = 8;
constexpr int kMaxUnitPages = 64;  // pages per work unit (one per lane)

__device__ __forceinline__ float u2f(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t f2u(float f) { return __float_as_uint(f); }
__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2_t, u); }
__device__ __forceinline__ half2_t as_half2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }

// First result of a lane-half swap; each lane keeps two values that belong
// together (same register role, lanes L and L^32, or L and L^16).
__device__ __forceinline__ uint32_t swap32_first(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_permlane32_swap(a, b, false, false)[0];
}
__device__ __forceinline__ uint32_t swap16_first(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_permlane16_swap(a, b, false, false)[0];
}

// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)p));
}

// 16 bytes per lane from base + voff into LDS at lds + 16 * lane (the
// instruction's immediate offset would move both addresses, so it stays 0).
// m0 is not otherwise used by this kernel. kNt selects the non-temporal
// form, for launches whose cache would not stay resident.
template <bool kNt>
__device__ __forceinline__ void dma16(uint32_t lds, uint32_t voff, const uint8_t* base) {
  if constexpr (kNt)
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                 :
                 : "s"(lds), "v"(voff), "s"(base)
                 : "memory");
  else
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(lds), "v"(voff), "s"(base)
                 : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// The ring: bytes per group, slots, DMA instructions per group.
template <bool kE4M3>
struct Ring;
template <>
struct Ring<true> {
  static constexpr int kGroupBytes = 4096;  // K 16 x 128 B, V 16 x 128 B
  static constexpr int kSlots = 4;
  static constexpr int kDma = 4;
};
template <>
struct Ring<false> {
  static constexpr int kGroupBytes = 8192;  // K 16 x 256 B, V 16 x 256 B
  static constexpr int kSlots = 3;
  static constexpr int kDma = 8;
};

struct __attribute__((aligned(16))) WaveLds {
  uint32_t ppair[2][8][kG];  // per group parity: (p[t], p[t+4]) halves, t = 8*(pi>>2) + (pi&3)
  float score[16][kG];       // scores of one group, for the rare max update
  float m[kG];               // running max per head (log2 domain)
  float alpha[kG];           // rescale factor of the last max update
  float l[kG];               // final denominators
};

template <bool kE4M3>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) decode_gqa_kernel(DecodeParams p) {
  using R = Ring<kE4M3>;
  constexpr int kVw = kE4M3 ? 2 : 4;  // V words per token row slice of a lane
  __shared__ WaveLds lds;
  __shared__ __attribute__((aligned(16))) uint8_t ring[R::kSlots * R::kGroupBytes];
  const int c = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int lane = threadIdx.x;

  if (p.abort_flags && p.abort_flags[b]) return;
  const int L = p.seq_lens[b];
  if (L > p.max_seq_len) return;
  const int t_begin = c * p.split_tokens;
  if (t_begin >= L) return;
  const int t_end = min(L, t_begin + p.split_tokens);
  const int n_groups = (t_end - t_begin + 15) >> 4;
  const int P = p.page_size;
  const int log2P = P == 16 ? 4 : (P == 32 ? 5 : 6);

  const int tq = lane & 15, cq = lane >> 4;
  const int tg = lane >> 4, dg = lane & 15;
  // Ownership after the score reduce-scatter: push head labels through the
  // same swap network the partial sums take (the token stays the lane's).
  const int my_tok = tq;
  int my_h0;
  {
    const uint32_t a = swap32_first(0u, 4u);
    const uint32_t bb = swap32_first(2u, 6u);
    my_h0 = static_cast<int>(swap16_first(a, bb));
  }
  // Heads this lane writes after the accumulator reduce-scatter.
  int out_h[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t a = swap32_first(static_cast<uint32_t>(h), static_cast<uint32_t>(h + 4));
    const uint32_t bb = swap32_first(static_cast<uint32_t>(h + 2), static_cast<uint32_t>(h + 6));
    out_h[h] = static_cast<int>(swap16_first(a, bb));
  }

  // q: dims [32cq, 32cq+32) of the 8 heads of this kv head, as bf16 pairs
  uint32_t qr[kG][16];
  {
    const uint16_t* qb = p.q + (static_cast<int64_t>(b) * p.num_q_heads + g * kG) * kD + cq * 32;
#pragma unroll
    for (int h = 0; h < kG; ++h)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint4 a = *reinterpret_cast<const uint4*>(qb + h * kD + 8 * k);
        qr[h][4 * k] = a.x; qr[h][4 * k + 1] = a.y; qr[h][4 * k + 2] = a.z; qr[h][4 * k + 3] = a.w;
      }
  }
  const float qk_scale = (kE4M3 ? p.k_scale[g] : 1.0f) * p.sm_scale_log2;
  const float o_scale = kE4M3 ? p.v_scale[g] : 1.0f;

  // The unit's pages (at most 64): lane j holds the byte offset of the
  // (page j, kv head g) block, read back per group with readlane; bit j of
  // valid says whether page id j is inside the pool (an invalid page is
  // replaced by page 0 for the loads and its tokens are masked).
  constexpr int64_t kElem = kE4M3 ? 1 : 2;
  constexpr int kRow = kD * kElem;  // bytes per cache row
  const int64_t head_stride = static_cast<int64_t>(P) * kRow;  // bytes of one (page, head) block
  const int32_t* bt = p.block_table + static_cast<int64_t>(b) * p.max_pages;
  const int first_page = t_begin >> log2P;
  const int n_unit_pages = (t_end - t_begin + P - 1) >> log2P;
  int pg = -1;
  if (lane < n_unit_pages) pg = bt[first_page + lane];
  // the launch's footprint; up to 64 requests its loads join the ones above
  const int64_t tokens = p.batch <= 64 ? pkv::wave_sum(pkv::footprint_len(pkv::unit_len(p, lane)))
                                       : pkv::launch_tokens(p);
  const bool stream = pkv::stream_cache(tokens * p.num_kv_heads * 2 * kRow);
  if (lane < kG) lds.m[lane] = kMInit;
  // Every compiler-issued load must be complete before the first DMA, or its
  // own wait for them would also wait for the ring.
#pragma unroll
  for (int h = 0; h < kG; ++h)
#pragma unroll
    for (int k = 0; k < 16; k += 8)
      asm volatile("" : : "v"(qr[h][k]), "v"(qr[h][k + 1]), "v"(qr[h][k + 2]), "v"(qr[h][k + 3]),
                   "v"(qr[h][k + 4]), "v"(qr[h][k + 5]), "v"(qr[h][k + 6]), "v"(qr[h][k + 7]));
  asm volatile("" : : "v"(qk_scale), "v"(o_scale), "v"(pg), "s"(static_cast<int>(stream)));
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" : : : "memory");
  const bool pg_ok = pg >= 0 && pg < p.num_pages;
  const uint64_t valid = __ballot(pg_ok);
  const int64_t blk_off = (static_cast<int64_t>(pg_ok ? pg : 0) * p.num_kv_heads + g) * head_stride;
  const int off_lo = static_cast<int>(static_cast<uint32_t>(blk_off));
  const int off_hi = static_cast<int>(static_cast<uint32_t>(static_cast<uint64_t>(blk_off) >> 32));

  float o[kG][8];
#pragma unroll
  for (int h = 0; h < kG; ++h)
#pragma unroll
    for (int d = 0; d < 8; ++d) o[h][d] = 0.0f;
  float mq[2] = {kMInit, kMInit};
  float l[2] = {0.0f, 0.0f};

  const uint8_t* kpool = static_cast<const uint8_t*>(p.k_pool);
  const uint8_t* vpool = static_cast<const uint8_t*>(p.v_pool);
  const uint32_t ring0 = lds_addr(ring);

  // per-lane DMA source offsets inside a group (see the ring layout above)
  uint32_t koff0, koff1 = 0;
  if constexpr (kE4M3) {
    koff0 = (lane >> 3) * kRow + (((lane & 7) ^ (lane >> 3)) << 4);
  } else {
    const int r0 = lane >> 4, r1 = 4 + (lane >> 4);
    koff0 = r0 * kRow + (((lane & 15) ^ (r0 & 7)) << 4);
    koff1 = r1 * kRow + (((lane & 15) ^ (r1 & 7)) << 4);
  }
  const uint32_t voff = lane << 4;

  auto group_valid = [&](int gi) __attribute__((always_inline)) {
    return ((valid >> ((gi << 4) >> log2P)) & 1u) != 0;
  };
  // DMA of group gi into its ring slot.
  auto issue = [&](int gi) __attribute__((always_inline)) {
    const int j = (gi << 4) >> log2P;
    const uint64_t off =
        (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(off_hi, j))) << 32) |
        static_cast<uint32_t>(__builtin_amdgcn_readlane(off_lo, j));
    const uint32_t row_off = static_cast<uint32_t>(((gi << 4) & (P - 1)) * kRow);
    const uint8_t* kb = kpool + off + row_off;
    const uint8_t* vb = vpool + off + row_off;
    const uint32_t slot = ring0 + (gi % R::kSlots) * R::kGroupBytes;
    // one branch per group selects the load form for all of its loads
    auto dmas = [&](auto nt) __attribute__((always_inline)) {
      constexpr bool kNt = decltype(nt)::value;
      if constexpr (kE4M3) {
        dma16<kNt>(slot, koff0, kb);
        dma16<kNt>(slot + 1024, koff0, kb + 1024);
        dma16<kNt>(slot + 2048, voff, vb);
        dma16<kNt>(slot + 3072, voff, vb + 1024);
      } else {
        dma16<kNt>(slot, koff0, kb);
        dma16<kNt>(slot + 1024, koff1, kb);
        dma16<kNt>(slot + 2048, koff0, kb + 2048);
        dma16<kNt>(slot + 3072, koff1, kb + 2048);
        dma16<kNt>(slot + 4096, voff, vb);
        dma16<kNt>(slot + 5120, voff, vb + 1024);
        dma16<kNt>(slot + 6144, voff, vb + 2048);
        dma16<kNt>(slot + 7168, voff, vb + 3072);
      }
    };
    if (stream)
      dmas(std::true_type{});
    else
      dmas(std::false_type{});
  };

  // V rows tg + 4j, dims [8dg, 8dg+8) of group gi; rows past the context
  // (last group) or of an invalid page are zeroed.
  auto read_v = [&](int gi, uint32_t (&vw)[4][kVw]) __attribute__((always_inline)) {
    const uint8_t* sv = ring + (gi % R::kSlots) * R::kGroupBytes + R::kGroupBytes / 2;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (kE4M3) {
        const uint2 x = *reinterpret_cast<const uint2*>(sv + (tg + 4 * j) * kRow + dg * 8);
        vw[j][0] = x.x; vw[j][1] = x.y;
      } else {
        const uint4 x = *reinterpret_cast<const uint4*>(sv + (tg + 4 * j) * kRow + dg * 16);
        vw[j][0] = x.x; vw[j][1] = x.y; vw[j][2] = x.z; vw[j][3] = x.w;
      }
    }
    const int nv = group_valid(gi) ? min(16, t_end - (t_begin + (gi << 4))) : 0;
    if (nv < 16) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (tg + 4 * j >= nv)
#pragma unroll
          for (int k = 0; k < kVw; ++k) vw[j][k] = 0u;
    }
  };

  // QK^T and the softmax numerators of group gi (into ppair[gi & 1]); returns
  // whether the running max moved (then alpha is in lds.alpha and o must be
  // rescaled once the previous group's PV is done).
  auto qk = [&](int gi) __attribute__((always_inline)) {
    const uint8_t* sk = ring + (gi % R::kSlots) * R::kGroupBytes;
    const int nv = group_valid(gi) ? min(16, t_end - (t_begin + (gi << 4))) : 0;
    float a[kG];
    {
      uint32_t kw[kE4M3 ? 8 : 16];
      const uint8_t* row = sk + tq * kRow;
      const int sw = tq & 7;
      if constexpr (kE4M3) {
        const uint4 k0 = *reinterpret_cast<const uint4*>(row + (((2 * cq) ^ sw) << 4));
        const uint4 k1 = *reinterpret_cast<const uint4*>(row + (((2 * cq + 1) ^ sw) << 4));
        kw[0] = k0.x; kw[1] = k0.y; kw[2] = k0.z; kw[3] = k0.w;
        kw[4] = k1.x; kw[5] = k1.y; kw[6] = k1.z; kw[7] = k1.w;
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint4 kk = *reinterpret_cast<const uint4*>(row + (((4 * cq + k) ^ sw) << 4));
          kw[4 * k] = kk.x; kw[4 * k + 1] = kk.y; kw[4 * k + 2] = kk.z; kw[4 * k + 3] = kk.w;
        }
      }
#pragma unroll
      for (int h = 0; h < kG; ++h) a[h] = 0.0f;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        bf16x2_t x0, x1;
        if constexpr (kE4M3) {
          x0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(kw[m], 1.0f, false);
          x1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(kw[m], 1.0f, true);
        } else {
          x0 = as_bf16x2(kw[2 * m]);
          x1 = as_bf16x2(kw[2 * m + 1]);
        }
#pragma unroll
        for (int h = 0; h < kG; ++h) {
          a[h] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qr[h][2 * m]), x0, a[h], false);
          a[h] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qr[h][2 * m + 1]), x1, a[h], false);
        }
      }
    }

    // reduce-scatter over the 4 chunk lanes
    float u[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const auto r = __builtin_amdgcn_permlane32_swap(f2u(a[h]), f2u(a[h + 4]), false, false);
      u[h] = u2f(r[0]) + u2f(r[1]);
    }
    float x[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const auto r = __builtin_amdgcn_permlane16_swap(f2u(u[j]), f2u(u[j + 2]), false, false);
      const float sc = (u2f(r[0]) + u2f(r[1])) * qk_scale;
      x[j] = (my_tok < nv) ? sc : -INFINITY;
    }

    // rare running-max update
    const bool over = (x[0] > mq[0] + kTau) || (x[1] > mq[1] + kTau);
    const bool moved = __any(over);
    if (moved) {
      lds.score[my_tok][my_h0] = x[0];
      lds.score[my_tok][my_h0 + 1] = x[1];
      __builtin_amdgcn_wave_barrier();
      if (lane < kG) {
        float pm = lds.score[0][lane];
#pragma unroll
        for (int r = 1; r < 16; ++r) pm = fmaxf(pm, lds.score[r][lane]);
        const float m_old = lds.m[lane];
        const float m_new = fmaxf(m_old, pm);
        lds.m[lane] = m_new;
        lds.alpha[lane] = __builtin_amdgcn_exp2f(m_old - m_new);
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        mq[j] = lds.m[my_h0 + j];
        l[j] *= lds.alpha[my_h0 + j];
      }
    }

    // probabilities to LDS, pairs (t, t+4)
    {
      const int pi = ((my_tok >> 3) << 2) | (my_tok & 3);
      const int half = (my_tok >> 2) & 1;
      uint16_t* pp = reinterpret_cast<uint16_t*>(&lds.ppair[gi & 1][pi][0]);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float pr = __builtin_amdgcn_exp2f(x[j] - mq[j]);
        uint16_t bits;
        float pr_used;
        if constexpr (kE4M3) {
          const _Float16 ph = static_cast<_Float16>(pr);
          bits = __builtin_bit_cast(uint16_t, ph);
          pr_used = static_cast<float>(ph);
        } else {
          const __bf16 pb = static_cast<__bf16>(pr);
          bits = __builtin_bit_cast(uint16_t, pb);
          pr_used = static_cast<float>(pb);
        }
        l[j] += pr_used;
        pp[(my_h0 + j) * 2 + half] = bits;
      }
    }
    __builtin_amdgcn_wave_barrier();
    return moved;
  };

  // o += P V for group gi, from ppair[gi & 1] and its V words.
  auto pv = [&](int gi, const uint32_t (&vw)[4][kVw]) __attribute__((always_inline)) {
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
      const uint4 pa = *reinterpret_cast<const uint4*>(&lds.ppair[gi & 1][pr * 4 + tg][0]);
      const uint4 pb = *reinterpret_cast<const uint4*>(&lds.ppair[gi & 1][pr * 4 + tg][4]);
      const uint32_t ph[kG] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
      uint32_t vp[8];
      const uint32_t* A = vw[2 * pr];      // token t
      const uint32_t* B = vw[2 * pr + 1];  // token t + 4
      if constexpr (kE4M3) {
        const uint32_t ws[4] = {__builtin_amdgcn_perm(B[0], A[0], 0x05010400u),
                                __builtin_amdgcn_perm(B[0], A[0], 0x07030602u),
                                __builtin_amdgcn_perm(B[1], A[1], 0x05010400u),
                                __builtin_amdgcn_perm(B[1], A[1], 0x07030602u)};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          vp[2 * k] = __builtin_bit_cast(uint32_t,
                                         __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(ws[k], 1.0f, false));
          vp[2 * k + 1] = __builtin_bit_cast(uint32_t,
                                             __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(ws[k], 1.0f, true));
        }
#pragma unroll
        for (int h = 0; h < kG; ++h)
#pragma unroll
          for (int d = 0; d < 8; ++d)
            o[h][d] = __builtin_amdgcn_fdot2(as_half2(ph[h]), as_half2(vp[d]), o[h][d], false);
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          vp[2 * k] = __builtin_amdgcn_perm(B[k], A[k], 0x05040100u);
          vp[2 * k + 1] = __builtin_amdgcn_perm(B[k], A[k], 0x07060302u);
        }
#pragma unroll
        for (int h = 0; h < kG; ++h)
#pragma unroll
          for (int d = 0; d < 8; ++d)
            o[h][d] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(ph[h]), as_bf16x2(vp[d]), o[h][d],
                                                      false);
      }
    }
  };

  auto rescale_o = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < kG; ++h) {
      const float a = lds.alpha[h];
#pragma unroll
      for (int d = 0; d < 8; ++d) o[h][d] *= a;
    }
  };

  // ---- main loop. Iteration gi computes QK^T of group gi, then P V of
  // group gi - 1 (its probabilities went to LDS one iteration earlier), so no
  // LDS round trip sits between the two halves. The ring starts full
  // (groups 0 .. kSlots-1); iteration gi >= 1 refills the slot of group
  // gi - 1 with group gi - 1 + kSlots once that group's V words are in
  // registers. So before group gi is used, the loads of groups up to
  // gi + kSlots - 1 (gi = 0) or gi + kSlots - 2 (gi >= 1) have been issued.
#pragma unroll
  for (int k = 0; k < R::kSlots; ++k)
    if (k < n_groups) issue(k);
  for (int gi = 0; gi <= n_groups; ++gi) {
    const int after = min(gi == 0 ? R::kSlots - 1 : R::kSlots - 2, n_groups - 1 - gi);
    if (after >= 3) wait_vm<3 * R::kDma>();
    else if (after == 2) wait_vm<2 * R::kDma>();
    else if (after == 1) wait_vm<R::kDma>();
    else wait_vm<0>();
    // (bf16 rows are twice as wide: their V words are read after QK^T so
    // that they do not hold registers through it)
    uint32_t vw[4][kVw];
    if (kE4M3 && gi > 0) read_v(gi - 1, vw);
    bool moved = false;
    if (gi < n_groups) moved = qk(gi);
    if (!kE4M3 && gi > 0) read_v(gi - 1, vw);
    if (gi > 0) {
      // the slot of group gi - 1 is free once its V words have arrived
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int k = 0; k < kVw; ++k) asm volatile("" : : "v"(vw[j][k]));
      if (gi - 1 + R::kSlots < n_groups) issue(gi - 1 + R::kSlots);
      pv(gi - 1, vw);
    }
    if (moved) rescale_o();
    __builtin_amdgcn_wave_barrier();
  }

  // ---- finish: denominators per head, accumulators over the 4 token lanes
  // lanes holding the same two heads differ only in the token bits 0..3
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    l[j] += __shfl_xor(l[j], 1);
    l[j] += __shfl_xor(l[j], 2);
    l[j] += __shfl_xor(l[j], 4);
    l[j] += __shfl_xor(l[j], 8);
  }
  if ((lane & 15) == 0) {
    lds.l[my_h0] = l[0];
    lds.l[my_h0 + 1] = l[1];
  }
  // reduce-scatter of o over the token lanes: heads {h, h+4} across lane
  // halves, then {h, h+2} across rows; each lane keeps two heads
  float o1[4][8];
#pragma unroll
  for (int h = 0; h < 4; ++h)
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const auto r = __builtin_amdgcn_permlane32_swap(f2u(o[h][d]), f2u(o[h + 4][d]), false, false);
      o1[h][d] = u2f(r[0]) + u2f(r[1]);
    }
  float o2[2][8];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const auto r = __builtin_amdgcn_permlane16_swap(f2u(o1[h][d]), f2u(o1[h + 2][d]), false, false);
      o2[h][d] = u2f(r[0]) + u2f(r[1]);
    }
  __builtin_amdgcn_wave_barrier();

  const int64_t bh0 = static_cast<int64_t>(b) * p.num_q_heads + g * kG;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int h = out_h[k];
    const float lh = lds.l[h];
    const float f = lh > 0.0f ? o_scale / lh : 0.0f;
    float* dst = p.o_part + ((bh0 + h) * p.max_splits + c) * kD + dg * 8;
    *reinterpret_cast<float4*>(dst) =
        make_float4(o2[k][0] * f, o2[k][1] * f, o2[k][2] * f, o2[k][3] * f);
    *reinterpret_cast<float4*>(dst + 4) =
        make_float4(o2[k][4] * f, o2[k][5] * f, o2[k][6] * f, o2[k][7] * f);
  }
  if (lane < kG) {
    const float lh = lds.l[lane];
    p.lse_part[(bh0 + lane) * p.max_splits + c] =
        lh > 0.0f ? (lds.m[lane] + __log2f(lh)) * kLn2 : -INFINITY;
  }
}

}  // namespace

bool gqa_fast_path_supported(int dk, int dv, int group, bool latent, int split_tokens,
                             int page_size) {
  return !latent && dk == kD && dv == kD && group == kG &&
         split_tokens <= kMaxUnitPages * page_size;
}

int launch_decode_gqa(const DecodeParams& p, bool e4m3, int n_split_blocks, int batch,
                      hipStream_t stream) {
  dim3 grid(n_split_blocks, p.num_kv_heads, batch);
  if (e4m3) {
    decode_gqa_kernel<true><<<grid, 64, 0, stream>>>(p);
  } else {
    decode_gqa_kernel<false><<<grid, 64, 0, stream>>>(p);
  }
  return pkv::launch_status();
}
