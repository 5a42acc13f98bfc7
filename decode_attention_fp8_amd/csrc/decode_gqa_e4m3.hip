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
// m per head, the largest score of the unit's first group. No rescale of the
// accumulators ever happens inside the loop; if any later score exceeds m by
// more than kRestart, the unit is recomputed once with m set to the unit's
// true maximum. Numerators are rounded to f16 (at most 2^kRestart, so they
// cannot overflow) for the PV products; the denominator sums them unrounded.
//
// PV. The numerators of a row's two heads are packed into f16 token pairs
// (tokens 2k, 2k + 1), exchanged through 256 bytes of LDS so every lane holds
// all four rows' packs, and again enter the dot products as row_newbcast
// operands. V is read with ds_read_tr8_b64, which gives lane i one dim of 8
// consecutive tokens, so token pairs come out of the converts already paired
// and each lane accumulates 8 heads x 2 dims over all 16 tokens.
//
// About 80 VGPRs and 12.5 KB of LDS per wave: three waves per SIMD.
#include <utility>

#include "common.h"
#include "decode_params.h"

namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef int v2i_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i_t lds_v2i_t;

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRestart = 15.0f;  // log2 headroom above the reference max
constexpr float kFloor = -1e30f;   // reference max of a unit with no valid token yet
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
      __builtin_amdgcn_update_dpp(0, static_cast<int>(f2u(v)), kCtrl, 0xf, 0xf, false)));
}
// Maximum / sum over the 16 lanes of a row, returned to every lane of it
// (xor 1, xor 2 within quads, then the half-row and row mirrors).
__device__ __forceinline__ float row_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x141>(v));
  return fmaxf(v, dpp<0x140>(v));
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

// Inclusive prefix sum over the wave.
__device__ __forceinline__ int wave_scan(int x) {
  const int lane = threadIdx.x;
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
__device__ bool find_unit(const DecodeParams& p, int u, int& b_out, int& g_out, int& c_out) {
  const int lane = threadIdx.x;
  const int S = p.split_tokens, H = p.num_kv_heads;
  auto splits = [&](int j) __attribute__((always_inline)) {
    int n = 0;
    if (j < p.batch) {
      const int L = p.seq_lens[j];
      const bool ab = p.abort_flags && p.abort_flags[j];
      if (!ab && L > 0 && L <= p.max_seq_len) n = (L + S - 1) / S;
    }
    return n;
  };
  int base = 0;  // full units of the requests before this batch of 64
  for (int b0 = 0; b0 < p.batch; b0 += 64) {
    const int n = splits(b0 + lane);
    const int full = n > 0 ? (n - 1) * H : 0;
    const int incl = wave_scan(full);
    const int total = __builtin_amdgcn_readlane(incl, 63);
    if (u < base + total) {
      const int bl = __popcll(__ballot(base + incl <= u));
      const int r = u - base - __builtin_amdgcn_readlane(incl - full, bl);
      b_out = b0 + bl;
      c_out = r / H;
      g_out = r - c_out * H;
      return true;
    }
    base += total;
  }
  int u2 = u - base;
  if (p.batch <= 64) {
    const int n = splits(lane);
    const int psz = n > 0 ? p.seq_lens[lane] - (n - 1) * S : -1;
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
    return true;
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
      return true;
    }
    u2 -= total;
  }
  return false;
}

template <int kSlots, int kWaves>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(kWaves)))
decode_gqa_e4m3_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[kSlots * kGroupBytes];
  __shared__ __attribute__((aligned(16))) uint32_t pbuf[16 * 4];  // [lane in row][row]
  __shared__ float fin[2][kG];                                    // l, m per head
  const int lane = threadIdx.x;
  int b, g, c;
  if (!find_unit(p, static_cast<int>(blockIdx.x), b, g, c)) return;
  const int L = p.seq_lens[b];
  const int t_begin = c * p.split_tokens;
  const int t_end = min(L, t_begin + p.split_tokens);
  const int n_groups = (t_end - t_begin + 15) >> 4;
  const int P = p.page_size;
  const int log2P = P == 16 ? 4 : (P == 32 ? 5 : 6);

  const int r = lane >> 4, i = lane & 15;
  const int tok = 2 * (i & 7) + (i >> 3);  // QK token of this lane
  const bool lo8 = i < 8;

  // query: qd[h] = bf16 pair (32r + 2i, 32r + 2i + 1) of head g*8 + h
  uint32_t qd[kG];
  {
    const uint32_t* qw = reinterpret_cast<const uint32_t*>(
        p.q + (static_cast<int64_t>(b) * p.num_q_heads + g * kG) * kD);
#pragma unroll
    for (int h = 0; h < kG; ++h) qd[h] = qw[h * (kD / 2) + 16 * r + i];
  }
  const float qk_scale = p.k_scale[g] * p.sm_scale_log2;
  const float o_scale = p.v_scale[g];

  // The unit's pages (at most 64): lane j holds the byte offset of the
  // (page j, kv head g) block, read back per group with readlane; bit j of
  // valid says whether page id j is inside the pool (an invalid page is
  // replaced by page 0 for the loads and its tokens are masked).
  const int64_t head_stride = static_cast<int64_t>(P) * kD;
  const int32_t* bt = p.block_table + static_cast<int64_t>(b) * p.max_pages;
  const int first_page = t_begin >> log2P;
  const int n_unit_pages = (t_end - t_begin + P - 1) >> log2P;
  int pg = -1;
  if (lane < n_unit_pages) pg = bt[first_page + lane];
  // Every compiler-issued load must be complete before the first DMA, or its
  // own wait for them would also wait for the ring.
  asm volatile("" : : "v"(qd[0]), "v"(qd[1]), "v"(qd[2]), "v"(qd[3]), "v"(qd[4]), "v"(qd[5]),
               "v"(qd[6]), "v"(qd[7]));
  asm volatile("" : : "v"(qk_scale), "v"(o_scale), "v"(pg));
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" : : : "memory");
  const bool pg_ok = pg >= 0 && pg < p.num_pages;
  const uint64_t valid = __ballot(pg_ok);
  const int64_t blk_off = (static_cast<int64_t>(pg_ok ? pg : 0) * p.num_kv_heads + g) * head_stride;
  const int off_lo = static_cast<int>(static_cast<uint32_t>(blk_off));
  const int off_hi = static_cast<int>(static_cast<uint32_t>(static_cast<uint64_t>(blk_off) >> 32));

  const uint8_t* kpool = static_cast<const uint8_t*>(p.k_pool);
  const uint8_t* vpool = static_cast<const uint8_t*>(p.v_pool);
  const uint32_t ring0 = lds_addr(ring);

  // DMA source offsets: lane L fills LDS chunk position L & 7 of row L >> 3
  // (first 1 KB) and of row 8 + (L >> 3) (second).
  const uint32_t dr0 = lane >> 3, dr1 = 8 + (lane >> 3), dpos = lane & 7;
  const uint32_t koff0 = dr0 * kD + ((dpos ^ kswz(dr0)) << 4);
  const uint32_t koff1 = dr1 * kD + ((dpos ^ kswz(dr1)) << 4);
  const uint32_t voff0 = dr0 * kD + ((dpos ^ vswz(dr0)) << 4);
  const uint32_t voff1 = dr1 * kD + ((dpos ^ vswz(dr1)) << 4);
  // LDS read offsets inside a slot: K chunks 2r, 2r + 1 of row tok; the
  // transposing V reads of octet o, chunk 2r + s address row 8o + (i >> 1).
  const uint32_t kr0 = tok * kD + (((2 * r) ^ kswz(tok)) << 4);
  const uint32_t kr1 = tok * kD + (((2 * r + 1) ^ kswz(tok)) << 4);
  uint32_t vr[2][2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int o = 0; o < 2; ++o) {
      const uint32_t t = 8 * o + (i >> 1);
      vr[s][o] = 2048 + t * kD + (((2 * r + s) ^ vswz(t)) << 4) + 8 * (i & 1);
    }

  auto group_tokens = [&](int gi) __attribute__((always_inline)) {
    const bool ok = ((valid >> ((gi << 4) >> log2P)) & 1u) != 0;
    return ok ? min(16, t_end - (t_begin + (gi << 4))) : 0;
  };
  auto issue = [&](int gi) __attribute__((always_inline)) {
    const int j = (gi << 4) >> log2P;
    const uint64_t off =
        (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(off_hi, j))) << 32) |
        static_cast<uint32_t>(__builtin_amdgcn_readlane(off_lo, j));
    const uint32_t row_off = static_cast<uint32_t>(((gi << 4) & (P - 1)) * kD);
    const uint8_t* kb = kpool + off + row_off;
    const uint8_t* vb = vpool + off + row_off;
    const uint32_t slot = ring0 + (gi % kSlots) * kGroupBytes;
    dma16(slot, koff0, kb);
    dma16(slot + 1024, koff1, kb);
    dma16(slot + 2048, voff0, vb);
    dma16(slot + 3072, voff1, vb);
  };

  float m_ref[2] = {kFloor, kFloor};
  float l[2], xmax[2];
  float o[kG][2];

  for (int pass = 0;; ++pass) {
    l[0] = l[1] = 0.0f;
    xmax[0] = xmax[1] = -INFINITY;
#pragma unroll
    for (int h = 0; h < kG; ++h) o[h][0] = o[h][1] = 0.0f;

#pragma unroll
    for (int k = 0; k < kSlots; ++k)
      if (k < n_groups) issue(k);

    for (int gi = 0; gi < n_groups; ++gi) {
      // groups gi + 1 .. gi + kSlots - 1 may still be in flight
      const int after = min(kSlots - 1, n_groups - 1 - gi);
      if (kSlots > 3 && after >= 3) wait_vm<12>();
      else if (kSlots > 2 && after >= 2) wait_vm<8>();
      else if (after >= 1) wait_vm<4>();
      else wait_vm<0>();

      const uint8_t* slot = ring + (gi % kSlots) * kGroupBytes;
      const uint4 kw0 = *reinterpret_cast<const uint4*>(slot + kr0);
      const uint4 kw1 = *reinterpret_cast<const uint4*>(slot + kr1);
      uint32_t vw[2][2][2];  // [chunk s][octet o][word]
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int o2 = 0; o2 < 2; ++o2) {
          const v2i_t x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_t*)(slot + vr[s][o2]));
          vw[s][o2][0] = static_cast<uint32_t>(x[0]);
          vw[s][o2][1] = static_cast<uint32_t>(x[1]);
        }
      // the slot is free once its bytes are in registers
      asm volatile("" : : "v"(kw0.x), "v"(kw0.y), "v"(kw0.z), "v"(kw0.w), "v"(kw1.x), "v"(kw1.y),
                   "v"(kw1.z), "v"(kw1.w));
      asm volatile("" : : "v"(vw[0][0][0]), "v"(vw[0][0][1]), "v"(vw[0][1][0]), "v"(vw[0][1][1]),
                   "v"(vw[1][0][0]), "v"(vw[1][0][1]), "v"(vw[1][1][0]), "v"(vw[1][1][1]));
      if (gi + kSlots < n_groups) issue(gi + kSlots);

      const int nv = group_tokens(gi);
      if (nv < 16) {
        // tokens past the context or of an invalid page: V bytes to 0
#pragma unroll
        for (int o2 = 0; o2 < 2; ++o2) {
          const int vo = min(8, max(0, nv - 8 * o2));
          const uint64_t m64 = vo >= 8 ? ~0ull : ((1ull << (8 * vo)) - 1ull);
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            vw[s][o2][0] &= static_cast<uint32_t>(m64);
            vw[s][o2][1] &= static_cast<uint32_t>(m64 >> 32);
          }
        }
      }

      // ---- QK^T: row partial dots of token tok for the 8 heads
      float a[kG];
#pragma unroll
      for (int h = 0; h < kG; ++h) a[h] = 0.0f;
      const uint32_t kw[8] = {kw0.x, kw0.y, kw0.z, kw0.w, kw1.x, kw1.y, kw1.z, kw1.w};
      unroll<8>([&](auto wc) {
        constexpr int w = decltype(wc)::value;
        const uint32_t x0 = __builtin_bit_cast(
            uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(kw[w], 1.0f, false));
        const uint32_t x1 = __builtin_bit_cast(
            uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(kw[w], 1.0f, true));
        unroll<kG>([&](auto hc) {
          constexpr int h = decltype(hc)::value;
          a[h] = dot2_bf16_bcast<2 * w>(a[h], qd[h], x0);
        });
        unroll<kG>([&](auto hc) {
          constexpr int h = decltype(hc)::value;
          a[h] = dot2_bf16_bcast<2 * w + 1>(a[h], qd[h], x1);
        });
      });
      // reduce-scatter over the four rows: row r keeps heads 2r, 2r + 1
      float u[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const auto rr = __builtin_amdgcn_permlane32_swap(f2u(a[h]), f2u(a[h + 4]), false, false);
        u[h] = u2f(rr[0]) + u2f(rr[1]);
      }
      float raw[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const auto rr = __builtin_amdgcn_permlane16_swap(f2u(u[j]), f2u(u[j + 2]), false, false);
        const float sc = (u2f(rr[0]) + u2f(rr[1])) * qk_scale;
        raw[j] = tok < nv ? sc : -INFINITY;
      }
      if (pass == 0 && gi == 0) {
#pragma unroll
        for (int j = 0; j < 2; ++j) m_ref[j] = fmaxf(row_max(raw[j]), kFloor);
      }

      // ---- softmax numerators, packed into f16 token pairs
      float pr[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        xmax[j] = fmaxf(xmax[j], raw[j]);
        pr[j] = __builtin_amdgcn_exp2f(raw[j] - m_ref[j]);
        l[j] += pr[j];
      }
      // lanes i and i ^ 8 hold tokens 2(i & 7) and 2(i & 7) + 1: lane i < 8
      // packs head 2r, lane i >= 8 head 2r + 1, both for pair k = i & 7
      const float send = lo8 ? pr[1] : pr[0];
      const float recv = dpp<0x128>(send);  // row_ror:8
      const float lo = lo8 ? pr[0] : recv;
      const float hi = lo8 ? recv : pr[1];
      const half2_t ph = {static_cast<_Float16>(lo), static_cast<_Float16>(hi)};
      pbuf[i * 4 + r] = __builtin_bit_cast(uint32_t, ph);
      __builtin_amdgcn_wave_barrier();
      const uint4 G4 = *reinterpret_cast<const uint4*>(&pbuf[i * 4]);
      const uint32_t Gp[4] = {G4.x, G4.y, G4.z, G4.w};  // Gp[j]: heads 2j (lanes 0-7), 2j+1 (8-15)

      // ---- PV: o[h][s] += sum over token pairs k of p[h][2k..2k+1] . v
      unroll<2>([&](auto sc_) {
        constexpr int s = decltype(sc_)::value;
        unroll<4>([&](auto wc) {
          constexpr int ow = decltype(wc)::value;  // octet ow >> 1, word ow & 1
          const uint32_t word = vw[s][ow >> 1][ow & 1];
          const uint32_t v0 = __builtin_bit_cast(
              uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word, 1.0f, false));
          const uint32_t v1 = __builtin_bit_cast(
              uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word, 1.0f, true));
          constexpr int k0 = 2 * ow;  // pair index of v0 (tokens 4ow, 4ow + 1)
          unroll<kG>([&](auto hc) {
            constexpr int h = decltype(hc)::value;
            o[h][s] = dot2_f16_bcast<8 * (h & 1) + k0>(o[h][s], Gp[h >> 1], v0);
          });
          unroll<kG>([&](auto hc) {
            constexpr int h = decltype(hc)::value;
            o[h][s] = dot2_f16_bcast<8 * (h & 1) + k0 + 1>(o[h][s], Gp[h >> 1], v1);
          });
        });
      });
    }

    // ---- a later score above the reference max by more than kRestart:
    // recompute the unit once with the true maximum
    float xm[2];
    bool over = false;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      xm[j] = row_max(xmax[j]);
      over = over || (xm[j] > m_ref[j] + kRestart);
    }
    if (pass > 0 || !__any(over)) break;
#pragma unroll
    for (int j = 0; j < 2; ++j) m_ref[j] = fmaxf(xm[j], kFloor);
  }

  // ---- finish: denominators per head, then o / l for this lane's 16 values
  float ls[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) ls[j] = row_sum(l[j]);
  if (i == 0) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      fin[0][2 * r + j] = ls[j];
      fin[1][2 * r + j] = m_ref[j];
    }
  }
  __builtin_amdgcn_wave_barrier();
  const int64_t bh0 = static_cast<int64_t>(b) * p.num_q_heads + g * kG;
#pragma unroll
  for (int h = 0; h < kG; ++h) {
    const float lh = fin[0][h];
    const float f = lh > 0.0f ? o_scale / lh : 0.0f;
    float* dst = p.o_part + ((bh0 + h) * p.max_splits + c) * kD + 32 * r + i;
    dst[0] = o[h][0] * f;
    dst[16] = o[h][1] * f;
  }
  if (lane < kG) {
    const float lh = fin[0][lane];
    p.lse_part[(bh0 + lane) * p.max_splits + c] =
        lh > 0.0f ? (fin[1][lane] + __log2f(lh)) * kLn2 : -INFINITY;
  }
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
  decode_gqa_e4m3_kernel<3, 3><<<dim3(static_cast<uint32_t>(units)), 64, 0, stream>>>(p);
  return pkv::launch_status();
}
