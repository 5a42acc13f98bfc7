// Grouped-query decode with head dim 128 on MFMA, e4m3 or bf16 cache, one
// work unit per wave in the hardware dispatcher's order.
//
// "Smaller, faster, safer: running Kimi and GLM at scale" (Cloudflare blog),
// section "Quantizing the KV cache": K and V are held as e4m3 and the
// attention kernel converts codes as it reads them; the bf16 cache it is
// compared with is read as stored. The tile math (QK^T and PV on MFMA
// 16x16x32, the softmax) is that of gqa_mfma_tile.h, in the same layouts for
// both: only the bytes per value, the conversion and the LDS swizzles differ.
//
// One wave per work unit (request, kv head, split), in the one-dimensional
// longest-first order of find_unit. A split runs in tiles of 32 tokens whose
// K and V bytes (4 KB each for e4m3, 8 KB for bf16) travel HBM -> LDS by
// direct-to-LDS loads into a ring of kSlots tiles. With scales set at append
// (one per row), a tile's 32 K and 32 V row scales travel with it (two more
// loads, 512 bytes of slot).
//
// In the step form (kStep) the kernel also does the two things a separate
// launch did before it ("Smaller, faster, safer", section "Protecting a
// shared KV cache": the mapping is checked before anything is returned from
// the request's pages, and an aborted request writes nothing). The units of
// kv head 0 check their split's pages (in the pool, pool tag equal to the
// recorded one) and write the verdict for (request, split); the splits of a
// request cover its pages, so the combine launch ORs them into the request's
// flag. And the unit holding a request's last token (the one appended this
// step) takes its K and V row from the new token's values, encoded as the
// append encodes them, in place of the pool row it loaded: the pool row is
// written by the combine launch, once the request is known to stand.
#include <type_traits>

#include "common.h"
#include "decode_params.h"
#include "gqa_mfma_tile.h"
#include "unit_order.h"

namespace {

using namespace gqa_mfma;

constexpr int kPageVecs = 4;  // page offsets per lane
constexpr int kMaxUnitPages = 64 * kPageVecs;
constexpr int kStepMaxUnitPages = 128;  // step form: tags of two page vectors in registers

// every tile is L loads; wait until only the `ahead` younger tiles remain
template <int N, int L>
__device__ __forceinline__ void wait_tiles(int ahead) {
  if (N >= 3 && ahead >= 3) {
    wait_vm<3 * L>();
  } else if (N >= 2 && ahead >= 2) {
    wait_vm<2 * L>();
  } else if (ahead >= 1) {
    wait_vm<L>();
  } else {
    wait_vm<0>();
  }
}

template <int kSlots, bool kRowScales, bool kBf16 = false, bool kStep = false>
__global__ void __launch_bounds__(64) decode_gqa_mfma_kernel(DecodeParams p) {
  static_assert(kSlots >= 2 && kSlots <= 4, "ring of 2 to 4 tiles");
  static_assert(!(kBf16 && kRowScales), "row scales are for e4m3 caches");
  static_assert(!(kStep && kRowScales), "the step form takes static scales or bf16");
  constexpr int kElem = kBf16 ? 2 : 1;
  constexpr int kSlotBytes = (kBf16 ? bf16c::kTileBytes : kTileBytes) + (kRowScales ? 512 : 0);
  constexpr int kLoads = kBf16 ? 16 : (kRowScales ? 10 : 8);  // loads per tile
  __shared__ __attribute__((aligned(16))) uint8_t ring[kSlots * kSlotBytes];
  const int lane = threadIdx.x;
  const int col = lane & 15, qg = lane >> 4;
  // The unit: with one request, unit u is split u / Hkv of kv head u % Hkv
  // (the work-unit order reduces to that), so its q, page ids and recorded
  // tags are loaded beside the request's length, one memory latency instead
  // of two, and the entries past the length are dropped once it is in.
  int b, g, c, L;
  const bool one_req = p.batch == 1;
  if (one_req) {
    c = static_cast<int>(blockIdx.x) / p.num_kv_heads;
    g = static_cast<int>(blockIdx.x) - c * p.num_kv_heads;
    b = 0;
    L = 0;
  } else if (!pkv::find_unit(p, static_cast<int>(blockIdx.x), b, g, c, L)) {
    return;
  }
  const int G = p.num_q_heads / p.num_kv_heads;
  const int t_begin = c * p.split_tokens;
  const int P = p.page_size;
  const int log2P = P == 16 ? 4 : (P == 32 ? 5 : 6);
  const int first_page = t_begin >> log2P;
  // pages loaded: the unit's, or with one request the whole split's (within
  // the block-table row: the launch has ceil(max_seq_len / S) splits)
  const int load_pages = one_req ? min(p.split_tokens >> log2P, p.max_pages - first_page)
                                 : (min(L, t_begin + p.split_tokens) - t_begin + P - 1) >> log2P;

  // query head col as B operands (heads G .. 15 are zero rows): k-step s,
  // slot 8 qg + j <-> dim 32 qg + 8 s + j. Every lane loads (a padding lane
  // reads head 0's row) and the padding rows are zeroed once the loads are
  // in: zeroing registers a load is still writing would make the first load
  // complete before the others are issued.
  const bool head_ok = col < G;
  bf16x8_t qf[4];
  {
    const uint16_t* qrow =
        p.q + (static_cast<int64_t>(b) * p.num_q_heads + g * G + (head_ok ? col : 0)) * kD +
        32 * qg;
#pragma unroll
    for (int s = 0; s < 4; ++s) qf[s] = *reinterpret_cast<const bf16x8_t*>(qrow + 8 * s);
  }
  // row scales: each row's own, applied per token in the tile math
  const float qk_scale = (kRowScales || kBf16) ? p.sm_scale_log2 : p.k_scale[g] * p.sm_scale_log2;
  const float o_scale = (kRowScales || kBf16) ? 1.0f : p.v_scale[g];

  // the unit's pages: lane j holds the byte offsets of (page 64 h + j, kv
  // head g) in vector h < kPageVecs (named variables, so that selecting one
  // by a uniform index stays in registers)
  const int32_t* bt = p.block_table + static_cast<int64_t>(b) * p.max_pages;
  auto load_page = [&](int h) __attribute__((always_inline)) {
    return 64 * h + lane < load_pages ? bt[first_page + 64 * h + lane] : -1;
  };
  int pg0 = load_page(0), pg1 = load_page(1), pg2 = load_page(2), pg3 = load_page(3);
  // with one request: its length and abort flag
  int L1 = 0, ab1 = 0;
  if (one_req) {
    L1 = p.seq_lens[0];
    if (p.abort_flags) ab1 = p.abort_flags[0];
  }
  // step form: the recorded tags of the unit's pages (kv head 0's units),
  // and the new token's K and V values (the request's last unit; with one
  // request every unit loads them, 256 bytes): lanes 0 .. 2 kNewChunks - 1
  // each hold one 16-byte chunk of a row, K first
  const bool checker = kStep && g == 0 && p.expected_tags != nullptr;
  constexpr int kNewChunks = kBf16 ? 16 : 8;  // chunks of a 128-value row
  uint32_t want0 = 0, want1 = 0;  // a step-form unit has at most 128 pages
  uint4 nw0 = make_uint4(0u, 0u, 0u, 0u), nw1 = nw0;
  if constexpr (kStep) {
    if (checker) {
      const uint32_t* er = p.expected_tags + static_cast<int64_t>(b) * p.max_pages + first_page;
      auto load_want = [&](int h) __attribute__((always_inline)) {
        return 64 * h + lane < load_pages ? er[64 * h + lane] : 0u;
      };
      want0 = load_want(0), want1 = load_want(1);
    }
    if ((one_req || min(L, t_begin + p.split_tokens) == L) && lane < 2 * kNewChunks) {
      const int ch = lane & (kNewChunks - 1);
      const uint16_t* src = (lane < kNewChunks ? p.k_new : p.v_new) +
                            (static_cast<int64_t>(b) * p.num_kv_heads + g) * kD +
                            (kBf16 ? 8 : 16) * ch;
      nw0 = *reinterpret_cast<const uint4*>(src);
      if constexpr (!kBf16) nw1 = *reinterpret_cast<const uint4*>(src + 8);
    }
  }
#pragma unroll
  for (int s = 0; s < 4; ++s) asm volatile("" : : "v"(qf[s]));
  asm volatile("" : : "v"(pg0), "v"(pg1), "v"(pg2), "v"(pg3));
  asm volatile("" : : "v"(qk_scale), "v"(o_scale));
  asm volatile("" : : "v"(L1), "v"(ab1));
  // from here on the only vector memory loads in flight are the ring's
  // (and, in the step form, the pool tags issued before them)
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" : : : "memory");
  if (one_req) {
    // the unit exists if the request has this split (as the work-unit
    // lookup would decide); the split's page entries past it are dropped
    L = __builtin_amdgcn_readfirstlane(L1);
    const int n = (__builtin_amdgcn_readfirstlane(ab1) == 0 && L > 0 && L <= p.max_seq_len)
                      ? (L + p.split_tokens - 1) / p.split_tokens
                      : 0;
    if (c >= n) return;
  }
  const int t_end = min(L, t_begin + p.split_tokens);
  const int n_tiles = (t_end - t_begin + kTile - 1) / kTile;
  const int n_pages = (t_end - t_begin + P - 1) >> log2P;
  if (one_req) {
    auto keep = [&](int h, int v) __attribute__((always_inline)) {
      return 64 * h + lane < n_pages ? v : -1;
    };
    pg0 = keep(0, pg0), pg1 = keep(1, pg1), pg2 = keep(2, pg2), pg3 = keep(3, pg3);
  }
  const bool inject = kStep && t_end == L;
  if (!head_ok) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[s][e] = static_cast<__bf16>(0.0f);
  }
  auto page_ok_lane = [&](int pg) __attribute__((always_inline)) {
    return pg >= 0 && pg < p.num_pages;
  };
  auto page_off = [&](int pg) __attribute__((always_inline)) {
    return (static_cast<int64_t>(page_ok_lane(pg) ? pg : 0) * p.num_kv_heads + g) *
           (static_cast<int64_t>(P) * kD * kElem);
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
  // step form: the pool tags of the unit's pages, loaded before the ring's
  // first tiles (so the ring's waits cover them) and compared at the end
  uint32_t have0 = 0, have1 = 0;
  if constexpr (kStep) {
    if (checker) {
      auto load_have = [&](int pg) __attribute__((always_inline)) {
        return page_ok_lane(pg) ? p.page_tags[pg] : 0u;
      };
      have0 = load_have(pg0), have1 = load_have(pg1);
    }
  }

  const uint8_t* kpool = static_cast<const uint8_t*>(p.k_pool);
  const uint8_t* vpool = static_cast<const uint8_t*>(p.v_pool);
  const uint32_t ring0 = lds_addr(ring);
  using Offsets = std::conditional_t<kBf16, bf16c::LaneOffsets, LaneOffsets>;
  Offsets lo;
  if constexpr (kBf16) {
    lo = bf16c::lane_offsets(lane);
  } else {
    lo = lane_offsets(lane);
  }

  auto group_base = [&](int gg) __attribute__((always_inline)) {
    const int j = (gg << 4) >> log2P;
    const int h = j >> 6, jl = j & 63;
    const int64_t o = pick4(h, off0, off1, off2, off3);
    const uint64_t off =
        (static_cast<uint64_t>(static_cast<uint32_t>(
             __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint64_t>(o) >> 32), jl)))
         << 32) |
        static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(o), jl));
    return off + static_cast<uint32_t>(((gg << 4) & (P - 1)) * kD * kElem);
  };
  // kLoads loads per tile, always: a 16-token group past the unit's end
  // loads the tile's first group again (its scores are masked and its V rows
  // zeroed)
  auto issue = [&](int t) __attribute__((always_inline)) {
    const uint32_t slot = ring0 + (t % kSlots) * kSlotBytes;
    uint64_t offs[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int gg = (t_begin + kTile * t + 16 * x < t_end) ? 2 * t + x : 2 * t;
      offs[x] = group_base(gg);
      if constexpr (kBf16) {
        bf16c::dma_group(slot, x, lo, kpool + offs[x], vpool + offs[x]);
      } else {
        dma_group(slot, x, lo, kpool + offs[x], vpool + offs[x]);
      }
    }
    if constexpr (kRowScales) {
      // a row's scale sits at 4 bytes per 128 of its codes; lanes 0..31 load
      // the tile rows' scales (lanes 32..63 repeat them)
      const uint32_t so = static_cast<uint32_t>(((lane >> 4) & 1 ? offs[1] : offs[0]) >> 5) +
                          4u * (lane & 15);
      const uint8_t* ks = reinterpret_cast<const uint8_t*>(p.k_row_scale);
      const uint8_t* vs = reinterpret_cast<const uint8_t*>(p.v_row_scale);
      dma4_stream(slot + kTileBytes, so, ks);
      dma4_stream(slot + kTileBytes + 256, so, vs);
    }
  };

  Acc a;
  acc_init(a);
#pragma unroll
  for (int k = 0; k < kSlots - 1; ++k)
    if (k < n_tiles) issue(k);
  // step form: the new token's codes (e4m3, encoded as the append encodes
  // them, under the kv head's static scales) or values (bf16)
  uint4 nrow = nw0;
  if constexpr (kStep && !kBf16) {
    if (inject && lane < 2 * kNewChunks)
      nrow = pkv::encode16(nw0, nw1, lane < kNewChunks ? p.k_scale[g] : p.v_scale[g]);
  }
  for (int t = 0; t < n_tiles; ++t) {
    if (t + kSlots - 1 < n_tiles) issue(t + kSlots - 1);
    wait_tiles<kSlots - 1, kLoads>(min(kSlots - 1, n_tiles - 1 - t));
    const int tile0 = t_begin + kTile * t;
    const bool g0_ok = page_ok(((2 * t) << 4) >> log2P);
    const bool g1_ok = tile0 + 16 < t_end && page_ok(((2 * t + 1) << 4) >> log2P);
    uint8_t* buf = ring + (t % kSlots) * kSlotBytes;
    if constexpr (kStep) {
      if (inject && t == n_tiles - 1) {
        // the last token's row of the tile (the ring loaded the pool's old
        // row there); chunk c of row r sits at the tile layout's position
        const uint32_t r = static_cast<uint32_t>(L - 1 - tile0);
        const uint32_t c = static_cast<uint32_t>(lane & (kNewChunks - 1));
        if (lane < 2 * kNewChunks) {
          uint32_t off;
          if constexpr (kBf16) {
            off = lane < kNewChunks ? r * 2 * kD + ((c ^ bf16c::kswz(r)) << 4)
                                    : bf16c::kHalf + r * 2 * kD + ((c ^ bf16c::vswz(r)) << 4);
          } else {
            off = lane < kNewChunks ? r * kD + ((c ^ kswz(r)) << 4)
                                    : kHalf + r * kD + ((c ^ vswz(r)) << 4);
          }
          *reinterpret_cast<uint4*>(buf + off) = nrow;
        }
        __builtin_amdgcn_wave_barrier();
      }
    }
    if constexpr (kBf16) {
      bf16c::tile_math(buf, lo, qf, qk_scale, g0_ok, g1_ok, min(kTile, t_end - tile0), a);
    } else {
      tile_math<kRowScales>(buf, lo, qf, qk_scale, g0_ok, g1_ok, min(kTile, t_end - tile0),
                            a, reinterpret_cast<const float*>(buf + kTileBytes));
    }
  }
  // scales set at append: O is relative to the unit's V reference scale
  finish(p, b, g, c, G, kRowScales ? a.vref : o_scale, a);
  if constexpr (kStep) {
    if (checker) {
      // a page of the unit outside the pool, or whose pool tag differs from
      // the recorded one, aborts the request
      auto bad = [&](int h, int pg, uint32_t have, uint32_t want) __attribute__((always_inline)) {
        return 64 * h + lane < n_pages && (!page_ok_lane(pg) || have != want);
      };
      const bool unit_bad = __any(bad(0, pg0, have0, want0) || bad(1, pg1, have1, want1));
      if (lane == 0) p.unit_flags[static_cast<int64_t>(b) * p.max_splits + c] = unit_bad ? 1 : 0;
    }
  }
}

}  // namespace

bool gqa_mfma_path_supported(int dk, int dv, int group, bool latent, int split_tokens,
                             int page_size) {
  return !latent && dk == kD && dv == kD && group >= 1 && group <= kRows &&
         split_tokens <= kMaxUnitPages * page_size;
}

int launch_decode_gqa_mfma(const DecodeParams& p, bool e4m3, int n_split_blocks, int batch,
                           hipStream_t stream) {
  const int64_t units = static_cast<int64_t>(n_split_blocks) * p.num_kv_heads * batch;
  if (units > 0x7FFFFFFF) return PKV_EUNSUPPORTED;
  if (!e4m3) {
    decode_gqa_mfma_kernel<2, false, true><<<dim3(static_cast<uint32_t>(units)), 64, 0, stream>>>(p);
    return pkv::launch_status();
  }
  if (p.k_row_scale) {
    // row-scale offsets are 32-bit
    if (static_cast<int64_t>(p.num_pages) * p.num_kv_heads * p.page_size * 4 > 0xFFFFFFFFLL)
      return PKV_EUNSUPPORTED;
    decode_gqa_mfma_kernel<2, true><<<dim3(static_cast<uint32_t>(units)), 64, 0, stream>>>(p);
  } else {
    decode_gqa_mfma_kernel<2, false><<<dim3(static_cast<uint32_t>(units)), 64, 0, stream>>>(p);
  }
  return pkv::launch_status();
}

int launch_decode_gqa_mfma_step(const DecodeParams& p, bool e4m3, int n_split_blocks, int batch,
                                hipStream_t stream) {
  const int64_t units = static_cast<int64_t>(n_split_blocks) * p.num_kv_heads * batch;
  if (units > 0x7FFFFFFF || p.k_row_scale || !p.unit_flags ||
      p.split_tokens > kStepMaxUnitPages * p.page_size)
    return PKV_EUNSUPPORTED;
  if (e4m3)
    decode_gqa_mfma_kernel<2, false, false, true>
        <<<dim3(static_cast<uint32_t>(units)), 64, 0, stream>>>(p);
  else
    decode_gqa_mfma_kernel<2, false, true, true>
        <<<dim3(static_cast<uint32_t>(units)), 64, 0, stream>>>(p);
  return pkv::launch_status();
}
