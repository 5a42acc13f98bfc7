// Decode attention of a token and its drafts verified together, over an e4m3
// cache with head dim 128.
//
// Cloudflare's post on serving extra-large models, speculative decoding
// section: a small draft model proposes a few future tokens, and the target
// model accepts or rejects them in one forward pass. In that pass each
// request has q_len query positions (the current token and q_len - 1 drafts,
// whose K and V were appended this step); query j sees the cached tokens up
// to and including its own position L - q_len + j. "Smaller, faster, safer",
// section "Quantizing the KV cache": the cache is read as e4m3 and converted
// on the way in.
//
// With G query heads per kv head, a kv head serves q_len * G query rows, so
// QK^T and PV are real dense contractions (32 rows for 4 positions of 8
// heads): this kernel runs them on MFMA 32x32x16 with fp32 accumulation, QK^T
// in bf16 (the query is bf16; K codes convert exactly) and PV in f16 (V codes
// convert exactly; numerators rounded to f16, 3 bits more than bf16).
//
// One wave per work unit (request, kv head, split, group of 32 query rows),
// in the unit order of the one-dimensional launches. The split is processed
// in tiles of 32 tokens; a tile's K and V bytes (4 KB each) travel HBM -> LDS
// by direct-to-LDS loads into a ring of kSlots tiles.
//
// MFMA operand layouts (32x32x16, lane l, c = l % 32, h = l / 32):
//   A: row c, k 8h .. 8h+7;  B: column c, k 8h .. 8h+7;
//   D element i: row 8(i/4) + 4h + i%4, column c.
// S^T = K Q^T per tile (M = tokens, N = query rows, 8 k-steps of 16 dims:
// k-step s covers dims 32(s/2) + 16h + 8(s%2) .. +7, so one 16-byte K read
// serves two k-steps). A lane then holds query row c's scores for tokens
// {8(i/4) + 4h + i%4}; those are the A operand of O += P V (M = query rows,
// k = tokens) once V is read in the same token order with ds_read_tr8_b64,
// which hands lane i of a 16-lane group byte i (one dim) of 8 rows.
//
// Softmax: log2 domain, per query row a reference max set by the row's first
// valid scores; a later score more than kTau above it raises it and rescales
// the row's accumulators (a uniform branch real scores almost never take), so
// numerators stay at most 2^kTau, inside f16 range.
#include "common.h"
#include "decode_params.h"
#include "mfma_tile.h"
#include "unit_order.h"

namespace {

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTau = 15.0f;      // f16 numerators stay at most 2^kTau
constexpr float kMUnset = -1e30f;  // reference max of a row with no valid score yet
constexpr int kD = 128;
constexpr int kTile = 32;                    // tokens per tile
constexpr int kHalf = kTile * kD;            // K (or V) bytes of a tile
constexpr int kTileBytes = 2 * kHalf;        // K then V: 8 KB
constexpr int kSlots = 2;
constexpr int kMaxUnitPages = 128;  // two vectors of page ids per lane

// Tile layouts: K chunk c of token row t at c ^ ((t >> 1) & 7) (the 32 rows
// a K read touches at one chunk land on distinct bank groups); V chunk c of
// row t at c ^ vswz(t), vswz(t) = bits 1 and 3 of t moved to bits 1 and 2
// (the 8 rows x 2 chunks of a half-wave's transposing read, likewise).
__device__ __forceinline__ uint32_t kswz(uint32_t t) { return (t >> 1) & 7u; }
__device__ __forceinline__ uint32_t vswz(uint32_t t) {
  return (((t >> 1) & 1u) << 1) | (((t >> 3) & 1u) << 2);
}

// W waves per workgroup, one group of 32 query rows each, share every tile:
// each wave issues 8 / W of the tile's loads, one barrier per tile makes the
// whole tile visible and frees the slot two tiles ahead (three slots). With
// W = 1 the wave runs its own two-slot ring without barriers. Up to two
// waves a workgroup the registers are held to 168, three waves per SIMD
// (they fit without spilling; four and eight waves would spill).
template <int W>
__global__ void __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(W <= 2 ? 3 : 1)))
decode_drafts_kernel(DecodeParams p, int row_groups) {
  constexpr int kRing = W == 1 ? kSlots : 3;
  constexpr int kMine = 8 / W;  // loads per tile issued by each wave
  __shared__ __attribute__((aligned(16))) uint8_t ring[kRing * kTileBytes];
  __shared__ float rowbufs[W][2][32];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  float (*rowbuf)[32] = rowbufs[wv];
  const int col = lane & 31, hl = lane >> 5;
  const int parts = (row_groups + W - 1) / W;
  const int rg = (static_cast<int>(blockIdx.x) % parts) * W + wv;
  int b, g, c, L;
  if (!pkv::find_unit(p, static_cast<int>(blockIdx.x) / parts, b, g, c, L)) return;
  const int G = p.num_q_heads / p.num_kv_heads;
  const int T = p.q_len;
  const int rows = T * G;
  const int t_begin = c * p.split_tokens;
  const int t_end = min(L, t_begin + p.split_tokens);
  const int n_tiles = (t_end - t_begin + kTile - 1) / kTile;
  const int P = p.page_size;
  const int log2P = P == 16 ? 4 : (P == 32 ? 5 : 6);

  // this lane's query row (S^T column): position j, head g*G + hh (a wave
  // past the last row group only helps with the loads)
  const int r_mine = 32 * rg + col;
  const bool row_ok = rg < row_groups && r_mine < rows;
  const int j_mine = row_ok ? r_mine / G : 0;
  // tokens this row may see inside the unit: [t_begin, lim)
  const int lim = row_ok ? min(t_end, L - T + j_mine + 1) : t_begin;

  // query as B operands: k-step s covers dims 32(s/2) + 16h + 8(s%2) .. +7.
  // Every lane loads (a lane past the rows reads row 0) and those lanes'
  // operands are zeroed once the loads are in: zeroing registers a load is
  // still writing would make the first load complete before the others are
  // issued.
  bf16x8_t qf[8];
  {
    const int hh = row_ok ? r_mine - j_mine * G : 0;
    const uint16_t* qrow =
        p.q + ((static_cast<int64_t>(b) * T + j_mine) * p.num_q_heads + g * G + hh) * kD;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      qf[s] = *reinterpret_cast<const bf16x8_t*>(qrow + 32 * (s >> 1) + 16 * hl + 8 * (s & 1));
  }
  const float qk_scale = p.k_scale[g] * p.sm_scale_log2;
  const float o_scale = p.v_scale[g];

  // the unit's pages: lane j holds the byte offset of (page j, kv head g)
  const int32_t* bt = p.block_table + static_cast<int64_t>(b) * p.max_pages;
  const int first_page = t_begin >> log2P;
  const int n_pages = (t_end - t_begin + P - 1) >> log2P;
  // the unit's pages: lane j holds pages j and 64 + j
  int pg = -1, pgh = -1;
  if (lane < n_pages) pg = bt[first_page + lane];
  if (64 + lane < n_pages) pgh = bt[first_page + 64 + lane];
#pragma unroll
  for (int s = 0; s < 8; ++s) asm volatile("" : : "v"(qf[s]));
  asm volatile("" : : "v"(qk_scale), "v"(o_scale), "v"(pg), "v"(pgh));
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" : : : "memory");
  if (!row_ok) {
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[s][e] = static_cast<__bf16>(0.0f);
  }
  const bool pg_ok = pg >= 0 && pg < p.num_pages;
  const bool pgh_ok = pgh >= 0 && pgh < p.num_pages;
  const uint64_t valid = __ballot(pg_ok), validh = __ballot(pgh_ok);
  auto block_of = [&](int page, bool ok) __attribute__((always_inline)) {
    return (static_cast<int64_t>(ok ? page : 0) * p.num_kv_heads + g) *
           (static_cast<int64_t>(P) * kD);
  };
  const int64_t blk = block_of(pg, pg_ok), blkh = block_of(pgh, pgh_ok);
  const int off_lo = static_cast<int>(static_cast<uint32_t>(blk));
  const int off_hi = static_cast<int>(static_cast<uint32_t>(static_cast<uint64_t>(blk) >> 32));
  const int offh_lo = static_cast<int>(static_cast<uint32_t>(blkh));
  const int offh_hi = static_cast<int>(static_cast<uint32_t>(static_cast<uint64_t>(blkh) >> 32));
  // page j of the unit is valid (j < 128; a uniform choice of vector)
  auto page_valid = [&](int j) __attribute__((always_inline)) {
    return (((j < 64 ? valid : validh) >> (j & 63)) & 1u) != 0;
  };

  // DMA source offsets inside a 16-token group block: lane L fills LDS chunk
  // position L & 7 of group row L >> 3 (first 1 KB) and 8 + (L >> 3)
  const uint32_t dr0 = lane >> 3, dr1 = 8 + (lane >> 3), dpos = lane & 7;
  const uint32_t koff0 = dr0 * kD + ((dpos ^ kswz(dr0)) << 4);
  const uint32_t koff1 = dr1 * kD + ((dpos ^ kswz(dr1)) << 4);
  const uint32_t voff0 = dr0 * kD + ((dpos ^ vswz(dr0)) << 4);
  const uint32_t voff1 = dr1 * kD + ((dpos ^ vswz(dr1)) << 4);
  const uint8_t* kpool = static_cast<const uint8_t*>(p.k_pool);
  const uint8_t* vpool = static_cast<const uint8_t*>(p.v_pool);
  const uint32_t ring0 = lds_addr(ring);

  auto group_base = [&](int gg) __attribute__((always_inline)) {
    const int j = (gg << 4) >> log2P;
    const uint64_t off =
        (static_cast<uint64_t>(static_cast<uint32_t>(
             __builtin_amdgcn_readlane(j < 64 ? off_hi : offh_hi, j & 63)))
         << 32) |
        static_cast<uint32_t>(__builtin_amdgcn_readlane(j < 64 ? off_lo : offh_lo, j & 63));
    return off + static_cast<uint32_t>(((gg << 4) & (P - 1)) * kD);
  };
  // 8 loads per tile, always: a 16-token group past the unit's end loads the
  // tile's first group again (its rows are masked and their V zeroed). Load
  // j = 4 x + kind: group x of the tile, kind 0 / 1 the K rows 0..7 / 8..15,
  // 2 / 3 the V rows; wave wv issues j = wv, wv + W, ...
  auto issue = [&](int t) __attribute__((always_inline)) {
    const uint32_t slot = ring0 + (t % kRing) * kTileBytes;
    uint32_t dst[kMine], src[kMine];
    const uint8_t* from[kMine];
#pragma unroll
    for (int i = 0; i < kMine; ++i) {
      const int j = wv + W * i;
      const int x = j >> 2, kind = j & 3;
      const int gg = (t_begin + kTile * t + 16 * x < t_end) ? 2 * t + x : 2 * t;
      dst[i] = __builtin_amdgcn_readfirstlane(slot + (kind >= 2 ? kHalf : 0) + 2048 * x +
                                              1024 * (kind & 1));
      src[i] = kind == 0 ? koff0 : (kind == 1 ? koff1 : (kind == 2 ? voff0 : voff1));
      from[i] = (kind < 2 ? kpool : vpool) + group_base(gg);
    }
#pragma unroll
    for (int i = 0; i < kMine; ++i) dma16_stream(dst[i], src[i], from[i]);
  };

  // per-lane LDS offsets. K operand, chunk 2kp + h of token row col.
  // V operand of (k-step u, dim block nb): the 16 lanes of a group address
  // row 16u + tokv (the e-th token of the step in P's order, e = (l & 15) / 2)
  // half l & 1 of chunk 2nb + ((l >> 4) & 1).
  uint32_t koff[4];
#pragma unroll
  for (int kp = 0; kp < 4; ++kp)
    koff[kp] = col * kD + ((static_cast<uint32_t>(2 * kp + hl) ^ kswz(col)) << 4);
  const int e_row = (lane & 15) >> 1;
  const int tokv = 4 * hl + (e_row & 3) + 8 * (e_row >> 2);
  const int a16 = (lane >> 4) & 1;
  uint32_t voff[2][4];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const uint32_t row = 16 * u + tokv;
      voff[u][nb] = kHalf + row * kD + ((static_cast<uint32_t>(2 * nb + a16) ^ vswz(row)) << 4) +
                    8 * (lane & 1);
    }

  floatx16_t O[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int i = 0; i < 16; ++i) O[nb][i] = 0.0f;
  float m = kMUnset;  // reference max of query row col (both halves agree)
  float l = 0.0f;     // this lane's part of row col's denominator

#pragma unroll
  for (int k = 0; k < kRing - 1; ++k)
    if (k < n_tiles) issue(k);
  for (int t = 0; t < n_tiles; ++t) {
    if constexpr (W == 1) {
      if (t + kSlots - 1 < n_tiles) {
        issue(t + kSlots - 1);
        wait_vm<8 * (kSlots - 1)>();
      } else {
        wait_vm<0>();
      }
    } else {
      if (t + 1 < n_tiles) {
        wait_vm<kMine>();
      } else {
        wait_vm<0>();
      }
      // every wave's share of tile t has landed, and every wave is done with
      // tile t - 1, whose slot tile t + 2 takes
      __syncthreads();
      if (t + 2 < n_tiles) issue(t + 2);
    }
    uint8_t* buf = ring + (t % kRing) * kTileBytes;
    const int tile0 = t_begin + kTile * t;
    // rows past the unit or of a page outside the pool: V to zero (their
    // scores are masked, and 0 * NaN must not reach the accumulators)
    const bool g0_ok = page_valid(((2 * t) << 4) >> log2P);
    const bool g1_ok = tile0 + 16 < t_end && page_valid(((2 * t + 1) << 4) >> log2P);
    const int nv = min(kTile, t_end - tile0);
    if (!g0_ok || !g1_ok || nv < kTile) {
      for (int q = static_cast<int>(threadIdx.x); q < kTile * (kD / 16); q += 64 * W) {
        const int row = q >> 3;
        const bool keep = row < nv && (row < 16 ? g0_ok : g1_ok);
        if (!keep) *reinterpret_cast<uint4*>(buf + kHalf + 16 * q) = make_uint4(0u, 0u, 0u, 0u);
      }
      if constexpr (W == 1) {
        __builtin_amdgcn_wave_barrier();
      } else {
        __syncthreads();  // the same condition in every wave of the unit
      }
    }

    // ---- S^T = K Q^T for the tile
    floatx16_t st;
#pragma unroll
    for (int i = 0; i < 16; ++i) st[i] = 0.0f;
#pragma unroll
    for (int kp = 0; kp < 4; ++kp) {
      const uint4 kq = *reinterpret_cast<const uint4*>(buf + koff[kp]);
      st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fp8x8_to_bf16(kq.x, kq.y), qf[2 * kp], st, 0, 0, 0);
      st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fp8x8_to_bf16(kq.z, kq.w), qf[2 * kp + 1], st, 0, 0, 0);
    }
    // st[i]: token tile0 + 8(i/4) + 4h + i%4 of query row col
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int tt = 8 * (i >> 2) + 4 * hl + (i & 3);
      const bool ok = tile0 + tt < lim && (tt < 16 ? g0_ok : g1_ok);
      st[i] = ok ? st[i] * qk_scale : -INFINITY;
      tmax = fmaxf(tmax, st[i]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    if (m == kMUnset && tmax > -INFINITY) m = tmax;
    if (__any(tmax > m + kTau)) {
      // rare: raise the reference max of the rows that need it, rescale
      const float mn = tmax > m + kTau ? tmax : m;
      const float al = __builtin_amdgcn_exp2f(m - mn);
      m = mn;
      l *= al;
      if (hl == 0) rowbuf[0][col] = al;
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float a = rowbuf[0][8 * (i >> 2) + 4 * hl + (i & 3)];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) O[nb][i] *= a;
      }
      __builtin_amdgcn_wave_barrier();
    }

    // ---- O += P V, two k-steps of 16 tokens
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      f16x8_t pf;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float pr = __builtin_amdgcn_exp2f(st[8 * u + k] - m);
        l += pr;
        pf[k] = static_cast<_Float16>(pr);
      }
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const v2i_t r8 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_t*)(buf + voff[u][nb]));
        O[nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
            pf, fp8x8_to_f16(static_cast<uint32_t>(r8[0]), static_cast<uint32_t>(r8[1])), O[nb],
            0, 0, 0);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  // ---- finish: per query row, o / l and lse = m + log2 l (natural-log units)
  l += __shfl_xor(l, 32);
  if (hl == 0) {
    rowbuf[0][col] = l;
    rowbuf[1][col] = m;
  }
  __builtin_amdgcn_wave_barrier();
  const int64_t heads_all = static_cast<int64_t>(T) * p.num_q_heads;
  auto out_head = [&](int r) __attribute__((always_inline)) {
    const int j = r / G;
    return static_cast<int64_t>(b) * heads_all + static_cast<int64_t>(j) * p.num_q_heads + g * G +
           (r - j * G);
  };
  if (hl == 0 && row_ok)
    p.lse_part[out_head(r_mine) * p.max_splits + c] =
        !(l <= 0.0f) ? (m + __log2f(l)) * kLn2 : -INFINITY;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int row = 8 * (i >> 2) + 4 * hl + (i & 3);
    const int r = 32 * rg + row;
    if (r >= rows) continue;
    const float lr = rowbuf[0][row];
    const float f = !(lr <= 0.0f) ? o_scale / lr : 0.0f;
    float* dst = p.o_part + (out_head(r) * p.max_splits + c) * kD + col;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) dst[32 * nb] = O[nb][i] * f;
  }
}

}  // namespace

bool drafts_path_supported(int dk, int dv, bool latent, bool e4m3) {
  return e4m3 && !latent && dk == kD && dv == kD;
}

template <int W>
int launch_w(const DecodeParams& p, int64_t units, int row_groups, hipStream_t stream) {
  const int64_t blocks = units * ((row_groups + W - 1) / W);
  if (blocks > 0x7FFFFFFF) return PKV_EUNSUPPORTED;
  decode_drafts_kernel<W><<<dim3(static_cast<uint32_t>(blocks)), 64 * W, 0, stream>>>(p, row_groups);
  return pkv::launch_status();
}

int launch_decode_drafts(const DecodeParams& p, int n_split_blocks, int batch, int row_groups,
                         hipStream_t stream) {
  if (p.split_tokens > kMaxUnitPages * p.page_size) return PKV_EUNSUPPORTED;
  const int64_t units = static_cast<int64_t>(n_split_blocks) * p.num_kv_heads * batch;
  // the row groups of a unit share its tiles, up to 8 waves a workgroup
  if (row_groups == 1) return launch_w<1>(p, units, row_groups, stream);
  if (row_groups == 2) return launch_w<2>(p, units, row_groups, stream);
  if (row_groups <= 4) return launch_w<4>(p, units, row_groups, stream);
  return launch_w<8>(p, units, row_groups, stream);
}
