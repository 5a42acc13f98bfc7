// INT4 weight-only linear layer of the decode phase: y = x W^T.
//
// "Smaller, faster, safer: running Kimi and GLM at scale" (Cloudflare blog),
// section on model weights: GLM's weights are held as 4-bit integers for
// decode, where producing each token streams them out of GPU memory, so the
// layer is bound by the bytes it reads.
//
// Format (the library's reading; the pages give none): codes are 4-bit two's
// complement, two per byte (even input k in the low nibble), w[n][k] =
// q[n][k] * scales[k / 128][n], bf16 scales, bf16 activations, bf16 output.
//
// Work: a workgroup of kWaves waves owns 16 M output rows; its waves split
// the inputs (k / kWaves each, whole 128-input groups) and add their partial
// sums through LDS at the end. Each wave streams its slice of the codes once.
// Two kernels: up to 8 tokens, every operand travels by direct-to-LDS loads
// of whole cache lines (int4_lds_kernel); above that, x is too large for a
// per-wave ring and the operands go straight to registers (int4_reg_kernel).
//
// MFMA 16x16x32 bf16 (lane l, c = l % 16, q = l / 16; A: row c, k 8q .. 8q+7;
// B: column c, same k; D element i: row 4q + i, column c): A = 16 weight rows,
// B = 16 tokens (batch padded to 16 T). The contraction order is permuted so
// that a lane's codes for one 128-input group are one 16-byte run of its row:
// k-step s, slot 8q + j <-> input 32q + 8s + j; x is read in the same order.
//
// Codes to bf16: a nibble n becomes the bf16 with bits 0x4300 | (n ^ 8), the
// value 128 + (n ^ 8) = 136 + q, exact, two per v_perm + v_and_or. MFMA sums
// (136 + q) x exactly in each product, on top of -136 sum(x) that one more
// MFMA chain per group and token gives (A = -136 everywhere); the group's
// scale is then applied to the sum of q x.
#include "common.h"
#include "mfma_tile.h"

namespace {

constexpr int kWaves = 8;    // waves per workgroup, each an eighth of the inputs
constexpr int kGroup = 128;  // inputs per scale
constexpr int kM = 2;        // 16-row weight tiles per workgroup

// eight codes (one dword, input order 0..7 in nibble order, every nibble
// already xored with 8 so that it reads q + 8) -> eight bf16 of 136 + q
// (mask = 0x000F000F, expo = 0x43004300, held in registers so that each
// pair is one v_perm and one v_and_or)
__device__ __forceinline__ bf16x8_t codes_to_bf16(uint32_t wd, uint32_t mask, uint32_t expo) {
  const uint32_t hi = wd >> 4;
  uint32_t p[4];
  // pair j: byte j of wd (low nibble: input 2j) in the low half, byte j of
  // wd >> 4 (low nibble: input 2j + 1) in the high half; then the nibbles
  // under exponent 0x43 (bf16 128 + n)
  p[0] = (__builtin_amdgcn_perm(hi, wd, 0x0C040C00u) & mask) | expo;
  p[1] = (__builtin_amdgcn_perm(hi, wd, 0x0C050C01u) & mask) | expo;
  p[2] = (__builtin_amdgcn_perm(hi, wd, 0x0C060C02u) & mask) | expo;
  p[3] = (__builtin_amdgcn_perm(hi, wd, 0x0C070C03u) & mask) | expo;
  bf16x8_t r;
  __builtin_memcpy(&r, p, sizeof(r));
  return r;
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b) {
  return __uint_as_float(b << 16);
}

// bf16 -136 in every slot: as the A operand it gives -136 sum(x) per token
__device__ __forceinline__ bf16x8_t neg136() {
  bf16x8_t v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = static_cast<__bf16>(-136.0f);
  return v;
}

// one 128-input group of kM row tiles against T token tiles: xv the B
// operands, c the codes of row 16 m + col, sq the scales of rows 16 m + 4 qg
// .. + 3
template <int T, int M = kM>
__device__ __forceinline__ void group_math(const bf16x8_t (&xv)[T][4], const uint4 (&c)[M],
                                           const uint2 (&sq)[M], bf16x8_t neg, uint32_t mask,
                                           uint32_t expo, floatx4_t (&acc)[M][T]) {
  floatx4_t dn[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    dn[t] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < 4; ++s)
      dn[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(neg, xv[t][s], dn[t], 0, 0, 0);
  }
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const bf16x8_t a0 = codes_to_bf16(c[m].x ^ 0x88888888u, mask, expo),
                   a1 = codes_to_bf16(c[m].y ^ 0x88888888u, mask, expo),
                   a2 = codes_to_bf16(c[m].z ^ 0x88888888u, mask, expo),
                   a3 = codes_to_bf16(c[m].w ^ 0x88888888u, mask, expo);
    float sc[4];
    sc[0] = bf16_bits_to_float(sq[m].x & 0xFFFFu);
    sc[1] = bf16_bits_to_float(sq[m].x >> 16);
    sc[2] = bf16_bits_to_float(sq[m].y & 0xFFFFu);
    sc[3] = bf16_bits_to_float(sq[m].y >> 16);
#pragma unroll
    for (int t = 0; t < T; ++t) {
      // sum over the group of (136 + q) x - 136 x = q x, exact products
      floatx4_t d = dn[t];
      d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, xv[t][0], d, 0, 0, 0);
      d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, xv[t][1], d, 0, 0, 0);
      d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a2, xv[t][2], d, 0, 0, 0);
      d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a3, xv[t][3], d, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[m][t][i] = fmaf(sc[i], d[i], acc[m][t][i]);
    }
  }
}

// the waves' partial sums added through LDS; wave 0 writes y
template <int T>
__device__ __forceinline__ void reduce_store(float (*red)[kM * T * 4][64], const floatx4_t (&acc)[kM][T],
                                             int wv, int lane, int r0, int batch, int N,
                                             uint16_t* y) {
  const int col = lane & 15, qg = lane >> 4;
  if (wv > 0) {
#pragma unroll
    for (int m = 0; m < kM; ++m)
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wv - 1][(m * T + t) * 4 + i][lane] = acc[m][t][i];
  }
  __syncthreads();
  if (wv == 0) {
#pragma unroll
    for (int m = 0; m < kM; ++m)
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const int token = 16 * t + col;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = acc[m][t][i];
#pragma unroll
          for (int u = 0; u < kWaves - 1; ++u) v += red[u][(m * T + t) * 4 + i][lane];
          if (token < batch)
            y[static_cast<size_t>(token) * N + r0 + 16 * m + 4 * qg + i] = pkv::f32_to_bf16_rne(v);
        }
      }
  }
}

// ---------------------------------------------------------------------------
// Batch up to 8: codes, scales and x travel HBM -> LDS by direct-to-LDS
// loads, each instruction a whole 1 KB of full 128-byte lines, through a
// two-tile ring per wave. A tile is the workgroup's 32 rows x 256 inputs
// (4 KB of codes: instruction j holds rows 8 j .. 8 j + 7, the 16-byte chunk
// p of row r at position p ^ ((r >> 1) & 7) so that the MFMA reads are free
// of bank conflicts), the tile's 2 x 32 scales, and the 256 inputs of each
// of up to 2 XB tokens (a token's 16-byte chunk p at p ^ (token & 7)).
template <int XB>
__global__ void __launch_bounds__(64 * kWaves)
    int4_lds_kernel(const uint16_t* x, const uint8_t* w, const uint16_t* scales, int batch,
                    int N, int K, uint16_t* y) {
  constexpr int kSlots = 2;
  constexpr int kCodeB = 32 * 128, kScB = 256, kSlot = kCodeB + kScB + XB * 1024;
  constexpr int kLoads = 4 + 1 + XB;  // loads per tile
  __shared__ __attribute__((aligned(16))) uint8_t ring[kWaves * kSlots * kSlot];
  __shared__ float red[kWaves - 1][kM * 4][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int col = lane & 15, qg = lane >> 4;
  const int r0 = blockIdx.x * 16 * kM;
  const int kw = K / kWaves, tiles = kw / 256, kb = wv * kw;
  const uint32_t half = static_cast<uint32_t>(K) / 2;
  const uint8_t* wring = ring + wv * kSlots * kSlot;
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(wring));

  uint32_t cvoff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 8 * j + (lane >> 3);
    cvoff[j] = (r0 + row) * half + kb / 2 + 16 * ((lane & 7) ^ ((row >> 1) & 7));
  }
  // lanes 0 .. 15: rows 2 p, 2 p + 1 of the tile's first group, 16 .. 31 the
  // second group (lanes 32 .. 63 repeat them)
  const uint32_t svoff =
      ((kb / kGroup + ((lane >> 4) & 1)) * N + r0 + 2 * (lane & 15)) * 2;
  uint32_t xvoff[XB];
#pragma unroll
  for (int j = 0; j < XB; ++j) {
    const int tok = min(2 * j + (lane >> 5), batch - 1);
    xvoff[j] = (tok * K + kb) * 2 + 16 * ((lane & 31) ^ (tok & 7));
  }
  const int xtok = min(col, batch - 1);
  const bf16x8_t neg = neg136();
  uint32_t mask = 0x000F000Fu, expo = 0x43004300u;
  asm volatile("" : "+v"(mask), "+v"(expo));
  floatx4_t acc[kM][1];
#pragma unroll
  for (int m = 0; m < kM; ++m) acc[m][0] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};

  auto issue = [&](int t) __attribute__((always_inline)) {
    const uint32_t slot = base + (t % kSlots) * kSlot;
#pragma unroll
    for (int j = 0; j < 4; ++j) dma16_stream(slot + 1024 * j, cvoff[j] + 128 * t, w);
    dma4(slot + kCodeB, svoff + 4 * N * t, reinterpret_cast<const uint8_t*>(scales));
#pragma unroll
    for (int j = 0; j < XB; ++j)
      dma16(slot + kCodeB + kScB + 1024 * j, xvoff[j] + 512 * t,
            reinterpret_cast<const uint8_t*>(x));
  };
  // nothing else is loaded while the ring runs
  asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
  issue(0);
  for (int t = 0; t < tiles; ++t) {
    if (t + 1 < tiles) {
      issue(t + 1);
      wait_vm<kLoads>();
    } else {
      wait_vm<0>();
    }
    const uint8_t* buf = wring + (t % kSlots) * kSlot;
#pragma unroll
    for (int gh = 0; gh < 2; ++gh) {
      bf16x8_t xv[1][4];
#pragma unroll
      for (int s = 0; s < 4; ++s)
        xv[0][s] = *reinterpret_cast<const bf16x8_t*>(
            buf + kCodeB + kScB + 512 * xtok + 16 * ((16 * gh + 4 * qg + s) ^ (xtok & 7)));
      uint4 c[kM];
      uint2 sq[kM];
#pragma unroll
      for (int m = 0; m < kM; ++m) {
        const int row = 16 * m + col;
        c[m] = *reinterpret_cast<const uint4*>(buf + 128 * row +
                                               16 * ((4 * gh + qg) ^ ((row >> 1) & 7)));
        sq[m] = *reinterpret_cast<const uint2*>(buf + kCodeB + 64 * gh + 2 * (16 * m + 4 * qg));
      }
      group_math<1>(xv, c, sq, neg, mask, expo, acc);
    }
  }
  reduce_store<1>(red, acc, wv, lane, r0, batch, N, y);
}

// ---------------------------------------------------------------------------
// Any batch up to 64: operands straight into registers. Each wave loads a
// chunk of kChunk groups at once (x of the whole chunk, then the codes and
// scales group by group) and computes group d as soon as its own loads have
// landed (loads return in order) while the later groups' are in flight.
template <int T>
__global__ void __launch_bounds__(64 * kWaves)
    int4_reg_kernel(const uint16_t* x, const uint8_t* w, const uint16_t* scales, int batch,
                    int N, int K, uint16_t* y) {
  __shared__ float red[kWaves - 1][kM * T * 4][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int col = lane & 15, qg = lane >> 4;
  const int r0 = blockIdx.x * 16 * kM;
  const int kw = K / kWaves;
  const int groups = kw / kGroup;
  const int kb = wv * kw;
  const size_t half = static_cast<size_t>(K) / 2;

  const uint8_t* wrow[kM];
#pragma unroll
  for (int m = 0; m < kM; ++m)
    wrow[m] = w + static_cast<size_t>(r0 + 16 * m + col) * half + kb / 2 + 16 * qg;
  const uint16_t* xrow[T];
#pragma unroll
  for (int t = 0; t < T; ++t)
    xrow[t] = x + static_cast<size_t>(min(16 * t + col, batch - 1)) * K + kb + 32 * qg;
  // scales of rows r0 + 16 m + 4 qg .. +3 of group kb / 128 + g
  const uint16_t* srow = scales + static_cast<size_t>(kb / kGroup) * N + r0 + 4 * qg;
  const bf16x8_t neg = neg136();
  uint32_t mask = 0x000F000Fu, expo = 0x43004300u;
  asm volatile("" : "+v"(mask), "+v"(expo));

  floatx4_t acc[kM][T];
#pragma unroll
  for (int m = 0; m < kM; ++m)
#pragma unroll
    for (int t = 0; t < T; ++t) acc[m][t] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};

  constexpr int kChunk = T == 1 ? 8 : (T == 2 ? 4 : 2);
  uint4 wq[kChunk][kM];
  uint2 sq[kChunk][kM];
  bf16x8_t xv[kChunk][T][4];
  for (int c0 = 0; c0 < groups; c0 += kChunk) {
#pragma unroll
    for (int d = 0; d < kChunk; ++d) {
      const int g = min(c0 + d, groups - 1);  // clamped: no branch around loads
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int s = 0; s < 4; ++s)
          xv[d][t][s] = *reinterpret_cast<const bf16x8_t*>(xrow[t] + g * kGroup + 8 * s);
    }
#pragma unroll
    for (int d = 0; d < kChunk; ++d) {
      const int g = min(c0 + d, groups - 1);
#pragma unroll
      for (int m = 0; m < kM; ++m) {
        wq[d][m] = *reinterpret_cast<const uint4*>(wrow[m] + g * (kGroup / 2));
        sq[d][m] = *reinterpret_cast<const uint2*>(srow + static_cast<size_t>(g) * N + 16 * m);
      }
    }
    // the chunk's loads stay here, ahead of their uses
    asm volatile("" : : : "memory");
#pragma unroll
    for (int d = 0; d < kChunk; ++d) {
      if (c0 + d >= groups) break;
      group_math<T>(xv[d], wq[d], sq[d], neg, mask, expo, acc);
    }
  }
  reduce_store<T>(red, acc, wv, lane, r0, batch, N, y);
}

// ---------------------------------------------------------------------------
// Above 8 tokens, with a workspace: the 8 waves of a workgroup take 16 rows
// each of a 128-row block over the same slice of the inputs, so the x tile
// (16 TT token rows x 256 inputs) is staged once through LDS for all of
// them. When there are too few row blocks to fill the chip, the inputs are
// split over KS workgroups of a block, which write fp32 partial sums to the
// workspace; int4_sum_kernel then adds the KS partials of each output in
// slice order and rounds to bf16. (The last workgroup of a block could add
// them itself, but making the partials of other XCDs visible to it takes a
// write-back of each XCD's L2 per workgroup, which costs more than the
// second launch.) Each tile: per wave 2 direct-to-LDS loads of
// codes (16 rows x 128 bytes, the same swizzle as above), one of scales and
// TT of x (each 1 KB: two token rows, 16-byte chunk p of row t at
// p ^ (t & 15)); three slots, two tiles in flight while one is computed.
constexpr int kBlockRows = 16 * kWaves;  // rows per workgroup

template <int TT>
__global__ void __launch_bounds__(64 * kWaves)
    int4_split_kernel(const uint16_t* x, const uint8_t* w, const uint16_t* scales, int batch,
                      int N, int K, int KC, float* part, uint16_t* y) {
  constexpr int kSlots = 3;
  constexpr int kXRowB = 512;                   // 256 inputs of one token
  constexpr int kXB = 16 * TT * kXRowB;         // x tile
  constexpr int kCodeB = 16 * 128, kScB = 256;  // one wave's codes and scales
  constexpr int kCSlot = kCodeB + kScB;
  constexpr int kLoads = 2 + 1 + TT;  // loads per wave and tile
  __shared__ __attribute__((aligned(16))) uint8_t xring[kSlots * kXB];
  __shared__ __attribute__((aligned(16))) uint8_t cring[kWaves * kSlots * kCSlot];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int col = lane & 15, qg = lane >> 4;
  const int r0 = blockIdx.x * kBlockRows + 16 * wv;  // this wave's 16 rows
  const int kc = blockIdx.y;
  const int kb = kc * KC, tiles = KC / 256;
  const uint32_t half = static_cast<uint32_t>(K) / 2;
  const uint8_t* wring = cring + wv * kSlots * kCSlot;
  const uint32_t cbase = __builtin_amdgcn_readfirstlane(lds_addr(wring));
  const uint32_t xbase = lds_addr(xring);

  uint32_t cvoff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = 8 * j + (lane >> 3);
    cvoff[j] = (r0 + row) * half + kb / 2 + 16 * ((lane & 7) ^ ((row >> 1) & 7));
  }
  // lanes 0 .. 7: rows 2 p, 2 p + 1 of the tile's first group, 8 .. 15 the
  // second (the other lanes repeat them)
  const uint32_t svoff = ((kb / kGroup + ((lane >> 3) & 1)) * N + r0 + 2 * (lane & 7)) * 2;
  // x: this wave's instructions wv + 8 i cover token rows 2 (wv + 8 i) + 0, 1
  uint32_t xvoff[TT];
#pragma unroll
  for (int i = 0; i < TT; ++i) {
    const int row = 2 * (wv + 8 * i) + (lane >> 5);
    const int tok = min(row, batch - 1);
    xvoff[i] = (tok * K + kb) * 2 + 16 * ((lane & 31) ^ (row & 15));
  }
  const bf16x8_t neg = neg136();
  uint32_t mask = 0x000F000Fu, expo = 0x43004300u;
  asm volatile("" : "+v"(mask), "+v"(expo));
  floatx4_t acc[1][TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) acc[0][tt] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};

  auto issue = [&](int t) __attribute__((always_inline)) {
    const uint32_t cs = __builtin_amdgcn_readfirstlane(cbase + (t % kSlots) * kCSlot);
    // codes are read once; the non-temporal hint pays with one token tile
    // and was measured slower with two or more
    if constexpr (TT == 1) {
      dma16_stream(cs, cvoff[0] + 128 * t, w);
      dma16_stream(cs + 1024, cvoff[1] + 128 * t, w);
    } else {
      dma16(cs, cvoff[0] + 128 * t, w);
      dma16(cs + 1024, cvoff[1] + 128 * t, w);
    }
    dma4(cs + kCodeB, svoff + 4 * N * t, reinterpret_cast<const uint8_t*>(scales));
    const uint32_t xs = __builtin_amdgcn_readfirstlane(xbase + (t % kSlots) * kXB);
#pragma unroll
    for (int i = 0; i < TT; ++i)
      dma16(xs + 1024 * (wv + 8 * i), xvoff[i] + kXRowB * t, reinterpret_cast<const uint8_t*>(x));
  };
  asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
  issue(0);
  if (tiles > 1) issue(1);
  for (int t = 0; t < tiles; ++t) {
    if (t + 1 < tiles) {
      wait_vm<kLoads>();
    } else {
      wait_vm<0>();
    }
    // every wave's part of tile t has landed, and every wave is done with
    // tile t - 1, whose slots tile t + 2 takes next
    __syncthreads();
    if (t + 2 < tiles) issue(t + 2);
    const uint8_t* cbuf = wring + (t % kSlots) * kCSlot;
    const uint8_t* xbuf = xring + (t % kSlots) * kXB;
#pragma unroll
    for (int gh = 0; gh < 2; ++gh) {
      uint4 c[1];
      uint2 sq[1];
      c[0] = *reinterpret_cast<const uint4*>(cbuf + 128 * col +
                                             16 * ((4 * gh + qg) ^ ((col >> 1) & 7)));
      sq[0] = *reinterpret_cast<const uint2*>(cbuf + kCodeB + 32 * gh + 8 * qg);
      bf16x8_t xv[TT][4];
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        const int row = 16 * tt + col;
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4)
          xv[tt][s4] = *reinterpret_cast<const bf16x8_t*>(
              xbuf + kXRowB * row + 16 * ((16 * gh + 4 * qg + s4) ^ (row & 15)));
      }
      group_math<TT, 1>(xv, c, sq, neg, mask, expo, acc);
    }
  }
  // rows r0 + 4 qg + i, tokens 16 tt + col
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    const int token = 16 * tt + col;
    if (token >= batch) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const size_t o = static_cast<size_t>(token) * N + r0 + 4 * qg + i;
      if (part) {
        part[static_cast<size_t>(kc) * batch * N + o] = acc[0][tt][i];
      } else {
        y[o] = pkv::f32_to_bf16_rne(acc[0][tt][i]);
      }
    }
  }
}

// y = bf16(sum over the KS input slices of the partials, in slice order),
// 4 outputs a thread
__global__ void __launch_bounds__(256) int4_sum_kernel(const float* part, int KS, size_t count,
                                                       uint16_t* y) {
  const size_t i = (static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (i >= count) return;
  float4 v = *reinterpret_cast<const float4*>(part + i);
  for (int s = 1; s < KS; ++s) {
    const float4 u = *reinterpret_cast<const float4*>(part + static_cast<size_t>(s) * count + i);
    v.x += u.x;
    v.y += u.y;
    v.z += u.z;
    v.w += u.w;
  }
  y[i] = pkv::f32_to_bf16_rne(v.x);
  y[i + 1] = pkv::f32_to_bf16_rne(v.y);
  y[i + 2] = pkv::f32_to_bf16_rne(v.z);
  y[i + 3] = pkv::f32_to_bf16_rne(v.w);
}

// input slices per row block for the split kernel: enough workgroups to fill
// the chip (about 192 or more), each slice whole tiles; 0 if the split kernel
// does not apply
int split_slices(int batch, int n, int k) {
  if (batch <= 8 || n % kBlockRows) return 0;
  if (static_cast<int64_t>(n) * k / 2 > 0xFFFFFFFFLL || static_cast<int64_t>(batch) * k * 2 > 0xFFFFFFFFLL)
    return 0;
  const int blocks = n / kBlockRows;
  int ks = 1;
  while (blocks * ks < 192 && ks < 8 && k % (256 * ks * 2) == 0) ks *= 2;
  return k % (256 * ks) == 0 ? ks : 0;
}

template <int T>
int launch_reg(const uint16_t* x, const uint8_t* w, const uint16_t* s, int batch, int n, int k,
               uint16_t* y, hipStream_t stream) {
  int4_reg_kernel<T><<<dim3(n / (16 * kM)), 64 * kWaves, 0, stream>>>(x, w, s, batch, n, k, y);
  return pkv::launch_status();
}

template <int XB>
int launch_lds(const uint16_t* x, const uint8_t* w, const uint16_t* s, int batch, int n, int k,
               uint16_t* y, hipStream_t stream) {
  int4_lds_kernel<XB><<<dim3(n / (16 * kM)), 64 * kWaves, 0, stream>>>(x, w, s, batch, n, k, y);
  return pkv::launch_status();
}

// workspace: fp32 partials [ks][batch][n]
int64_t partial_bytes(int ks, int batch, int n) { return static_cast<int64_t>(ks) * batch * n * 4; }

template <int TT>
int launch_split(const uint16_t* x, const uint8_t* w, const uint16_t* s, int batch, int n, int k,
                 int ks, void* workspace, uint16_t* y, hipStream_t stream) {
  float* part = ks > 1 ? static_cast<float*>(workspace) : nullptr;
  int4_split_kernel<TT><<<dim3(n / kBlockRows, ks), 64 * kWaves, 0, stream>>>(
      x, w, s, batch, n, k, k / ks, part, y);
  int st = pkv::launch_status();
  if (st || ks == 1) return st;
  const size_t count = static_cast<size_t>(batch) * n;
  int4_sum_kernel<<<dim3(static_cast<uint32_t>((count / 4 + 255) / 256)), 256, 0, stream>>>(
      part, ks, count, y);
  return pkv::launch_status();
}

}  // namespace

extern "C" int64_t pkv_int4_linear_workspace(int32_t batch, int32_t n, int32_t k) {
  if (batch < 1 || batch > 64 || n < 1 || k < 1) return PKV_EINVAL;
  const int ks = split_slices(batch, n, k);
  return ks > 1 ? partial_bytes(ks, batch, n) : 0;
}

extern "C" int pkv_int4_linear(const void* x, const uint8_t* w, const void* scales,
                               int32_t batch, int32_t n, int32_t k, void* y, void* workspace,
                               hipStream_t stream) {
  if (!x || !w || !scales || !y) return PKV_EINVAL;
  if (batch < 1 || batch > 64 || n < 1 || k < 1) return PKV_EINVAL;
  if (n % (16 * kM) || k % (kWaves * kGroup)) return PKV_EINVAL;
  if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(w) |
       reinterpret_cast<uintptr_t>(scales) | reinterpret_cast<uintptr_t>(workspace)) & 15)
    return PKV_EINVAL;
  const auto* xs = static_cast<const uint16_t*>(x);
  const auto* ss = static_cast<const uint16_t*>(scales);
  auto* ys = static_cast<uint16_t*>(y);
  // the LDS path: whole 256-input tiles per wave and 32-bit byte offsets
  const bool lds_ok = k % (kWaves * 256) == 0 &&
                      static_cast<int64_t>(n) * k / 2 <= 0xFFFFFFFFLL &&
                      static_cast<int64_t>(batch) * k * 2 <= 0xFFFFFFFFLL;
  if (lds_ok && batch <= 8) {
    if (batch <= 2) return launch_lds<1>(xs, w, ss, batch, n, k, ys, stream);
    if (batch <= 4) return launch_lds<2>(xs, w, ss, batch, n, k, ys, stream);
    return launch_lds<4>(xs, w, ss, batch, n, k, ys, stream);
  }
  const int ks = split_slices(batch, n, k);
  if (ks == 1 || (ks > 1 && workspace)) {
    switch ((batch + 15) / 16) {
      case 1: return launch_split<1>(xs, w, ss, batch, n, k, ks, workspace, ys, stream);
      case 2: return launch_split<2>(xs, w, ss, batch, n, k, ks, workspace, ys, stream);
      case 3: return launch_split<3>(xs, w, ss, batch, n, k, ks, workspace, ys, stream);
      default: return launch_split<4>(xs, w, ss, batch, n, k, ks, workspace, ys, stream);
    }
  }
  switch ((batch + 15) / 16) {
    case 1: return launch_reg<1>(xs, w, ss, batch, n, k, ys, stream);
    case 2: return launch_reg<2>(xs, w, ss, batch, n, k, ys, stream);
    case 3: return launch_reg<3>(xs, w, ss, batch, n, k, ys, stream);
    default: return launch_reg<4>(xs, w, ss, batch, n, k, ys, stream);
  }
}
