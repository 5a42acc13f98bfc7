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
//
// MFMA 16x16x32 bf16 (lane l, c = l % 16, q = l / 16; A: row c, k 8q .. 8q+7;
// B: column c, same k; D element i: row 4q + i, column c): A = 16 weight rows,
// B = 16 tokens (batch padded to 16 T). The contraction order is permuted so
// that a lane's codes for one 128-input group are one 16-byte run of its row:
// k-step s, slot 8q + j <-> input 32q + 8s + j; x is read in the same order.
//
// Codes to bf16: a nibble n becomes the bf16 with bits 0x4300 | (n ^ 8), the
// value 128 + (n ^ 8) = 136 + q, exact, two per v_perm + v_xor. MFMA then
// sums (136 + q) x exactly in each product, and 136 sum(x) is taken off per
// (group, token) before the group's scale is applied.
#include "common.h"
#include "mfma_tile.h"

namespace {

constexpr int kWaves = 8;    // waves per workgroup, each an eighth of the inputs
constexpr int kGroup = 128;  // inputs per scale
constexpr int kM = 2;        // 16-row weight tiles per workgroup

// eight codes (one dword, input order 0..7 in nibble order) -> eight bf16
// of 136 + q
__device__ __forceinline__ bf16x8_t codes_to_bf16(uint32_t wd) {
  const uint32_t lo = wd & 0x0F0F0F0Fu;
  const uint32_t hi = (wd >> 4) & 0x0F0F0F0Fu;
  uint32_t p[4];
  // pair j: low nibble of byte j (even input) in the low half, high nibble
  // (odd input) in the high half; 0x0C selects a zero byte
  p[0] = __builtin_amdgcn_perm(hi, lo, 0x0C040C00u) ^ 0x43084308u;
  p[1] = __builtin_amdgcn_perm(hi, lo, 0x0C050C01u) ^ 0x43084308u;
  p[2] = __builtin_amdgcn_perm(hi, lo, 0x0C060C02u) ^ 0x43084308u;
  p[3] = __builtin_amdgcn_perm(hi, lo, 0x0C070C03u) ^ 0x43084308u;
  bf16x8_t r;
  __builtin_memcpy(&r, p, sizeof(r));
  return r;
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b) {
  return __uint_as_float(b << 16);
}

template <int T>
__global__ void __launch_bounds__(64 * kWaves)
    int4_linear_kernel(const uint16_t* x, const uint8_t* w, const uint16_t* scales, int batch,
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

  floatx4_t acc[kM][T];
#pragma unroll
  for (int m = 0; m < kM; ++m)
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[m][t][i] = 0.0f;

  // a chunk of kChunk groups: x of the whole chunk, then the codes and
  // scales group by group, all issued before any is used. Loads return in
  // order, so group d is computed as soon as its own codes have landed while
  // the later groups' are still in flight.
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
      const int g = c0 + d;
      if (g >= groups) break;
      const int cur = d;

      // sum of this lane's 32 inputs per token, then over the four lanes of
      // the token's column
      float xs[T];
#pragma unroll
      for (int t = 0; t < T; ++t) {
        float a = 0.0f;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const uint4 u = *reinterpret_cast<const uint4*>(&xv[cur][t][s]);
          const uint32_t wv4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            a += bf16_bits_to_float(wv4[e] & 0xFFFFu) + bf16_bits_to_float(wv4[e] >> 16);
        }
        a += __shfl_xor(a, 16);
        a += __shfl_xor(a, 32);
        xs[t] = a * 136.0f;
      }
#pragma unroll
      for (int m = 0; m < kM; ++m) {
        const uint4 c = wq[d][m];
        const bf16x8_t a0 = codes_to_bf16(c.x), a1 = codes_to_bf16(c.y),
                       a2 = codes_to_bf16(c.z), a3 = codes_to_bf16(c.w);
        float sc[4];
        sc[0] = bf16_bits_to_float(sq[d][m].x & 0xFFFFu);
        sc[1] = bf16_bits_to_float(sq[d][m].x >> 16);
        sc[2] = bf16_bits_to_float(sq[d][m].y & 0xFFFFu);
        sc[3] = bf16_bits_to_float(sq[d][m].y >> 16);
#pragma unroll
        for (int t = 0; t < T; ++t) {
          floatx4_t dacc = {0.0f, 0.0f, 0.0f, 0.0f};
          dacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, xv[cur][t][0], dacc, 0, 0, 0);
          dacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, xv[cur][t][1], dacc, 0, 0, 0);
          dacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a2, xv[cur][t][2], dacc, 0, 0, 0);
          dacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a3, xv[cur][t][3], dacc, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[m][t][i] += sc[i] * (dacc[i] - xs[t]);
        }
      }
    }
  }

  // ---- sum the waves' partials; wave 0 writes y
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

template <int T>
int launch(const uint16_t* x, const uint8_t* w, const uint16_t* s, int batch, int n, int k,
           uint16_t* y, hipStream_t stream) {
  int4_linear_kernel<T><<<dim3(n / (16 * kM)), 64 * kWaves, 0, stream>>>(x, w, s, batch, n, k,
                                                                          y);
  return pkv::launch_status();
}

}  // namespace

extern "C" int pkv_int4_linear(const void* x, const uint8_t* w, const void* scales,
                               int32_t batch, int32_t n, int32_t k, void* y,
                               hipStream_t stream) {
  if (!x || !w || !scales || !y) return PKV_EINVAL;
  if (batch < 1 || batch > 64 || n < 1 || k < 1) return PKV_EINVAL;
  if (n % (16 * kM) || k % (kWaves * kGroup)) return PKV_EINVAL;
  if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(w) |
       reinterpret_cast<uintptr_t>(scales)) & 15)
    return PKV_EINVAL;
  const auto* xs = static_cast<const uint16_t*>(x);
  const auto* ss = static_cast<const uint16_t*>(scales);
  auto* ys = static_cast<uint16_t*>(y);
  switch ((batch + 15) / 16) {
    case 1: return launch<1>(xs, w, ss, batch, n, k, ys, stream);
    case 2: return launch<2>(xs, w, ss, batch, n, k, ys, stream);
    case 3: return launch<3>(xs, w, ss, batch, n, k, ys, stream);
    default: return launch<4>(xs, w, ss, batch, n, k, ys, stream);
  }
}
