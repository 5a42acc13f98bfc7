// Internal helpers shared by the libpkv translation units (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "pkv.h"

namespace pkv {

constexpr int kWave = 64;

// ---------------------------------------------------------------- host side
inline bool valid_page_size(int p) { return p == 16 || p == 32 || p == 64; }

inline int check_cache(const pkv_cache* c) {
  if (!c || !c->k_pool) return PKV_EINVAL;
  if (c->dtype != PKV_KV_E4M3 && c->dtype != PKV_KV_BF16) return PKV_EINVAL;
  if (c->num_pages < 1 || c->num_kv_heads < 1 || !valid_page_size(c->page_size)) return PKV_EINVAL;
  if (c->head_dim_k < 16 || c->head_dim_k % 16 || c->head_dim_v < 16 || c->head_dim_v % 16)
    return PKV_EINVAL;
  if (!c->v_pool && c->head_dim_v > c->head_dim_k) return PKV_EINVAL;
  const bool rows = c->k_row_scale || c->v_row_scale;
  if (rows && (!c->k_row_scale || !c->v_row_scale || c->dtype != PKV_KV_E4M3 || !c->v_pool))
    return PKV_EINVAL;
  if (c->dtype == PKV_KV_E4M3 && !rows && (!c->k_scale || (c->v_pool && !c->v_scale)))
    return PKV_EINVAL;
  return PKV_OK;
}

inline int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? PKV_OK : PKV_EHIP;
}

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Scales set at append: the dim / 16 threads of a row must tile the 64 lanes
// of a wave (a power of two at most 64).
inline bool row_lanes_ok(int dim) {
  const int chunks = dim / 16;
  return chunks >= 1 && chunks <= 64 && (chunks & (chunks - 1)) == 0;
}

// -------------------------------------------------------------- device side
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Largest magnitude of 16 bf16 values (two 16-byte words); fmaxf leaves
// NaNs out.
__device__ __forceinline__ float abs_max16(const uint4& w0, const uint4& w1) {
  const uint32_t u[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    m = fmaxf(m, fabsf(__uint_as_float(u[j] << 16)));
    m = fmaxf(m, fabsf(__uint_as_float(u[j] & 0xFFFF0000u)));
  }
  return m;
}

// float32 -> bf16, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// float32 -> e4m3 code, round to nearest even, saturating, from the IEEE
// bit layout: 4-bit exponent with bias 7 and 3 mantissa bits; below 2^-6
// the grid is the multiples of 2^-9.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7Fu;   // NaN
  if (a >= 0x43E00000u) return sign | 0x7Eu;  // |y| >= 448 or infinite
  if (a < 0x3C800000u) {                      // |y| < 2^-6: count of 2^-9 steps
    return sign | static_cast<uint32_t>(rintf(__uint_as_float(a) * 512.0f));
  }
  uint32_t code = (((a >> 23) - 120u) << 3) | ((a >> 20) & 7u);
  const uint32_t rem = a & 0xFFFFFu;
  code += (rem > 0x80000u) || (rem == 0x80000u && (code & 1u));
  return sign | code;
}

// 16 bf16 values (two 16-byte words) -> 16 e4m3 codes of fl32(x / s), one
// 16-byte word: the definition step by step (correctly rounded division,
// then the IEEE-bit encoder).
__device__ __forceinline__ uint4 encode16_exact(const uint4& w0, const uint4& w1, float s) {
  const uint32_t in[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
  uint32_t out[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t pair = in[2 * k + j];
      const float lo = __uint_as_float(pair << 16);
      const float hi = __uint_as_float(pair & 0xFFFF0000u);
      const uint32_t c0 = e4m3_rne_sat(__fdiv_rn(lo, s));
      const uint32_t c1 = e4m3_rne_sat(__fdiv_rn(hi, s));
      word |= (c0 | (c1 << 8)) << (16 * j);
    }
    out[k] = word;
  }
  return make_uint4(out[0], out[1], out[2], out[3]);
}

// fl32(x / s) clamped to +-448, for s in [2^-60, 2^60] and x not NaN, with
// r = fl32(1 / s) and c = 512 s. Markstein's division: q0 = fl32(x r) is
// within one ulp of x / s, the residual x - q0 s is exact in one FMA, and
// q0 + (x - q0 s) r then rounds to the correctly rounded quotient. The scale
// range and the clamp of x to +-c keep every step clear of overflow and
// underflow wherever the e4m3 code depends on more than the sign (quotients
// at or above 2^-11); the sign comes from q0, which keeps that of x even when
// the correction returns +0 for x = -0.
__device__ __forceinline__ float quotient_sat(float x, float s, float r, float c) {
  const float xc = fminf(fmaxf(x, -c), c);
  const float q0 = xc * r;
  const float e = fmaf(-q0, s, xc);
  const float q = copysignf(fmaf(e, r, q0), q0);
  return fminf(fmaxf(q, -448.0f), 448.0f);
}

// encode16_exact, faster: the quotient by quotient_sat and the rounding by
// the e4m3 conversion instruction, which rounds to nearest even on
// [-448, 448] (the clamp gives the saturation). A word holding a NaN, or a
// scale outside [2^-60, 2^60], takes encode16_exact.
__device__ __forceinline__ uint4 encode16(const uint4& w0, const uint4& w1, float s) {
  const uint32_t in[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
  // a bf16 half h is NaN iff (h & 0x7FFF) > 0x7F80, iff adding 0x7F to it
  // sets its bit 15 (no carry leaves the half)
  uint32_t nan = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) nan |= (in[i] & 0x7FFF7FFFu) + 0x007F007Fu;
  if ((nan & 0x80008000u) != 0 || !(s >= 0x1p-60f && s <= 0x1p60f))
    return encode16_exact(w0, w1, s);
  const float r = __fdiv_rn(1.0f, s), c = 512.0f * s;
  uint32_t out[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t p0 = in[2 * k], p1 = in[2 * k + 1];
    const float y0 = quotient_sat(__uint_as_float(p0 << 16), s, r, c);
    const float y1 = quotient_sat(__uint_as_float(p0 & 0xFFFF0000u), s, r, c);
    const float y2 = quotient_sat(__uint_as_float(p1 << 16), s, r, c);
    const float y3 = quotient_sat(__uint_as_float(p1 & 0xFFFF0000u), s, r, c);
    uint32_t word = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false));
    word = static_cast<uint32_t>(
        __builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, static_cast<int>(word), true));
    out[k] = word;
  }
  return make_uint4(out[0], out[1], out[2], out[3]);
}

// The tag check of request b by one workgroup of 256 threads ("Smaller,
// faster, safer", section "Protecting a shared KV cache"): nonzero (the same
// in every thread) if the request must be aborted. Each thread takes entries
// j = j0 + 256u + tid for u < 8 of every 2048-entry round: first all eight
// block-table entries and recorded tags, then all eight pool tags, so a
// round costs two memory latencies whatever the request length.
__device__ __forceinline__ int check_request(const uint32_t* __restrict__ page_tags,
                                             int32_t num_pages, int32_t page_size,
                                             const int32_t* __restrict__ block_table,
                                             const uint32_t* __restrict__ expected,
                                             const int32_t* __restrict__ seq_lens,
                                             int32_t max_pages, int b) {
  constexpr int kThreads = 256, kUnroll = 8;
  const int tid = threadIdx.x;
  const int32_t L = seq_lens[b];
  const int64_t need = L > 0 ? (static_cast<int64_t>(L) + page_size - 1) / page_size : 0;
  // a request needing more pages than its row holds cannot be mapped
  int bad = need > max_pages ? 1 : 0;
  const int64_t n = bad ? 0 : need;
  const int32_t* row = block_table + static_cast<int64_t>(b) * max_pages;
  const uint32_t* exp = expected + static_cast<int64_t>(b) * max_pages;
  for (int64_t j0 = 0; j0 < n; j0 += kThreads * kUnroll) {
    int32_t pid[kUnroll];
    uint32_t want[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t j = j0 + u * kThreads + tid;
      pid[u] = 0;
      want[u] = 0;
      if (j < n) {
        pid[u] = row[j];
        want[u] = exp[j];
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t j = j0 + u * kThreads + tid;
      if (j < n) {
        const bool in_pool = pid[u] >= 0 && pid[u] < num_pages;
        const uint32_t have = in_pool ? page_tags[pid[u]] : 0u;
        bad |= (!in_pool || have != want[u]) ? 1 : 0;
      }
    }
  }
  return __syncthreads_or(bad);
}

}  // namespace pkv
