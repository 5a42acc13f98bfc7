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

// -------------------------------------------------------------- device side
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
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
// 16-byte word.
__device__ __forceinline__ uint4 encode16(const uint4& w0, const uint4& w1, float s) {
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

}  // namespace pkv
