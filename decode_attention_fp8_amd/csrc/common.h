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
  if (c->dtype == PKV_KV_E4M3 && (!c->k_scale || (c->v_pool && !c->v_scale))) return PKV_EINVAL;
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

}  // namespace pkv
