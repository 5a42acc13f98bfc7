// Helpers of the MFMA decode kernels (internal): direct-to-LDS loads, their
// waits, and exact conversion of e4m3 codes into MFMA operands.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef int v2i_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i_t lds_v2i_t;
typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s_t lds_v4s_t;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)p));
}

// 16 bytes per lane, global -> LDS: lane i's bytes land at lds + 16 i
__device__ __forceinline__ void dma16(uint32_t lds, uint32_t voff, const uint8_t* base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds), "v"(voff), "s"(base)
               : "memory");
}

// 4 bytes per lane, global -> LDS: lane i's bytes land at lds + 4 i
__device__ __forceinline__ void dma4(uint32_t lds, uint32_t voff, const uint8_t* base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2"
               :
               : "s"(lds), "v"(voff), "s"(base)
               : "memory");
}

// The same two loads marked non-temporal, for bytes a launch reads once (the
// KV stream): the line is not kept in the caches for reuse. On random 2 KB
// blocks this lifts the read rate from about 6.0 to about 6.7 TB/s.
__device__ __forceinline__ void dma16_stream(uint32_t lds, uint32_t voff, const uint8_t* base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
               :
               : "s"(lds), "v"(voff), "s"(base)
               : "memory");
}

__device__ __forceinline__ void dma4_stream(uint32_t lds, uint32_t voff, const uint8_t* base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2 nt"
               :
               : "s"(lds), "v"(voff), "s"(base)
               : "memory");
}

// wait until at most N of this wave's vector memory loads are outstanding
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// eight e4m3 codes (little-endian in w0, w1) -> eight bf16 / f16, exact
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  return bf16x8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// two transposing reads of four bf16 each -> one MFMA operand of eight
__device__ __forceinline__ bf16x8_t join_bf16x4(v4s_t a, v4s_t b) {
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& u) {
  return __builtin_bit_cast(bf16x8_t, u);
}

__device__ __forceinline__ f16x8_t fp8x8_to_f16(uint32_t w0, uint32_t w1) {
  const f16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false);
  const f16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true);
  const f16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false);
  const f16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true);
  return f16x8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

}  // namespace
