// pkv_fill_u32 and pkv_read_u32: plain write and read kernels (not part of
// the method), the measurement's last-level cache flush.
//
// A timed decode step should find none of the previous step's cache lines
// in the 256 MB last-level cache (MALL), as in serving, where the other
// layers of the model run in between. Writing a buffer of several times that
// size between timed steps evicts them; reading it back afterwards evicts
// the dirty lines the writes left, so that their write-back happens during
// the flush rather than inside the next timed step. Kernels rather than a
// memset, so that they behave the same inside a captured graph.
#include "common.h"

namespace {

__global__ void __launch_bounds__(256) fill_u32_kernel(uint4* __restrict__ dst, int64_t n16,
                                                       uint32_t* __restrict__ tail,
                                                       int n_tail, uint32_t value) {
  const uint4 v = make_uint4(value, value, value, value);
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16;
       i += stride)
    dst[i] = v;
  if (blockIdx.x == 0 && static_cast<int>(threadIdx.x) < n_tail) tail[threadIdx.x] = value;
}

// Reads every word; each workgroup XORs what it read into one word of sink
// (so the loads cannot be dropped).
__global__ void __launch_bounds__(256) read_u32_kernel(const uint4* __restrict__ src, int64_t n16,
                                                       uint32_t* __restrict__ sink) {
  uint32_t x = 0;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16;
       i += stride) {
    const uint4 v = src[i];
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  for (int off = 32; off > 0; off >>= 1) x ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(x), off));
  __shared__ uint32_t red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) atomicXor(sink, red[0] ^ red[1] ^ red[2] ^ red[3]);
}

}  // namespace

extern "C" int pkv_read_u32(const void* src, int64_t n_words, uint32_t* sink, hipStream_t stream) {
  if (!src || !sink || n_words < 0 || (reinterpret_cast<uintptr_t>(src) & 15u)) return PKV_EINVAL;
  const int64_t n16 = n_words / 4;
  if (n16 == 0) return PKV_OK;
  const int blocks = static_cast<int>(std::min<int64_t>(pkv::cdiv(n16, 256), 8192));
  read_u32_kernel<<<blocks, 256, 0, stream>>>(static_cast<const uint4*>(src), n16, sink);
  return pkv::launch_status();
}

extern "C" int pkv_fill_u32(void* dst, int64_t n_words, uint32_t value, hipStream_t stream) {
  if (!dst || n_words < 0 || (reinterpret_cast<uintptr_t>(dst) & 15u)) return PKV_EINVAL;
  if (n_words == 0) return PKV_OK;
  const int64_t n16 = n_words / 4;
  const int n_tail = static_cast<int>(n_words - 4 * n16);
  uint32_t* tail = static_cast<uint32_t*>(dst) + 4 * n16;
  const int blocks = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(pkv::cdiv(n16, 256), 8192)));
  fill_u32_kernel<<<blocks, 256, 0, stream>>>(static_cast<uint4*>(dst), n16, tail, n_tail, value);
  return pkv::launch_status();
}
