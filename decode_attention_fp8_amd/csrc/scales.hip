// pkv_scales_from_amax: static e4m3 scales s = fl32(amax / 448).
//
// "Smaller, faster, safer", section "Quantizing the KV cache", stores the
// cache in e4m3 without stating a scale rule; the rule taken here is one
// static scale per tensor or per kv head from the largest magnitude, 448
// being the largest e4m3 value.
//
// Three launches on the caller's stream, no allocation: clear the output
// (used as uint32 scratch), a max-of-|x| reduction with one atomicMax per
// workgroup, then the division. |bf16| bit patterns order like their
// magnitudes, so the reduction works on integers.
#include "common.h"

namespace {

__global__ void clear_u32(uint32_t* p, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// grid (x, heads): workgroup (x, h) scans rows x, x + gridDim.x, ... of head h.
__global__ void __launch_bounds__(256) amax_kernel(const uint16_t* __restrict__ x, int64_t n_rows,
                                                   int heads, int dim, int per_head,
                                                   uint32_t* __restrict__ out_bits) {
  const int h = blockIdx.y;
  const int vec_per_row = dim / 8;  // 8 bf16 per 16-byte load
  const int64_t n_vec = n_rows * vec_per_row;
  uint32_t m = 0;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n_vec;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t row = i / vec_per_row;
    const int v = static_cast<int>(i - row * vec_per_row);
    const uint4 w = *reinterpret_cast<const uint4*>(x + (row * heads + h) * dim + v * 8);
    const uint32_t words[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      m = max(m, words[k] & 0x7FFFu);
      m = max(m, (words[k] >> 16) & 0x7FFFu);
    }
  }
  // workgroup max
  for (int off = 32; off > 0; off >>= 1) m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), off)));
  __shared__ uint32_t red[4];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (lane == 0) red[wid] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = red[0];
    for (int k = 1; k < (blockDim.x >> 6); ++k) r = max(r, red[k]);
    atomicMax(out_bits + (per_head ? h : 0), r);
  }
}

__global__ void finalize_kernel(float* scale_out, int heads, int per_head) {
  const int h = threadIdx.x;
  const uint32_t* bits = reinterpret_cast<const uint32_t*>(scale_out);
  uint32_t b = 0;
  if (h < heads) b = bits[per_head ? h : 0];
  __syncthreads();  // every read of the scratch words happens before any write
  if (h < heads) {
    const float amax = __uint_as_float(b << 16);
    scale_out[h] = (amax == 0.0f) ? 1.0f : __fdiv_rn(amax, 448.0f);
  }
}

}  // namespace

extern "C" int pkv_scales_from_amax(const void* x, int64_t n_rows, int32_t num_heads,
                                    int32_t head_dim, int32_t per_head, float* scale_out,
                                    hipStream_t stream) {
  if ((reinterpret_cast<uintptr_t>(x) & 15u) != 0) return PKV_EINVAL;
  if (!x || !scale_out || n_rows < 1 || num_heads < 1 || num_heads > 1024 || head_dim < 8 ||
      head_dim % 8)
    return PKV_EINVAL;
  auto* bits = reinterpret_cast<uint32_t*>(scale_out);
  clear_u32<<<1, 1024, 0, stream>>>(bits, num_heads);
  const int64_t n_vec = n_rows * (head_dim / 8);
  int gx = static_cast<int>(std::min<int64_t>(pkv::cdiv(n_vec, 256), 2048 / num_heads + 1));
  amax_kernel<<<dim3(gx, num_heads), 256, 0, stream>>>(static_cast<const uint16_t*>(x), n_rows,
                                                         num_heads, head_dim, per_head, bits);
  finalize_kernel<<<1, 1024, 0, stream>>>(scale_out, num_heads, per_head);
  return pkv::launch_status();
}
