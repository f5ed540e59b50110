// Bandwidth reference kernels: a streaming read and a plain copy, launched
// with the same 16-byte-per-lane access width as the GEMM's weight stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8bs {

// Grid-stride streaming read, 4 loads in flight per lane per step. The XOR
// of everything read is stored only if it equals a value no real input
// produces in practice, so the loads cannot be removed.
__global__ __launch_bounds__(256) void diag_read_kernel(const uint4* __restrict__ src,
                                                        int64_t n16, uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^
           d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9E3779B9u) sink[threadIdx.x & 3] = acc;
}

__global__ __launch_bounds__(256) void diag_copy_kernel(const uint4* __restrict__ src,
                                                        uint4* __restrict__ dst, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

}  // namespace fp8bs
