// Second-stage kernels of the GEMM: the fixed-order sum of split-K partials
// and the zero fill used when K is empty.
#pragma once

#include "fp8bs_device.h"

namespace fp8bs {

// Sum of the split partials in split order, rounded once to bf16.
// Each thread produces 4 consecutive outputs.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part,
                                                            int split, int64_t mn4,
                                                            uint16_t* __restrict__ y) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= mn4) return;
  const float4* src = reinterpret_cast<const float4*>(part);
  float4 a = src[i];
  for (int s = 1; s < split; ++s) {
    const float4 b = src[(int64_t)s * mn4 + i];
    a.x += b.x;
    a.y += b.y;
    a.z += b.z;
    a.w += b.w;
  }
  reinterpret_cast<uint2*>(y)[i] = make_uint2(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w));
}

// Y = 0 (the empty sum, k == 0). Count in units of 8 bytes.
__global__ __launch_bounds__(256) void zero_fill_kernel(uint2* __restrict__ y, int64_t n8) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n8) y[i] = make_uint2(0u, 0u);
}

}  // namespace fp8bs
