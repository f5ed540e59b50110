// Second-stage kernels of the GEMM: the fixed-order sum of split-K partials
// (plain, or with the MLP epilogue fused in) and the zero fill used when K is
// empty.
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

// The split sum fused with the MLP epilogue (SwiGLU and the 1x128 cast of
// its output; output columns [0, I) are the gate, [I, 2I) the up projection,
// I = n/2). One wave per (128-column block b of h, activation row m): lane l
// takes columns 2l, 2l+1 of the block. Each lane sums the split partials of
// its gate and up columns in split order and rounds them once to bf16,
// stores them to y (the bits splitk_reduce_kernel gives), and the wave
// applies swiglu_cast_wave. Grid: (I/128, m) waves of 64 threads.
__global__ __launch_bounds__(64) void splitk_reduce_swiglu_kernel(
    const float* __restrict__ part, int split, int m, int n, uint16_t* __restrict__ y,
    uint8_t* __restrict__ hq, float* __restrict__ hs) {
  const int b = blockIdx.x, row = blockIdx.y, l = threadIdx.x;
  const int inter = n >> 1;
  const size_t mn = (size_t)m * (size_t)n;
  const size_t go = (size_t)row * (size_t)n + (size_t)b * BLK + 2 * l;
  const size_t uo = go + (size_t)inter;
  float2 g = *reinterpret_cast<const float2*>(part + go);
  float2 u = *reinterpret_cast<const float2*>(part + uo);
  for (int s = 1; s < split; ++s) {
    const float2 gs = *reinterpret_cast<const float2*>(part + (size_t)s * mn + go);
    const float2 us = *reinterpret_cast<const float2*>(part + (size_t)s * mn + uo);
    g.x += gs.x;
    g.y += gs.y;
    u.x += us.x;
    u.y += us.y;
  }
  const uint32_t gw = pack_bf16x2(g.x, g.y), uw = pack_bf16x2(u.x, u.y);
  *reinterpret_cast<uint32_t*>(y + go) = gw;
  *reinterpret_cast<uint32_t*>(y + uo) = uw;
  swiglu_cast_wave(gw, uw, l, hq + (size_t)row * (size_t)inter + (size_t)b * BLK,
                   hs + (size_t)row * (size_t)(inter / BLK) + b);
}

// Y = 0 (the empty sum, k == 0). Count in units of 8 bytes.
__global__ __launch_bounds__(256) void zero_fill_kernel(uint2* __restrict__ y, int64_t n8) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n8) y[i] = make_uint2(0u, 0u);
}

}  // namespace fp8bs
