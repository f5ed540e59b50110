// Quantization kernels: weights in 128x128 blocks, activations in 1x128
// blocks, and the fp32 -> E4M3 encoder utility.
#pragma once

#include "fp8bs_device.h"

namespace fp8bs {

// Weight codes from row-major [n][k] to the tile layout the GEMM kernels
// read with FP8BS_LAYOUT_TILES (tile_layout_off in fp8bs_gemm.h): 16-row x
// 128-column tiles of 2 KB, each half of a wave's MFMA A operand one
// contiguous KB. One thread per 16-byte chunk W[R][128kb + 32g + 16h ..]:
// consecutive threads read consecutive chunks; the chunk goes to tile
// (R/16, kb), half h, lane slot 16g + R%16.
__global__ __launch_bounds__(256) void pack_weight_kernel(const uint4* __restrict__ src,
                                                          int64_t chunks, int64_t kc, int64_t kbn,
                                                          uint4* __restrict__ dst) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= chunks) return;
  const int64_t r = c / kc;
  const int rem = (int)(c - r * kc);
  const int kb = rem >> 3, g = (rem >> 1) & 3, h = rem & 1;
  dst[((r >> 4) * kbn + kb) * 128 + h * 64 + 16 * g + (r & 15)] = src[c];
}

// One workgroup of 256 threads per 128x128 weight block. Thread t handles
// half a block row: row t/2, columns 64*(t%2) .. +63 (128 contiguous bytes of
// bf16 in, 64 contiguous bytes of codes out).
__global__ __launch_bounds__(256) void quant_weight_kernel(const uint16_t* __restrict__ w,
                                                           int64_t k, uint8_t* __restrict__ q,
                                                           float* __restrict__ scale) {
  const int nb = blockIdx.x, kb = blockIdx.y;
  const int tid = threadIdx.x;
  const int row = tid >> 1, half = tid & 1;
  const size_t off = (size_t)(nb * BLK + row) * (size_t)k + (size_t)kb * BLK + half * 64;
  const uint4* src = reinterpret_cast<const uint4*>(w + off);
  float x[64];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint4 v = src[i];
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[8 * i + 2 * j] = bf16_lo(d[j]);
      x[8 * i + 2 * j + 1] = bf16_hi(d[j]);
    }
  }
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < 64; ++i) am = __builtin_fmaxf(am, __builtin_fabsf(x[i]));
  am = wave_max(am);
  __shared__ float red[4];
  if ((tid & 63) == 0) red[tid >> 6] = am;
  __syncthreads();
  am = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
  const float s = am / 448.0f;
  block_quotients(x, am, s);
  uint4* dst = reinterpret_cast<uint4*>(q + off);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint4 c;
    c.x = e4m3x4(x[16 * i + 0], x[16 * i + 1], x[16 * i + 2], x[16 * i + 3]);
    c.y = e4m3x4(x[16 * i + 4], x[16 * i + 5], x[16 * i + 6], x[16 * i + 7]);
    c.z = e4m3x4(x[16 * i + 8], x[16 * i + 9], x[16 * i + 10], x[16 * i + 11]);
    c.w = e4m3x4(x[16 * i + 12], x[16 * i + 13], x[16 * i + 14], x[16 * i + 15]);
    dst[i] = c;
  }
  if (tid == 0) scale[(size_t)nb * (size_t)(k / BLK) + kb] = s;
}

// Activations: one DPP quad of lanes per 1x128 block (lane q of the quad
// handles columns 32q .. 32q+31), 64 blocks per 256-thread workgroup. The
// block math is cast_quarter, the same function the fused GEMM runs.
__global__ __launch_bounds__(256) void quant_act_kernel(const uint16_t* __restrict__ x,
                                                        int64_t nblocks, int64_t k,
                                                        uint8_t* __restrict__ q,
                                                        float* __restrict__ scale) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;  // quarter index
  const int64_t b = g >> 2;                                    // block index = row*KB + kb
  const bool valid = b < nblocks;
  const int64_t bc = valid ? b : nblocks - 1;                  // whole quads are valid or not
  const int64_t kbn = k / BLK;
  const int64_t row = bc / kbn, kb = bc - row * kbn;
  const int qq = (int)(g & 3);
  const size_t off = (size_t)row * (size_t)k + (size_t)kb * BLK + qq * 32;
  const uint4* src = reinterpret_cast<const uint4*>(x + off);
  uint4 xw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) xw[i] = src[i];
  uint32_t codes[8];
  const float s = cast_quarter(xw, codes);
  if (valid) {
    uint4* dst = reinterpret_cast<uint4*>(q + off);
    dst[0] = make_uint4(codes[0], codes[1], codes[2], codes[3]);
    dst[1] = make_uint4(codes[4], codes[5], codes[6], codes[7]);
    if (qq == 0) scale[bc] = s;
  }
}

// Standalone MLP epilogue: y[m][2I] bf16 (gate in columns 0..I-1, up in
// I..2I-1) -> h = silu(gate) * up rounded to bf16, cast per row per 128
// columns: codes hq[m][I], scales hs[m][I/128]. One wave per (128-column
// block, row), running swiglu_cast_wave, the function the fused GEMM
// epilogues run on the same bf16 values. Grid: (I/128, m) waves.
__global__ __launch_bounds__(64) void swiglu_quant_kernel(const uint16_t* __restrict__ y,
                                                          int64_t inter,
                                                          uint8_t* __restrict__ hq,
                                                          float* __restrict__ hs) {
  const int64_t b = blockIdx.x, row = blockIdx.y;
  const int l = threadIdx.x;
  const uint16_t* g = y + row * (2 * inter) + b * BLK + 2 * l;
  const uint32_t gw = *reinterpret_cast<const uint32_t*>(g);
  const uint32_t uw = *reinterpret_cast<const uint32_t*>(g + inter);
  swiglu_cast_wave(gw, uw, l, hq + row * inter + b * BLK, hs + row * (inter / BLK) + b);
}

// Encoder utility: mode 0 = the quantizers' encoder, 1 = hardware, 2 = software.
__global__ __launch_bounds__(256) void encode_kernel(const float* __restrict__ in, int64_t count,
                                                     uint8_t* __restrict__ out, int mode) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t base = i * 4;
  if (base >= count) return;
  float v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = (base + j < count) ? in[base + j] : 0.0f;
  uint32_t c;
  if (mode == 1)
    c = e4m3x4_hw(v[0], v[1], v[2], v[3]);
  else if (mode == 2)
    c = e4m3x4_sw(v[0], v[1], v[2], v[3]);
  else
    c = e4m3x4(v[0], v[1], v[2], v[3]);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (base + j < count) out[base + j] = (uint8_t)(c >> (8 * j));
}

}  // namespace fp8bs
