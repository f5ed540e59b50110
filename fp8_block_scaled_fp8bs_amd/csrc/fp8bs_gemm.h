// GEMM kernels: Y[m][n] = sum_kb (block dot of E4M3 codes) * xs[m][kb] * ws[n/128][kb].
//
// Decode shapes (a handful of activation rows) make the product a stream
// over the weight codes: one weight byte is used by m multiply-adds, far
// below any matrix-core ridge point ("Kernel-Level Optimisations for LLM
// Inference and Training", section "Start with the bound: memory or
// compute"). The design splits the long K dimension across waves and
// workgroups and sums the partials in a fixed order ("A 23% faster GPU
// kernel, and a model that did not move", section "Why this shape is
// hard"); each per-block partial is rescaled in fp32 by its activation and
// weight block scales before it is accumulated.
//
// Work decomposition (both paths):
//   grid.x = row group (ROWS consecutive output columns n), grid.y = K split s.
//   A workgroup stages the activations of its K range in LDS once (casting
//   bf16 to E4M3 when fused), then its waves stream weight tiles from HBM
//   with 16-byte loads, several K blocks in flight per wave. waves_k waves
//   share a row range and interleave its K blocks; their fp32 partials are
//   summed in LDS in wave order. With split_k > 1 each workgroup writes an
//   fp32 partial tile that is summed over s in order by a second kernel.
#pragma once

#include "fp8bs_device.h"

namespace fp8bs {

struct GemmParams {
  const uint16_t* x;    // bf16 [m][k] (fused cast) or nullptr
  const uint8_t* xq;    // E4M3 [m][k] (pre-quantized) or nullptr
  const float* xs;      // fp32 [m][k/128] (pre-quantized)
  const uint8_t* wq;    // E4M3 [n][k]
  const float* ws;      // fp32 [n/128][k/128]
  uint16_t* y;          // bf16 [m][n]
  float* part;          // fp32 [split][m][n] when split > 1
  int m, n, k, kbn;     // kbn = k / 128
  int split;
};

// LDS layout of a workgroup:
//   act   [nblk][m][ACT_STRIDE] E4M3 codes of the staged activations
//   act_s [nblk][m] fp32 scales
//   red   partial-sum exchange area for waves_k > 1
__host__ __device__ inline int lds_act_bytes(int nblk, int m) {
  return ((nblk * m * (ACT_STRIDE + 4)) + 15) & ~15;
}

// Number of K blocks of split s (balanced: sizes differ by at most one).
__device__ __forceinline__ void split_range(int s, int split, int kbn, int& kb0, int& kb1) {
  kb0 = (int)((int64_t)s * kbn / split);
  kb1 = (int)((int64_t)(s + 1) * kbn / split);
}

// Stage the activations of blocks [kb0, kb0+nblk) into LDS. Fused: each
// thread casts CR quarter-blocks whose bf16 were loaded (before the weight
// prefetch) into xr; any remainder is loaded and cast afterwards.
// Pre-quantized: codes and scales are copied.
template <int NT, int CR>
__device__ __forceinline__ void load_act_quarters(const GemmParams& p, int kb0, int nblk, int tid,
                                                  int base, uint4 (&xr)[CR][4]) {
  const int G = nblk * p.m * 4;
#pragma unroll
  for (int i = 0; i < CR; ++i) {
    int g = base + tid + i * NT;
    g = g < G ? g : G - 1;
    const int qq = g & 3, bm = g >> 2;
    const int kbl = bm / p.m, m = bm - kbl * p.m;
    const uint4* src = reinterpret_cast<const uint4*>(
        p.x + (size_t)m * (size_t)p.k + (size_t)(kb0 + kbl) * BLK + qq * 32);
#pragma unroll
    for (int j = 0; j < 4; ++j) xr[i][j] = src[j];
  }
}

template <int NT, int CR>
__device__ __forceinline__ void cast_act_quarters(const GemmParams& p, int nblk, int tid, int base,
                                                  const uint4 (&xr)[CR][4], uint8_t* act,
                                                  float* act_s) {
  const int G = nblk * p.m * 4;
#pragma unroll
  for (int i = 0; i < CR; ++i) {
    const int gi = base + tid + i * NT;
    const int g = gi < G ? gi : G - 1;
    const int qq = g & 3, bm = g >> 2;  // bm = kbl * m + row
    uint32_t codes[8];
    const float s = cast_quarter(xr[i], codes);
    if (gi < G) {
      uint4* d = reinterpret_cast<uint4*>(act + bm * ACT_STRIDE + qq * 32);
      d[0] = make_uint4(codes[0], codes[1], codes[2], codes[3]);
      d[1] = make_uint4(codes[4], codes[5], codes[6], codes[7]);
      if (qq == 0) act_s[bm] = s;
    }
  }
}

template <int NT>
__device__ __forceinline__ void copy_act(const GemmParams& p, int kb0, int nblk, int tid,
                                         uint8_t* act, float* act_s) {
  const int rows = nblk * p.m;
  for (int i = tid; i < rows * 8; i += NT) {
    const int r = i >> 3, c = i & 7;
    const int kbl = r / p.m, m = r - kbl * p.m;
    const uint4 v = *reinterpret_cast<const uint4*>(p.xq + (size_t)m * (size_t)p.k +
                                                    (size_t)(kb0 + kbl) * BLK + 16 * c);
    *reinterpret_cast<uint4*>(act + r * ACT_STRIDE + 16 * c) = v;
  }
  for (int i = tid; i < rows; i += NT) {
    const int kbl = i / p.m, m = i - kbl * p.m;
    act_s[i] = p.xs[(size_t)m * (size_t)p.kbn + kb0 + kbl];
  }
}

// Cast (or copy) the activations of this workgroup's K range into LDS.
// The first CR quarters per thread were loaded into xr earlier.
template <int NT, int CR, bool FUSED>
__device__ __forceinline__ void stage_act(const GemmParams& p, int kb0, int nblk, int tid,
                                          const uint4 (&xr)[CR][4], uint8_t* act, float* act_s) {
  if constexpr (FUSED) {
    cast_act_quarters<NT, CR>(p, nblk, tid, 0, xr, act, act_s);
    const int G = nblk * p.m * 4;
    for (int base = CR * NT; base < G; base += CR * NT) {
      uint4 xr2[CR][4];
      load_act_quarters<NT, CR>(p, kb0, nblk, tid, base, xr2);
      cast_act_quarters<NT, CR>(p, nblk, tid, base, xr2, act, act_s);
    }
  } else {
    copy_act<NT>(p, kb0, nblk, tid, act, act_s);
  }
}

// ====================================================================
// MFMA path: v_mfma_f32_16x16x128_f8f6f4, A = 16 weight rows x 128 K,
// B = 128 K x 16 activation rows (zero beyond m). Lane l holds A row l%16
// and B column l%16, 32 bytes each, at K offsets 16*(l/16) .. +15 and
// 64 + 16*(l/16) .. +15 of the block (the same K positions for A and B, so
// the dot product is the block's). The result D[n][m] sits in lane l as
// rows 4*(l/16) + i, column l%16.
// ====================================================================

template <int MT, int TN, int WN, int WK, int D, bool FUSED, bool SPLIT>
__global__ __launch_bounds__(64 * WN * WK) void gemm_mfma_kernel(GemmParams p) {
  constexpr int NT = 64 * WN * WK;
  constexpr int ROWS = 16 * TN * WN;
  constexpr int CR = FUSED ? 4 : 1;
  extern __shared__ __align__(16) uint8_t lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave % WN, wk = wave / WN;
  const int s = blockIdx.y;
  int kb0, kb1;
  split_range(s, p.split, p.kbn, kb0, kb1);
  const int nblk = kb1 - kb0;
  const int M = p.m;

  uint8_t* act = lds;
  float* act_s = reinterpret_cast<float*>(lds + nblk * M * ACT_STRIDE);
  f32x4* red = reinterpret_cast<f32x4*>(lds + lds_act_bytes(nblk, M));

  const int row0 = blockIdx.x * ROWS + wn * 16 * TN;
  const int l16 = lane & 15, g16 = lane >> 4;
  const uint8_t* wrow = p.wq + (size_t)(row0 + l16) * (size_t)p.k + 16 * g16;
  const int nj = nblk > wk ? (nblk - wk + WK - 1) / WK : 0;  // this wave's K blocks

  // 1. activation bf16 loads first (so their wait does not wait on weights)
  uint4 xr[CR][4];
  if constexpr (FUSED) load_act_quarters<NT, CR>(p, kb0, nblk, tid, 0, xr);

  // 2. weight prefetch: D blocks per wave in flight
  i32x8 wb[D][TN];
  auto load_block = [&](int d, int j) {
    const int jc = j < nj ? j : (nj > 0 ? nj - 1 : 0);
    int kb = kb0 + wk + jc * WK;
    kb = kb < p.kbn ? kb : p.kbn - 1;
    const uint8_t* src = wrow + (size_t)kb * BLK;
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      const uint4* st = reinterpret_cast<const uint4*>(src + (size_t)t * 16 * (size_t)p.k);
      const uint4 lo = st[0];
      const uint4 hi = st[4];
      wb[d][t] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                       (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
  };
#pragma unroll
  for (int d = 0; d < D; ++d) load_block(d, d);

  // 3. stage activations in LDS
  stage_act<NT, CR, FUSED>(p, kb0, nblk, tid, xr, act, act_s);
  __syncthreads();

  // 4. stream K blocks
  f32x4 acc[TN][MT];
#pragma unroll
  for (int t = 0; t < TN; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int d, int j) {
    const int kbl = wk + j * WK;
    const int kb = kb0 + kbl;
    i32x8 bop[MT];
    float sa[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = l16 + 16 * mt;
      if (m < M) {
        const uint8_t* a = act + (kbl * M + m) * ACT_STRIDE + 16 * g16;
        const uint4 lo = *reinterpret_cast<const uint4*>(a);
        const uint4 hi = *reinterpret_cast<const uint4*>(a + 64);
        bop[mt] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                        (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        sa[mt] = act_s[kbl * M + m];
      } else {
        bop[mt] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
        sa[mt] = 0.0f;
      }
    }
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      const int nb = (row0 + 16 * t) / BLK;
      const float sw = p.ws[(size_t)nb * (size_t)p.kbn + kb];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        const f32x4 pb =
            __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wb[d][t], bop[mt], z, 0, 0, 0, 0, 0, 0);
        const float sc = sa[mt] * sw;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[t][mt][i] = __builtin_fmaf(pb[i], sc, acc[t][mt][i]);
      }
    }
  };

  const int ngrp = (nj + D - 1) / D;
  for (int g = 0; g + 1 < ngrp; ++g) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      compute(d, g * D + d);
      load_block(d, (g + 1) * D + d);
    }
  }
  if (ngrp > 0) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int j = (ngrp - 1) * D + d;
      if (j < nj) compute(d, j);
    }
  }

  // 5. sum the waves_k partials in wave order
  if constexpr (WK > 1) {
    if (wk > 0) {
#pragma unroll
      for (int t = 0; t < TN; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          red[((((wk - 1) * WN + wn) * TN + t) * MT + mt) * 64 + lane] = acc[t][mt];
    }
    __syncthreads();
    if (wk == 0) {
      for (int w = 1; w < WK; ++w)
#pragma unroll
        for (int t = 0; t < TN; ++t)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            acc[t][mt] += red[((((w - 1) * WN + wn) * TN + t) * MT + mt) * 64 + lane];
    }
  }

  // 6. output: rows n = row0 + 16t + 4*(l/16) + i, column m = l%16 + 16mt
  if (wk == 0) {
#pragma unroll
    for (int t = 0; t < TN; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int m = l16 + 16 * mt;
        if (m < M) {
          const int n = row0 + 16 * t + 4 * g16;
          if constexpr (SPLIT) {
            float4* dst = reinterpret_cast<float4*>(p.part + ((size_t)s * M + m) * (size_t)p.n + n);
            *dst = make_float4(acc[t][mt][0], acc[t][mt][1], acc[t][mt][2], acc[t][mt][3]);
          } else {
            uint2* dst = reinterpret_cast<uint2*>(p.y + (size_t)m * (size_t)p.n + n);
            *dst = make_uint2(pack_bf16x2(acc[t][mt][0], acc[t][mt][1]),
                              pack_bf16x2(acc[t][mt][2], acc[t][mt][3]));
          }
        }
      }
  }
}

// ====================================================================
// DOT path (smallest m): lane l handles weight row (l/8) of each 8-row
// group and the 16-byte K segment l%8 of each block; it converts its 16
// codes to fp32 and forms m dot products against the decoded activation
// codes of the same K positions. Per block the lane rescales its partial by
// xs * ws; the 8 lanes of a row are summed once at the end.
// ====================================================================

template <int MD, int RT, int WN, int WK, int D, bool FUSED, bool SPLIT>
__global__ __launch_bounds__(64 * WN * WK) void gemm_dot_kernel(GemmParams p) {
  constexpr int NT = 64 * WN * WK;
  constexpr int ROWS = 8 * RT * WN;
  constexpr int CR = FUSED ? 4 : 1;
  extern __shared__ __align__(16) uint8_t lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave % WN, wk = wave / WN;
  const int s = blockIdx.y;
  int kb0, kb1;
  split_range(s, p.split, p.kbn, kb0, kb1);
  const int nblk = kb1 - kb0;
  const int M = p.m;

  uint8_t* act = lds;
  float* act_s = reinterpret_cast<float*>(lds + nblk * M * ACT_STRIDE);
  float* red = reinterpret_cast<float*>(lds + lds_act_bytes(nblk, M));

  const int row0 = blockIdx.x * ROWS + wn * 8 * RT;
  const int r8 = lane >> 3, seg = lane & 7;
  const uint8_t* wrow = p.wq + (size_t)(row0 + r8) * (size_t)p.k + 16 * seg;
  const int nj = nblk > wk ? (nblk - wk + WK - 1) / WK : 0;

  uint4 xr[CR][4];
  if constexpr (FUSED) load_act_quarters<NT, CR>(p, kb0, nblk, tid, 0, xr);

  uint4 wb[D][RT];
  auto load_block = [&](int d, int j) {
    const int jc = j < nj ? j : (nj > 0 ? nj - 1 : 0);
    int kb = kb0 + wk + jc * WK;
    kb = kb < p.kbn ? kb : p.kbn - 1;
    const uint8_t* src = wrow + (size_t)kb * BLK;
#pragma unroll
    for (int t = 0; t < RT; ++t)
      wb[d][t] = *reinterpret_cast<const uint4*>(src + (size_t)t * 8 * (size_t)p.k);
  };
#pragma unroll
  for (int d = 0; d < D; ++d) load_block(d, d);

  stage_act<NT, CR, FUSED>(p, kb0, nblk, tid, xr, act, act_s);
  __syncthreads();

  float acc[RT][MD];
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int m = 0; m < MD; ++m) acc[t][m] = 0.0f;

  auto compute = [&](int d, int j) {
    const int kbl = wk + j * WK;
    const int kb = kb0 + kbl;
    float av[MD][16];
    float sa[MD];
#pragma unroll
    for (int m = 0; m < MD; ++m) {
      if (m < M) {
        const uint4 c = *reinterpret_cast<const uint4*>(act + (kbl * M + m) * ACT_STRIDE + 16 * seg);
        const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) e4m3x4_decode(cw[i], &av[m][4 * i]);
        sa[m] = act_s[kbl * M + m];
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) av[m][i] = 0.0f;
        sa[m] = 0.0f;
      }
    }
    const int nb = row0 / BLK;
    const float sw = p.ws[(size_t)nb * (size_t)p.kbn + kb];
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const uint32_t ww[4] = {wb[d][t].x, wb[d][t].y, wb[d][t].z, wb[d][t].w};
      float wv[16];
#pragma unroll
      for (int i = 0; i < 4; ++i) e4m3x4_decode(ww[i], &wv[4 * i]);
#pragma unroll
      for (int m = 0; m < MD; ++m) {
        float pd = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) pd = __builtin_fmaf(wv[i], av[m][i], pd);
        acc[t][m] = __builtin_fmaf(pd, sa[m] * sw, acc[t][m]);
      }
    }
  };

  const int ngrp = (nj + D - 1) / D;
  for (int g = 0; g + 1 < ngrp; ++g) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      compute(d, g * D + d);
      load_block(d, (g + 1) * D + d);
    }
  }
  if (ngrp > 0) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int j = (ngrp - 1) * D + d;
      if (j < nj) compute(d, j);
    }
  }

  // sum the 8 K segments of each row (fixed pairing), then the waves_k partials
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int m = 0; m < MD; ++m) acc[t][m] = octet_sum(acc[t][m]);

  if constexpr (WK > 1) {
    if (wk > 0) {
#pragma unroll
      for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int m = 0; m < MD; ++m)
          red[((((wk - 1) * WN + wn) * RT + t) * MD + m) * 64 + lane] = acc[t][m];
    }
    __syncthreads();
    if (wk == 0) {
      for (int w = 1; w < WK; ++w)
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
          for (int m = 0; m < MD; ++m)
            acc[t][m] += red[((((w - 1) * WN + wn) * RT + t) * MD + m) * 64 + lane];
    }
  }

  if (wk == 0 && seg == 0) {
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const int n = row0 + 8 * t + r8;
#pragma unroll
      for (int m = 0; m < MD; ++m) {
        if (m < M) {
          if constexpr (SPLIT)
            p.part[((size_t)s * M + m) * (size_t)p.n + n] = acc[t][m];
          else
            p.y[(size_t)m * (size_t)p.n + n] = (uint16_t)bf16_rne(acc[t][m]);
        }
      }
    }
  }
}

}  // namespace fp8bs
