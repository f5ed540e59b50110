// Prefill-size GEMM (many activation rows): the same block-scaled product,
// Y[m][n] = sum_kb (block dot of E4M3 codes) * xs[m][kb] * ws[n/128][kb], in
// the regime where the multiply is bound by the matrix cores rather than by
// streaming the weights ("Kernel-Level Optimisations for LLM Inference and
// Training", section "Start with the bound: memory or compute": prefill
// processes thousands of tokens at once and is compute-bound).
//
// Decomposition: a workgroup of 2 WN waves owns a 64 WN (n) x 128 (m) output
// tile (WN = 2 or 4 waves along n, 2 along m); each wave owns a 64 x 64 part.
// K advances one 128-deep block at a time through two LDS stages: the weight
// rows and the activation rows of the block (128 bytes each, padded to 144 so
// the MFMA operand reads of 16 consecutive rows spread over the banks) and
// the block's activation scales. While the waves multiply out of one stage,
// the codes of the next block are on their way from memory into registers;
// they are written to the other stage after the multiplies. When the output
// tiles alone cannot fill the GPU, K is split across workgroups and the fp32
// partials are summed in split order by the reduce kernel. Each wave issues one
// v_mfma_f32_16x16x128_f8f6f4 per (16-row weight tile, 16-row activation
// tile) pair and block, with the weight tile as the A operand: the four
// results a lane holds share one activation row and one weight block, so the
// per-block rescale is one product of scales per lane and tile, applied with
// fp32 fused multiply-adds in block order.
#pragma once

#include "fp8bs_gemm.h"

namespace fp8bs {

constexpr int PF_TILE_M = 128;   // output tile rows along m
constexpr int PF_STRIDE = 144;   // LDS bytes per staged row (128 + 16 pad)

// Output columns (n) of a workgroup with WN waves along n.
__host__ __device__ constexpr int pf_tile_n(int wn) { return 64 * wn; }

// LDS bytes of one stage: weight rows, activation rows, activation scales.
__host__ __device__ constexpr int pf_stage_bytes(int wn) {
  return pf_tile_n(wn) * PF_STRIDE + PF_TILE_M * PF_STRIDE + PF_TILE_M * 4;
}
__host__ __device__ constexpr int pf_lds_bytes(int wn) { return 2 * pf_stage_bytes(wn); }

// The global loads of one K block, held in registers until they are written
// to LDS. With T = 128 WN threads, thread tid fetches the 16-byte segments
// c % 8 of weight rows c / 8 for c = tid + T i (i = 0..3), of activation
// rows c / 8 for c = tid + T i (i < 8 / WN), and (threads 0..127) the
// activation scale of row tid. Named members rather than arrays, so the set
// always lives in registers.
struct PrefillSet {
  uint4 w0, w1, w2, w3, x0, x1, x2, x3;
  float s;
};

// Activation rows past m load row m-1 again (their outputs are dropped).
__device__ __forceinline__ uint4 prefill_load_x(const GemmParams& p, int m0, int kb, int c) {
  const int r = c >> 3, seg = c & 7;
  int mr = m0 + r;
  mr = mr < p.m ? mr : p.m - 1;
  return *reinterpret_cast<const uint4*>(p.xq + (size_t)mr * (size_t)p.k + (size_t)kb * BLK +
                                         16 * seg);
}

// plain (cached) loads: every weight tile is read by all m tiles
__device__ __forceinline__ uint4 prefill_load_w(const GemmParams& p, int n0, int kb, int c) {
  const int r = c >> 3, seg = c & 7;
  return *reinterpret_cast<const uint4*>(p.wq + (size_t)(n0 + r) * (size_t)p.k +
                                         (size_t)kb * BLK + 16 * seg);
}

template <int WN>
__device__ __forceinline__ void prefill_fetch(const GemmParams& p, int n0, int m0, int kb,
                                              int tid, PrefillSet& f) {
  constexpr int T = 128 * WN;
  f.w0 = prefill_load_w(p, n0, kb, tid);
  f.x0 = prefill_load_x(p, m0, kb, tid);
  f.w1 = prefill_load_w(p, n0, kb, tid + T);
  f.x1 = prefill_load_x(p, m0, kb, tid + T);
  f.w2 = prefill_load_w(p, n0, kb, tid + 2 * T);
  f.w3 = prefill_load_w(p, n0, kb, tid + 3 * T);
  if constexpr (WN == 2) {
    f.x2 = prefill_load_x(p, m0, kb, tid + 2 * T);
    f.x3 = prefill_load_x(p, m0, kb, tid + 3 * T);
  }
  int ms = m0 + (tid & (PF_TILE_M - 1));
  ms = ms < p.m ? ms : p.m - 1;
  f.s = p.xs[(size_t)ms * (size_t)p.kbn + kb];
}

__device__ __forceinline__ void prefill_put(uint8_t* rows, int c, uint4 v) {
  *reinterpret_cast<uint4*>(rows + (c >> 3) * PF_STRIDE + 16 * (c & 7)) = v;
}

template <int WN>
__device__ __forceinline__ void prefill_stage(const PrefillSet& f, int tid, uint8_t* stage) {
  constexpr int T = 128 * WN;
  uint8_t* wl = stage;
  uint8_t* xl = stage + pf_tile_n(WN) * PF_STRIDE;
  prefill_put(wl, tid, f.w0);
  prefill_put(wl, tid + T, f.w1);
  prefill_put(wl, tid + 2 * T, f.w2);
  prefill_put(wl, tid + 3 * T, f.w3);
  prefill_put(xl, tid, f.x0);
  prefill_put(xl, tid + T, f.x1);
  if constexpr (WN == 2) {
    prefill_put(xl, tid + 2 * T, f.x2);
    prefill_put(xl, tid + 3 * T, f.x3);
  }
  if (tid < PF_TILE_M)
    reinterpret_cast<float*>(stage + pf_tile_n(WN) * PF_STRIDE + PF_TILE_M * PF_STRIDE)[tid] = f.s;
}

// 32 K bytes of staged row `row` for lane group g (the MFMA operand layout:
// lane l holds row l % 16, K bytes 32 (l / 16) .. +31).
__device__ __forceinline__ i32x8 prefill_operand(const uint8_t* rows, int row, int g) {
  const uint8_t* a = rows + row * PF_STRIDE + 32 * g;
  const uint4 lo = *reinterpret_cast<const uint4*>(a);
  const uint4 hi = *reinterpret_cast<const uint4*>(a + 16);
  return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// One K block out of an LDS stage: 16 MFMAs per wave (weight rows
// 64 wn .. +63 of the tile, activation rows 64 wm .. +63), rescaled into acc.
template <int WN>
__device__ __forceinline__ void prefill_block(const uint8_t* stage, float sw, int wn, int wm,
                                              int l16, int g, f32x4 (&acc)[4][4]) {
  const uint8_t* wl = stage;
  const uint8_t* xl = stage + pf_tile_n(WN) * PF_STRIDE;
  const float* sl = reinterpret_cast<const float*>(xl + PF_TILE_M * PF_STRIDE);
  i32x8 bop[4];
  float sc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int mr = 64 * wm + 16 * j + l16;
    bop[j] = prefill_operand(xl, mr, g);
    sc[j] = sl[mr] * sw;
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const i32x8 aop = prefill_operand(wl, 64 * wn + 16 * t + l16, g);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      const f32x4 pb =
          __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop, bop[j], z, 0, 0, 0, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[t][j][i] = __builtin_fmaf(pb[i], sc[j], acc[t][j][i]);
    }
  }
}

// grid: (n / (64 WN), ceil(m / 128), split); 128 WN threads; pf_lds_bytes(WN)
// of dynamic LDS. Activations are E4M3 codes and scales (p.xq, p.xs); n is a
// multiple of 64 WN. Workgroup z takes the K blocks of split range z and
// writes bf16 outputs (split 1) or an fp32 partial tile part[z][m][n].
// Block kb + 1 is fetched into registers while block kb is multiplied out of
// LDS, and staged after it; a compute unit holds two 4-wave or one 8-wave
// workgroup (at least 2 waves per SIMD, at most 256 VGPRs), so while one
// wave waits on its loads the other multiplies.
template <int WN>
__global__ __launch_bounds__(128 * WN, 2) void gemm_prefill_kernel(GemmParams p) {
  extern __shared__ __align__(16) uint8_t lds_all[];
  constexpr int STAGE = pf_stage_bytes(WN);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave % WN, wm = wave / WN;
  const int n0 = blockIdx.x * pf_tile_n(WN), m0 = blockIdx.y * PF_TILE_M;
  const int l16 = lane & 15, g = lane >> 4;
  int kb0, kb1;
  split_range(blockIdx.z, p.split, p.kbn, kb0, kb1);
  const int last = kb1 - 1;
  // this wave's 64 weight rows lie in one 128-row scale block
  const float* wsrow = p.ws + (size_t)((n0 + 64 * wn) / BLK) * (size_t)p.kbn;

  f32x4 acc[4][4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  PrefillSet f;
  prefill_fetch<WN>(p, n0, m0, kb0, tid, f);
  prefill_stage<WN>(f, tid, lds_all);
  lds_barrier();
  // iteration kb: stage (kb - kb0) & 1 holds block kb (the last iteration
  // loads its own block again; what it stages is never read)
  for (int kb = kb0; kb <= last; ++kb) {
    const int sel = (kb - kb0) & 1;
    prefill_fetch<WN>(p, n0, m0, kb < last ? kb + 1 : kb, tid, f);
    prefill_block<WN>(lds_all + sel * STAGE, load_invariant(wsrow, (size_t)kb), wn, wm, l16, g,
                      acc);
    prefill_stage<WN>(f, tid, lds_all + (sel ^ 1) * STAGE);
    lds_barrier();
  }

  // output: lane holds rows n = n0 + 64 wn + 16 t + 4 g .. +3 of column m
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = m0 + 64 * wm + 16 * j + l16;
    if (m < p.m) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int n = n0 + 64 * wn + 16 * t + 4 * g;
        if (p.out == OUT_PARTIAL) {
          *reinterpret_cast<float4*>(p.part + ((size_t)blockIdx.z * p.m + m) * (size_t)p.n + n) =
              make_float4(acc[t][j][0], acc[t][j][1], acc[t][j][2], acc[t][j][3]);
        } else {
          *reinterpret_cast<uint2*>(p.y + (size_t)m * (size_t)p.n + n) =
              make_uint2(pack_bf16x2(acc[t][j][0], acc[t][j][1]),
                         pack_bf16x2(acc[t][j][2], acc[t][j][3]));
        }
      }
    }
  }
}

}  // namespace fp8bs
