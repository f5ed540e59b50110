// Row-range decode kernel whose weight stream runs through LDS (tile-layout
// weights, m <= 16).
//
// The work split is the row-range kernel's: one workgroup per compute unit
// owns a contiguous range of output columns (a multiple of 4) over the
// whole K range; 8 compute waves take the K blocks of each 16-row tile in
// turn (wave w: blocks w, w + 8, ...) and their fp32 partials are summed in
// wave order. The difference is how the weight tiles arrive. Four more
// waves (one per SIMD) only issue direct loads (global_load_lds_dwordx4,
// non-temporal: 16 bytes per lane, 1 KB per instruction, written to LDS at
// the address in M0) into a ring of S stages; a step is the 8 K blocks the
// compute waves take together, 16 contiguous KB of one tile in the tile
// layout. The loads start at the kernel's first instruction, so the weight
// stream runs while the compute waves cast the activations, and no compute
// wave ever waits at the issue of a load (a wave with a full memory queue
// stalls there, and its arithmetic with it). One workgroup barrier per step
// publishes the next step's stage and frees the one just read; at the end of
// each tile the partials cross through LDS at the same barrier and wave 0
// adds them and writes the outputs.
//
// The workgroup works through the 16-row tiles of the tile layout that
// overlap its range. Where a range starts or ends inside a tile, the loader
// lanes of rows outside it read the nearest row inside it instead (each
// lane gives its own address; those lanes' bytes lie on the same lines as
// rows of the range, so they cost no extra memory traffic), and only rows
// inside the range are written.
//
// The products, their per-block rescale and both summation orders are those
// of the row-range kernel with 8 waves along K, so the outputs are the same
// bits.
#pragma once

#include "fp8bs_gemm.h"

namespace fp8bs {

constexpr int RD_WK = 8;          // compute waves (waves along K)
constexpr int RD_LOADERS = 4;     // loader waves, one per SIMD
constexpr int RD_STEP = 16384;    // LDS bytes of a step: RD_WK blocks of 2 KB
constexpr int RD_PER_STEP = 4;    // loads per loader wave and step

// LDS layout: the range's weight scales, the staged activations, two
// partial-exchange areas (RD_WK - 1 partials of 1 KB each), the ring.
__host__ __device__ inline int rd_act_off(int rows, int nblk) {
  return lds_wscale_bytes(rows, nblk);
}
__host__ __device__ inline int rd_red_off(int rows, int nblk, int m) {
  return rd_act_off(rows, nblk) + lds_act_bytes(nblk, m);
}
__host__ __device__ inline int rd_ring_off(int rows, int nblk, int m) {
  return rd_red_off(rows, nblk, m) + 2 * (RD_WK - 1) * 64 * 16;
}
__host__ __device__ inline int rd_lds_bytes(int rows, int nblk, int m, int stages) {
  return rd_ring_off(rows, nblk, m) + stages * RD_STEP;
}

__device__ __forceinline__ void rd_dma16(uint32_t m0, const void* base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
               :
               : "s"(m0), "v"(voff), "s"(base)
               : "memory", "m0");
}

template <int S, bool FUSED, int CR>
__device__ __forceinline__ void gemm_rows_dma_body(const GemmParams& p, uint8_t* lds_all) {
  static_assert(S >= 2 && (S - 1) * RD_PER_STEP <= 63, "vmcnt range");
  constexpr int NT = 64 * RD_WK;  // compute threads (they stage the activations)
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int M = p.m;
  const int nblk = p.kbn;
  const int r0 = blockIdx.x * p.rows_per_wg;  // a multiple of 4
  const int r1 = r0 + p.rows_per_wg < p.n ? r0 + p.rows_per_wg : p.n;
  const int tb = r0 >> 4;                     // first tile overlapping the range
  const int ntile = ((r1 - 1) >> 4) - tb + 1;
  const int spt = (nblk + RD_WK - 1) / RD_WK;  // steps per tile
  const int nsteps = ntile * spt;
  const int nbf = r0 / BLK, nbr = (r1 - 1) / BLK - nbf + 1;
  float* wsl = reinterpret_cast<float*>(lds_all);
  uint8_t* act = lds_all + rd_act_off(p.rows_per_wg, nblk);
  float* act_s = reinterpret_cast<float*>(act + nblk * M * ACT_STRIDE);
  f32x4* red = reinterpret_cast<f32x4*>(lds_all + rd_red_off(p.rows_per_wg, nblk, M));
  uint8_t* ring = lds_all + rd_ring_off(p.rows_per_wg, nblk, M);

  if (wave >= RD_WK) {
    // Loader wave l: slots 2l and 2l + 1 (compute waves' blocks) of every
    // step, both 1 KB halves. Steps past the last reload the last step's
    // bytes into the stage they would use (freed, and never read again), so
    // every step issues the same number of loads and one wait count holds.
    // Lane 16 q + r holds row r of the tile (quarter q); a row outside the
    // range is replaced by the range's nearest row of the same tile.
    const int l = wave - RD_WK;
    const uint32_t ring0 = (uint32_t)reinterpret_cast<uintptr_t>(ring);
    const uint8_t* tiles = p.wq + (size_t)tb * (size_t)p.kbn * 2048u;
    auto issue = [&](int i) {
      const uint32_t st = ring0 + (uint32_t)((i % S) * RD_STEP);
      const int ic = i < nsteps ? i : nsteps - 1;
      const int t = ic / spt, g = ic - t * spt;
      int r = 16 * (tb + t) + (lane & 15);
      r = r < r0 ? r0 : (r >= r1 ? r1 - 1 : r);
      const uint32_t lo = (uint32_t)((lane & 48) + (r & 15)) * 16u;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int w = 2 * l + s2;
        int kb = RD_WK * g + w;
        kb = kb < nblk ? kb : nblk - 1;
        const uint8_t* src = tiles + ((size_t)t * (size_t)p.kbn + (size_t)kb) * 2048u;
        rd_dma16(st + (uint32_t)w * 2048u, src, lo);
        rd_dma16(st + (uint32_t)w * 2048u + 1024u, src + 1024, lo);
      }
    };
    for (int i = 0; i < S - 1; ++i) issue(i);
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"((S - 2) * RD_PER_STEP) : "memory");
    lds_barrier();  // step 0 and the activations are in LDS
    for (int i = 0; i < nsteps; ++i) {
      issue(i + S - 1);  // into the stage of step i - 1, freed by the last barrier
      asm volatile("s_waitcnt vmcnt(%0)" : : "n"((S - 2) * RD_PER_STEP) : "memory");
      lds_barrier();  // step i + 1 published, step i free
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    return;
  }

  // compute waves: weight scales of the range and activations into LDS
  const int w = wave;
  stage_act_tail<NT, CR, FUSED>(p, 0, nblk, tid, act, act_s);
  ScaleFetch sf;
  load_wscales<NT>(p, nbf, nbr, 0, nblk, tid, sf);
  uint4 xr[CR][4];
  if constexpr (FUSED) load_act_quarters<NT, CR>(p, 0, nblk * M * 4, tid, 0, xr);
  stage_act<NT, CR, FUSED>(p, 0, nblk, tid, xr, act, act_s);
  store_wscales<NT>(p, nbf, nbr, 0, nblk, tid, sf, wsl);
  lds_barrier();

  const int l16 = lane & 15, g16 = lane >> 4;
  const bool row_ok = l16 < M;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < nsteps; ++i) {
    const int t = i / spt, g = i - t * spt;
    const int kb = RD_WK * g + w;
    if (kb < nblk) {
      const uint8_t* slot = ring + (i % S) * RD_STEP + w * 2048 + lane * 16;
      const uint4 lo = *reinterpret_cast<const uint4*>(slot);
      const uint4 hi = *reinterpret_cast<const uint4*>(slot + 1024);
      const i32x8 aop = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                         (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      i32x8 bop = {0, 0, 0, 0, 0, 0, 0, 0};
      float sa = 0.0f;
      if (row_ok) {
        const uint8_t* a = act + (kb * M + l16) * ACT_STRIDE + 32 * g16;
        const uint4 alo = *reinterpret_cast<const uint4*>(a);
        const uint4 ahi = *reinterpret_cast<const uint4*>(a + 16);
        bop = i32x8{(int)alo.x, (int)alo.y, (int)alo.z, (int)alo.w,
                    (int)ahi.x, (int)ahi.y, (int)ahi.z, (int)ahi.w};
        sa = act_s[kb * M + l16];
      }
      // this lane's four output rows lie in one 128-row scale block; lanes
      // outside the range read a valid entry
      int nbl = (16 * (tb + t) + 4 * g16) / BLK - nbf;
      nbl = nbl < 0 ? 0 : (nbl < nbr ? nbl : nbr - 1);
      const float sw = wsl[nbl * nblk + kb];
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      const f32x4 pb = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop, bop, z, 0, 0, 0, 0, 0, 0);
      const float sc = sa * sw;
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = __builtin_fmaf(pb[q], sc, acc[q]);
    }
    const bool tile_end = g == spt - 1;
    f32x4* rt = red + (t & 1) * (RD_WK - 1) * 64;
    if (tile_end && w > 0) rt[(w - 1) * 64 + lane] = acc;
    lds_barrier();  // (with the loaders) this step's stage is free; the partials are visible
    if (tile_end) {
      if (w == 0) {
        for (int ww = 1; ww < RD_WK; ++ww) acc += rt[(ww - 1) * 64 + lane];
        // this lane's four rows (r0 and r1 are multiples of 4: all in or out)
        const int rg = 16 * (tb + t) + 4 * g16;
        if (row_ok && rg >= r0 && rg < r1) {
          uint2* dst = reinterpret_cast<uint2*>(p.y + (size_t)l16 * (size_t)p.n + rg);
          *dst = make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
        }
      }
      acc = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
}

// rd_lds_bytes(rows_per_wg, k / 128, m, S) of dynamic LDS; 768 threads (8
// compute and 4 loader waves); grid: one workgroup per row range.
template <int S, bool FUSED>
__global__ __launch_bounds__(64 * (RD_WK + RD_LOADERS), 1) void gemm_rows_dma_kernel(GemmParams p) {
  constexpr int NT = 64 * RD_WK;
  extern __shared__ __align__(16) uint8_t lds_all[];
  if constexpr (FUSED) {
    const int rounds = act_rounds(p.kbn * p.m * 4, NT);
    if (rounds == 1)
      gemm_rows_dma_body<S, true, 1>(p, lds_all);
    else if (rounds == 2)
      gemm_rows_dma_body<S, true, 2>(p, lds_all);
    else
      gemm_rows_dma_body<S, true, 3>(p, lds_all);
  } else {
    gemm_rows_dma_body<S, false, 1>(p, lds_all);
  }
}

}  // namespace fp8bs
