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
//   with 16-byte loads that cover whole 128-byte lines, several K blocks in
//   flight per wave. waves_k waves share a row range and interleave its K
//   blocks; their fp32 partials are summed in LDS in wave order. With
//   split_k > 1 each workgroup writes an fp32 partial tile; the partials of a
//   row group are summed over s in order, either by a second kernel or, in
//   the same launch, by the workgroup of the row group that finishes last.
#pragma once

#include <type_traits>

#include "fp8bs_device.h"

namespace fp8bs {

// Output handling of a kernel instance.
// OUT_SWIGLU: as OUT_DIRECT, and the workgroup finishing the last columns of
// a 128-column block of the SwiGLU output runs the MLP epilogue for it.
enum { OUT_DIRECT = 0, OUT_PARTIAL = 1, OUT_LAST_ARRIVER = 2, OUT_SWIGLU = 3 };

struct GemmParams {
  const uint16_t* x;    // bf16 [m][k] (fused cast) or nullptr
  const uint8_t* xq;    // E4M3 [m][k] (pre-quantized) or nullptr
  const float* xs;      // fp32 [m][k/128] (pre-quantized)
  const uint8_t* wq;    // E4M3 [n][k]
  const float* ws;      // fp32 [n/128][k/128]
  uint16_t* y;          // bf16 [m][n]
  float* part;          // fp32 [split][m][n] when split > 1
  uint64_t* counters;   // arrival counters: [row groups] (last-arriver reduce) or
                        // [n/256] (SwiGLU epilogue)
  uint64_t epoch;       // nonzero tag of this launch (last-arriver reduce)
  int m, n, k, kbn;     // kbn = k / 128
  int split;
  int out;              // OUT_DIRECT, OUT_PARTIAL or OUT_LAST_ARRIVER
  int rows_per_wg;      // row-range kernel: output columns per workgroup (multiple of 4)
  uint8_t* hq;          // SwiGLU epilogue: E4M3 codes [m][n/2]
  float* hs;            // SwiGLU epilogue: fp32 scales [m][n/256]
  int sk_whole;         // stream-K kernel: whole-cell partition
  int pf_full, pf_1d;   // wide prefill kernel: whole tiles of the 1-D schedule, schedule
};

// LDS layout of a workgroup:
//   act   [nblk][m][ACT_STRIDE] E4M3 codes of the staged activations
//   act_s [nblk][m] fp32 scales
//   red   partial-sum exchange area for waves_k > 1
__host__ __device__ inline int lds_act_bytes(int nblk, int m) {
  return ((nblk * m * (ACT_STRIDE + 4)) + 15) & ~15;
}

// K blocks [kb0, kb1) of split s (balanced: sizes differ by at most one).
__device__ __forceinline__ void split_range(int s, int split, int kbn, int& kb0, int& kb1) {
  kb0 = (int)((int64_t)s * kbn / split);
  kb1 = (int)((int64_t)(s + 1) * kbn / split);
}

// ------------------------------------------------- weight-scale staging ---

// The weight scales a workgroup needs are staged in LDS once, at the start,
// instead of being read with a dependent scalar load per K block: block rows
// nbf .. nbf + nbr - 1 (clamped to the matrix), K blocks kb0 .. kb0 + nblk - 1,
// as wsl[(nb - nbf) * nblk + (kb - kb0)]. The area sits at the start of the
// workgroup's LDS; its size covers any range of `rows` output columns.
__host__ __device__ inline int lds_wscale_bytes(int rows, int nblk) {
  return ((rows / BLK + 2) * nblk * 4 + 15) & ~15;
}

constexpr int SCALE_REGS = 4;  // scales fetched into registers per thread

struct ScaleFetch {
  float v[SCALE_REGS];
};

// Issue the scale loads (the first SCALE_REGS * NT of them into registers,
// so they are in flight together with the other prologue loads).
// (Unconditional loads with clamped indices, as for the activations.)
template <int NT>
__device__ __forceinline__ void load_wscales(const GemmParams& p, int nbf, int nbr, int kb0,
                                             int nblk, int tid, ScaleFetch& f) {
  const int total = nbr * nblk;
  const int nbn = p.n / BLK;
#pragma unroll
  for (int i = 0; i < SCALE_REGS; ++i) {
    int e = tid + i * NT;
    e = e < total ? e : total - 1;
    const int r = e / nblk, kb = e - r * nblk;
    const int nb = nbf + r < nbn ? nbf + r : nbn - 1;
    f.v[i] = p.ws[(size_t)nb * (size_t)p.kbn + kb0 + kb];
  }
}

// Store the fetched scales to LDS (and fetch any beyond SCALE_REGS * NT
// directly). The caller's next barrier makes them visible.
template <int NT>
__device__ __forceinline__ void store_wscales(const GemmParams& p, int nbf, int nbr, int kb0,
                                              int nblk, int tid, const ScaleFetch& f, float* wsl) {
  const int total = nbr * nblk;
#pragma unroll
  for (int i = 0; i < SCALE_REGS; ++i) {
    const int e = tid + i * NT;
    if (e < total) wsl[e] = f.v[i];
  }
  const int nbn = p.n / BLK;
  for (int e = tid + SCALE_REGS * NT; e < total; e += NT) {
    const int r = e / nblk, kb = e - r * nblk;
    const int nb = nbf + r < nbn ? nbf + r : nbn - 1;
    wsl[e] = p.ws[(size_t)nb * (size_t)p.kbn + kb0 + kb];
  }
}

// ---------------------------------------------------- activation staging ---

// Quarter-block g of the workgroup's activation range: block bm = g / 4
// (bm = kbl * m + row), columns 32 * (g % 4) .. +31 of that block. Indices
// past G load the last quarter again (unused): the loads are unconditional,
// so the compiler's wait counts for them stay exact and later loads (the
// weight prefetch) are never held back behind them. Kernels that serve
// very different activation sizes pick CR per launch (see the grid kernels)
// so that few of these loads are redundant.
template <int NT, int CR>
__device__ __forceinline__ void load_act_quarters(const GemmParams& p, int kb0, int G, int tid,
                                                  int base, uint4 (&xr)[CR][4]) {
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
__device__ __forceinline__ void cast_act_quarters(int G, int tid, int base,
                                                  const uint4 (&xr)[CR][4], uint8_t* act,
                                                  float* act_s) {
#pragma unroll
  for (int i = 0; i < CR; ++i) {
    const int g = base + tid + i * NT;
    if (g < G) {  // G is a multiple of 4: the four lanes of a quad agree
      const int qq = g & 3, bm = g >> 2;
      uint32_t codes[8];
      const float s = cast_quarter(xr[i], codes);
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

// Cast the activation quarters beyond the first CR * NT (needed only when a
// workgroup's K range holds more than CR * NT quarter blocks). Runs before
// the weight prefetch is issued, so its waits cover activation loads only.
template <int NT, int CR, bool FUSED>
__device__ __forceinline__ void stage_act_tail(const GemmParams& p, int kb0, int nblk, int tid,
                                               uint8_t* act, float* act_s) {
  if constexpr (FUSED) {
    const int G = nblk * p.m * 4;
    for (int base = CR * NT; base < G; base += CR * NT) {
      uint4 xr2[CR][4];
      load_act_quarters<NT, CR>(p, kb0, G, tid, base, xr2);
      cast_act_quarters<NT, CR>(G, tid, base, xr2, act, act_s);
    }
  }
}

// Cast the first CR * NT activation quarters (loaded into xr before the
// weight prefetch), or copy pre-quantized codes and scales into LDS.
template <int NT, int CR, bool FUSED>
__device__ __forceinline__ void stage_act(const GemmParams& p, int kb0, int nblk, int tid,
                                          const uint4 (&xr)[CR][4], uint8_t* act, float* act_s) {
  if constexpr (FUSED) {
    cast_act_quarters<NT, CR>(nblk * p.m * 4, tid, 0, xr, act, act_s);
  } else {
    copy_act<NT>(p, kb0, nblk, tid, act, act_s);
  }
}

// ------------------------------------------------------ split-K epilogue ---

// Cross-workgroup handoff in one launch (last-arriver reduce, SwiGLU
// epilogue). Workgroups on different XCDs do not share an L2, so the data
// one workgroup hands to another are written and read only with
// device-scope atomic accesses: the stores write through this XCD's L2 and
// the loads are not served from stale lines of the reader's caches. Each
// thread waits until its own stores are performed (vmcnt counts stores on
// this architecture), a barrier orders the whole workgroup's stores before
// the arrival, and the arrival is a device-scope read-modify-write on an
// integer counter. The arrival that completes the count reads the data after
// it. The protocol needs no cache-wide write-back or invalidate (those cost
// far more than the handoff itself when every workgroup arrives).
//
// Counter: 64 bits, (launch epoch << 8) | arrivals. An arrival that finds
// another epoch (a previous launch, or whatever the memory held) starts this
// launch's count at 1; the arrival that brings the count to `expected` is the
// last one, and clears the counter. The epoch is unique per host-side launch
// call, so the counters never need initialization; a replayed graph reuses
// its epoch, which the clearing makes safe.

__device__ __forceinline__ void store_coherent64(void* dst, uint64_t v) {
  __hip_atomic_store(reinterpret_cast<uint64_t*>(dst), v, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t load_coherent64(const void* src) {
  return __hip_atomic_load(reinterpret_cast<const uint64_t*>(src), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// One arrival (any single thread). Returns whether it completed the count.
__device__ __forceinline__ bool arrive(uint64_t* c, uint64_t epoch, uint64_t expected) {
  uint64_t old = __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  uint64_t nv;
  for (;;) {
    nv = ((old >> 8) == epoch) ? old + 1 : ((epoch << 8) | 1u);
    if (__hip_atomic_compare_exchange_strong(c, &old, nv, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT))
      break;
  }
  const bool last = (nv & 0xFFu) == expected;
  if (last) __hip_atomic_store(c, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return last;
}

// Every thread: wait for this thread's coherent stores, then meet the others.
__device__ __forceinline__ void stores_performed_barrier() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

// Store an fp32 partial of 4 consecutive outputs: plain when a second kernel
// sums the partials, coherent for the last-arriver reduce.
__device__ __forceinline__ void store_partial4(const GemmParams& p, float* dst, float a, float b,
                                               float c, float d) {
  if (p.out == OUT_LAST_ARRIVER) {
    store_coherent64(dst, (uint64_t)__float_as_uint(a) | ((uint64_t)__float_as_uint(b) << 32));
    store_coherent64(dst + 2, (uint64_t)__float_as_uint(c) | ((uint64_t)__float_as_uint(d) << 32));
  } else {
    *reinterpret_cast<float4*>(dst) = make_float4(a, b, c, d);
  }
}

// Called by every thread of a workgroup after it stored its fp32 partial
// tile part[s][m][n0 .. n0+ROWS). The last of the split workgroups of a row
// group (one counter per row group) sums the split partials in order
// s = 0, 1, ..., split-1 and writes the bf16 outputs.
template <int NT, int ROWS>
__device__ __forceinline__ void last_arriver_reduce(const GemmParams& p, int n0, int tid) {
  __shared__ int s_last;
  stores_performed_barrier();
  if (tid == 0) s_last = arrive(p.counters + blockIdx.x, p.epoch, (uint64_t)p.split);
  __syncthreads();
  if (!s_last) return;
  const int M = p.m;
  const size_t mn = (size_t)M * (size_t)p.n;
  for (int i = tid; i < M * (ROWS / 4); i += NT) {
    const int m = i / (ROWS / 4), r4 = i - m * (ROWS / 4);
    const size_t off = (size_t)m * (size_t)p.n + n0 + 4 * r4;
    float a[4];
    for (int s = 0; s < p.split; ++s) {
      const uint64_t lo = load_coherent64(p.part + (size_t)s * mn + off);
      const uint64_t hi = load_coherent64(p.part + (size_t)s * mn + off + 2);
      const float v[4] = {__uint_as_float((uint32_t)lo), __uint_as_float((uint32_t)(lo >> 32)),
                          __uint_as_float((uint32_t)hi), __uint_as_float((uint32_t)(hi >> 32))};
#pragma unroll
      for (int q = 0; q < 4; ++q) a[q] = s == 0 ? v[q] : a[q] + v[q];
    }
    *reinterpret_cast<uint2*>(p.y + off) =
        make_uint2(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]));
  }
}

// ------------------------------------------------- SwiGLU epilogue ---

// The MLP up/gate projection with SwiGLU and the 1x128 FP8 cast of its
// result fused in ("Kernel-Level Optimisations for LLM Inference and
// Training", section "Scheduling decides the shapes your kernels see", on
// fusing element-wise steps into the matmul). Output columns [0, I) are the
// gate, [I, 2I) the up projection (I = n/2). A 128-column block b of h needs
// gate columns 128b.. and up columns I+128b.., which other workgroups may
// produce. Every workgroup stores its bf16 outputs coherently and arrives on
// the counter of each block b it produced columns of, once per side, all
// arrivals at the same time (one lane each); the workgroup whose arrival
// completes a block's count runs the epilogue for that block from the stored
// bf16 outputs (swiglu_cast_wave, the function the standalone epilogue
// runs). The result therefore depends only on the bf16 outputs, never on
// which workgroup arrives last.

constexpr int SWIGLU_MAX_ARRIVALS = 64;  // (side, block) pairs of one workgroup

// Store 4 consecutive bf16 outputs (8 bytes): coherent when another
// workgroup reads them in the same launch.
__device__ __forceinline__ void store_y4(const GemmParams& p, uint16_t* dst, float a, float b,
                                         float c, float d) {
  const uint32_t lo = pack_bf16x2(a, b), hi = pack_bf16x2(c, d);
  if (p.out == OUT_SWIGLU)
    store_coherent64(dst, (uint64_t)lo | ((uint64_t)hi << 32));
  else
    *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
}

// Row-range kernels with the SwiGLU epilogue (instantiated with SW = true)
// keep their bf16 outputs in LDS
// ([m][rows_per_wg], after the kernel's own areas) until the last tile and
// then write them all at once: a device-coherent store is slow to complete,
// and since stores and the weight loads share one in-order wait counter, a
// store issued after every tile would hold up the weight stream.
__host__ __device__ inline int lds_ystage_bytes(int m, int rows) { return (m * rows * 2 + 15) & ~15; }

__device__ __forceinline__ void stage_y4(uint16_t* ystage, int rows, int m, int rl, float a,
                                         float b, float c, float d) {
  *reinterpret_cast<uint2*>(ystage + (size_t)m * rows + rl) =
      make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
}

// Every thread: copy the staged outputs of rows [r0, r0 + nrows) to y with
// coherent stores (after a barrier that makes the staging visible).
template <int NT>
__device__ __forceinline__ void flush_ystage(const GemmParams& p, const uint16_t* ystage, int r0,
                                             int nrows, int tid) {
  __syncthreads();
  const int rows = p.rows_per_wg, q4 = rows / 4;
  for (int i = tid; i < p.m * q4; i += NT) {
    const int m = i / q4, rl = 4 * (i - m * q4);
    if (rl < nrows) {
      const uint2 v = *reinterpret_cast<const uint2*>(ystage + (size_t)m * rows + rl);
      store_coherent64(p.y + (size_t)m * (size_t)p.n + r0 + rl,
                       (uint64_t)v.x | ((uint64_t)v.y << 32));
    }
  }
}

// Workgroups (consecutive ranges of R output columns, nwg of them) holding a
// column of [lo, lo + 128).
__device__ __forceinline__ int wgs_touching(int lo, int R, int nwg) {
  const int a = lo / R;
  int b = (lo + BLK - 1) / R;
  b = b < nwg - 1 ? b : nwg - 1;
  return b - a + 1;
}

// Called by every thread of a workgroup after its last output store. The
// workgroup produced output columns [r0, r1); workgroups own consecutive
// ranges of R columns, nwg of them.
template <int NT>
__device__ __forceinline__ void swiglu_arrive(const GemmParams& p, int r0, int r1, int R,
                                              int nwg, int tid) {
  __shared__ int s_done[SWIGLU_MAX_ARRIVALS];
  __shared__ int s_ndone;
  const int inter = p.n >> 1;
  // gate blocks [g0, g1] and up blocks [u0, u1] this workgroup produced columns of
  int g0 = 0, g1 = -1, u0 = 0, u1 = -1;
  if (r0 < inter) {
    g0 = r0 / BLK;
    g1 = ((r1 < inter ? r1 : inter) - 1) / BLK;
  }
  if (r1 > inter) {
    u0 = ((r0 > inter ? r0 : inter) - inter) / BLK;
    u1 = (r1 - 1 - inter) / BLK;
  }
  const int ng = g1 - g0 + 1, na = ng + (u1 - u0 + 1);  // na <= SWIGLU_MAX_ARRIVALS (host check)
  if (tid == 0) s_ndone = 0;
  stores_performed_barrier();
  if (tid < na) {
    const int b = tid < ng ? g0 + tid : u0 + (tid - ng);
    const uint64_t expected =
        (uint64_t)(wgs_touching(b * BLK, R, nwg) + wgs_touching(inter + b * BLK, R, nwg));
    if (arrive(p.counters + b, p.epoch, expected)) s_done[atomicAdd(&s_ndone, 1)] = b;
  }
  __syncthreads();
  const int nd = s_ndone;
  // the epilogue of every completed block: one wave per (block, row) task
  const int wave = tid >> 6, l = tid & 63;
  for (int t = wave; t < nd * p.m; t += NT / 64) {
    const int b = s_done[t / p.m], m = t - (t / p.m) * p.m;
    const uint16_t* gp = p.y + (size_t)m * (size_t)p.n + b * BLK + 2 * l;
    const uint32_t gw = __hip_atomic_load(reinterpret_cast<const uint32_t*>(gp),
                                          __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t uw = __hip_atomic_load(reinterpret_cast<const uint32_t*>(gp + inter),
                                          __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    swiglu_cast_wave(gw, uw, l, p.hq + (size_t)m * (size_t)inter + b * BLK,
                     p.hs + (size_t)m * (size_t)(inter / BLK) + b);
  }
}

// ====================================================================
// MFMA path: v_mfma_f32_16x16x128_f8f6f4, A = 16 weight rows x 128 K,
// B = 128 K x 16 activation rows (zero beyond m). Lane l holds A row l%16
// and B column l%16: the 32 K positions 32*(l/16) .. +31 of the block, in
// order (the same K positions in A and B, so the product is the block's
// dot product). The result D[n][m] sits in lane l as rows 4*(l/16) + i,
// column l%16.
//
// Weight loads cover whole 128-byte rows: load P takes rows 0-7 of the
// tile, load Q rows 8-15; lane l reads 16 bytes of row (l&7) (P) or
// 8+(l&7) (Q). A per-lane select and a rotate by 8 lanes within each row of
// 16 lanes then give every lane the two 16-byte pieces of its own row.
// ====================================================================

struct TileLoad {
  uint4 p, q;
};

__device__ __forceinline__ i32x8 tile_operand(const TileLoad& t, bool lo8) {
  const uint32_t pp[4] = {t.p.x, t.p.y, t.p.z, t.p.w};
  const uint32_t qq[4] = {t.q.x, t.q.y, t.q.z, t.q.w};
  i32x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t xv = lo8 ? pp[i] : qq[i];
    const uint32_t zv = lo8 ? qq[i] : pp[i];
    r[i] = (int)xv;
    r[4 + i] = __builtin_amdgcn_mov_dpp((int)zv, DPP_ROW_ROR8, 0xF, 0xF, false);
  }
  return r;
}

// Tile layout of the weight codes (written by fp8bs_pack_weight): the codes
// of 16 rows x 128 columns (one MFMA A operand per K block) are 2 KB of
// consecutive bytes, tile (R/16, kb) at byte ((R/16) * kbn + kb) * 2048.
// Inside a tile, half h (columns 16h .. 16h+15 of each 32-column quarter)
// fills the h-th KB, and lane 16g + R%16 of a wave (row R%16, quarter g,
// the operand's lane order) owns the 16 bytes at (16g + R%16) * 16 of it.
// One 16-byte load per lane and half then reads each half of an operand as
// one contiguous KB, and the loaded registers are the operand as they are.
// Returns the offset of W[R][128kb + 32g .. +15] (half 0; half 1 is +1024).
__device__ __forceinline__ size_t tile_layout_off(int R, int kb, int kbn, int g) {
  return ((size_t)(R >> 4) * (size_t)kbn + (size_t)kb) * 2048u +
         (size_t)((16 * g + (R & 15)) * 16);
}

// The MFMA A operand of a loaded weight tile in either layout.
template <bool PK>
__device__ __forceinline__ i32x8 weight_operand(const TileLoad& t, bool lo8) {
  if constexpr (PK) {
    return i32x8{(int)t.p.x, (int)t.p.y, (int)t.p.z, (int)t.p.w,
                 (int)t.q.x, (int)t.q.y, (int)t.q.z, (int)t.q.w};
  } else {
    return tile_operand(t, lo8);
  }
}

// Body of the grid kernel for CR activation-load rounds per thread.
template <int MT, int TN, int WN, int WK, int D, bool FUSED, int CR, bool PK>
__device__ __forceinline__ void gemm_mfma_body(const GemmParams& p, uint8_t* lds_all) {
  constexpr int NT = 64 * WN * WK;
  constexpr int ROWS = 16 * TN * WN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave % WN, wk = wave / WN;
  const int s = blockIdx.y;
  int kb0, kb1;
  split_range(s, p.split, p.kbn, kb0, kb1);
  const int nblk = kb1 - kb0;
  const int M = p.m;

  const int n0 = blockIdx.x * ROWS;
  const int row0 = n0 + wn * 16 * TN;
  uint8_t* lds = lds_all;
  uint8_t* act = lds;
  float* act_s = reinterpret_cast<float*>(lds + nblk * M * ACT_STRIDE);
  f32x4* red = reinterpret_cast<f32x4*>(lds + lds_act_bytes(nblk, M));
  const int l16 = lane & 15, g16 = lane >> 4;
  const int l7 = lane & 7, hb = (lane >> 3) & 1;
  const bool lo8 = hb == 0;
  // row-major: load P takes rows 0-7 of a tile, load Q rows 8-15 (see above);
  // tile layout: lane l loads both halves of its own operand row l%16
  const uint8_t* wp = PK ? p.wq + tile_layout_off(row0 + l16, 0, p.kbn, g16)
                         : p.wq + (size_t)(row0 + l7) * (size_t)p.k + 16 * (2 * g16 + hb);
  const uint8_t* wqp =
      PK ? wp + 1024 : p.wq + (size_t)(row0 + 8 + l7) * (size_t)p.k + 16 * (2 * g16 + 1 - hb);
  const int nj = nblk > wk ? (nblk - wk + WK - 1) / WK : 0;  // this wave's K blocks

  // 1. activation bf16 loads first (so waiting for them does not wait on weights)
  //    The tail (a loop with its own waits) runs before any other load is
  //    issued, so the compiler's wait counts for the straight-line loads
  //    below are exact.
  stage_act_tail<NT, CR, FUSED>(p, kb0, nblk, tid, act, act_s);
  uint4 xr[CR][4];
  if constexpr (FUSED) load_act_quarters<NT, CR>(p, kb0, nblk * M * 4, tid, 0, xr);
  __builtin_amdgcn_sched_barrier(0);  // activation loads stay ahead of the weight loads

  // 2. weight prefetch: D blocks per wave in flight
  TileLoad wb[D][TN];
  auto load_block = [&](int d, int j) {
    const int jc = j < nj ? j : (nj > 0 ? nj - 1 : 0);
    int kb = kb0 + wk + jc * WK;
    kb = kb < p.kbn ? kb : p.kbn - 1;
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      const size_t off = PK ? ((size_t)t * (size_t)p.kbn + (size_t)kb) * 2048u
                            : (size_t)t * 16 * (size_t)p.k + (size_t)kb * BLK;
      wb[d][t].p = load_stream16(wp + off);
      wb[d][t].q = load_stream16(wqp + off);
    }
  };
  // At most two blocks are issued before the cast (see gemm_rows_kernel).
  constexpr int PRE = D < 2 ? D : 2;
#pragma unroll
  for (int d = 0; d < PRE; ++d) load_block(d, d);

  // 3. stage activations and weight scales in LDS
  stage_act<NT, CR, FUSED>(p, kb0, nblk, tid, xr, act, act_s);
#pragma unroll
  for (int d = PRE; d < D; ++d) load_block(d, d);
  lds_barrier();

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
        const uint8_t* a = act + (kbl * M + m) * ACT_STRIDE + 32 * g16;
        const uint4 lo = *reinterpret_cast<const uint4*>(a);
        const uint4 hi = *reinterpret_cast<const uint4*>(a + 16);
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
      const float sw = load_invariant(p.ws, (size_t)nb * (size_t)p.kbn + kb);
      const i32x8 aop = weight_operand<PK>(wb[d][t], lo8);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        const f32x4 pb =
            __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop, bop[mt], z, 0, 0, 0, 0, 0, 0);
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
          if (p.out == OUT_DIRECT || p.out == OUT_SWIGLU) {
            store_y4(p, p.y + (size_t)m * (size_t)p.n + n, acc[t][mt][0], acc[t][mt][1],
                     acc[t][mt][2], acc[t][mt][3]);
          } else {
            store_partial4(p, p.part + ((size_t)s * M + m) * (size_t)p.n + n, acc[t][mt][0],
                           acc[t][mt][1], acc[t][mt][2], acc[t][mt][3]);
          }
        }
      }
  }
  if (p.out == OUT_LAST_ARRIVER) last_arriver_reduce<NT, ROWS>(p, n0, tid);
  if (p.out == OUT_SWIGLU) swiglu_arrive<NT>(p, n0, n0 + ROWS, ROWS, gridDim.x, tid);
}

// Rounds of activation loads a workgroup needs for its G quarter blocks
// (1 .. 3; beyond 3 * NT the rest is cast in a loop first). The choice is
// made once at kernel entry, before any load, so each body is straight-line
// code whose loads are all needed.
__device__ __forceinline__ int act_rounds(int G, int NT) {
  const int r = (G + NT - 1) / NT;
  return r < 1 ? 1 : (r > 3 ? 3 : r);
}

template <int MT, int TN, int WN, int WK, int D, bool FUSED, bool PK = false>
__global__ __launch_bounds__(64 * WN * WK) void gemm_mfma_kernel(GemmParams p) {
  constexpr int NT = 64 * WN * WK;
  extern __shared__ __align__(16) uint8_t lds_all[];
  if constexpr (FUSED) {
    int kb0, kb1;
    split_range(blockIdx.y, p.split, p.kbn, kb0, kb1);
    const int rounds = act_rounds((kb1 - kb0) * p.m * 4, NT);
    if (rounds == 1)
      gemm_mfma_body<MT, TN, WN, WK, D, true, 1, PK>(p, lds_all);
    else if (rounds == 2)
      gemm_mfma_body<MT, TN, WN, WK, D, true, 2, PK>(p, lds_all);
    else
      gemm_mfma_body<MT, TN, WN, WK, D, true, 3, PK>(p, lds_all);
  } else {
    gemm_mfma_body<MT, TN, WN, WK, D, false, 1, PK>(p, lds_all);
  }
}

// ====================================================================
// MFMA row-range kernel: one workgroup per compute unit. Workgroup g owns
// the output columns [g*R, g*R + R) (R = rows_per_wg, the last 16-row tile
// partly masked) over the whole K range, so no partial sums leave the
// workgroup and the activations are cast once per workgroup. Its WK waves
// interleave the K blocks of each 16-row weight tile (wave w takes blocks
// w, w+WK, ...), so at any time the workgroup reads one contiguous stretch of
// weight rows. Each wave streams the sequence (tile, block) with D tiles in
// flight across tile boundaries; at the end of a tile the waves' partial
// sums are added in wave order through LDS (two alternating LDS areas, one
// barrier per tile) and wave 0 writes the tile's outputs.
// ====================================================================

// OUTK selects the output: ROWS_OUT_BF16 (bf16 y), ROWS_OUT_SWIGLU (bf16 y
// staged in LDS, then the in-GEMM SwiGLU epilogue), ROWS_OUT_PARTIAL (K split
// over grid.y: fp32 partial tiles part[s][m][n], summed by the reduce kernel).
enum { ROWS_OUT_BF16 = 0, ROWS_OUT_SWIGLU = 1, ROWS_OUT_PARTIAL = 2 };

template <int MT, int WK, int D, int PRE, bool FUSED, int OUTK = ROWS_OUT_BF16, bool PK = false>
__global__ __launch_bounds__(64 * WK) void gemm_rows_kernel(GemmParams p) {
  constexpr int NT = 64 * WK;
  constexpr int CR = FUSED ? 3 : 1;
  constexpr bool SW = OUTK == ROWS_OUT_SWIGLU;
  extern __shared__ __align__(16) uint8_t lds_all[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wk = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int M = p.m;
  // this workgroup's K blocks: [kb0, kb0 + nblk) (all of K unless split)
  int kb0 = 0, kb1 = p.kbn;
  if constexpr (OUTK == ROWS_OUT_PARTIAL) split_range(blockIdx.y, p.split, p.kbn, kb0, kb1);
  const int nblk = kb1 - kb0;
  const int r0 = blockIdx.x * p.rows_per_wg;
  const int r1 = r0 + p.rows_per_wg < p.n ? r0 + p.rows_per_wg : p.n;
  const int nrows = r1 - r0;
  const int ntile = (nrows + 15) >> 4;
  const int njw = (nblk + WK - 1) / WK;  // blocks per tile per wave (same for every wave)
  const int nitem = ntile * njw;

  const int nbf = r0 / BLK, nbr = (r1 - 1) / BLK - nbf + 1;
  float* wsl = reinterpret_cast<float*>(lds_all);
  uint8_t* lds = lds_all + lds_wscale_bytes(p.rows_per_wg, nblk);
  uint8_t* act = lds;
  float* act_s = reinterpret_cast<float*>(lds + nblk * M * ACT_STRIDE);
  f32x4* red = reinterpret_cast<f32x4*>(lds + lds_act_bytes(nblk, M));
  uint16_t* ystage = reinterpret_cast<uint16_t*>(lds + lds_act_bytes(nblk, M) +
                                                 2 * (WK - 1) * MT * 64 * 16);

  const int l16 = lane & 15, g16 = lane >> 4;
  const int l7 = lane & 7, hb = (lane >> 3) & 1;
  const bool lo8 = hb == 0;

  // 1. activations beyond the first CR * NT quarters (a loop with its own
  //    waits, before any other load), then the weight-scale loads and the
  //    first CR * NT quarters' loads
  stage_act_tail<NT, CR, FUSED>(p, kb0, nblk, tid, act, act_s);
  ScaleFetch sf;
  load_wscales<NT>(p, nbf, nbr, kb0, nblk, tid, sf);
  uint4 xr[CR][4];
  if constexpr (FUSED) load_act_quarters<NT, CR>(p, kb0, nblk * M * 4, tid, 0, xr);
  __builtin_amdgcn_sched_barrier(0);  // activation loads stay ahead of the weight loads

  // 2. weight prefetch. Item i = (tile i / njw, block wk + (i % njw) * WK of
  //    the range). Rows past the range and blocks past it are clamped to
  //    valid addresses (their products are discarded).
  TileLoad wb[D];
  auto load_item = [&](int d, int i) {
    i = i < nitem ? i : nitem - 1;
    const int t = i / njw, j = i - t * njw;
    int kbl = wk + j * WK;
    kbl = kbl < nblk ? kbl : nblk - 1;
    if constexpr (PK) {
      // the range need not start on a 16-row tile: each lane addresses its row
      int ra = 16 * t + l16;
      ra = ra < nrows ? ra : nrows - 1;
      const uint8_t* a = p.wq + tile_layout_off(r0 + ra, kb0 + kbl, p.kbn, g16);
      wb[d].p = load_stream16(a);
      wb[d].q = load_stream16(a + 1024);
    } else {
      int ra = 16 * t + l7, rb = 16 * t + 8 + l7;
      ra = ra < nrows ? ra : nrows - 1;
      rb = rb < nrows ? rb : nrows - 1;
      const uint8_t* base = p.wq + (size_t)(kb0 + kbl) * BLK;
      wb[d].p = load_stream16(base + (size_t)(r0 + ra) * (size_t)p.k + 16 * (2 * g16 + hb));
      wb[d].q = load_stream16(base + (size_t)(r0 + rb) * (size_t)p.k + 16 * (2 * g16 + 1 - hb));
    }
  };
  // Only PRE items are issued before the cast: a wave stalls at issue once
  // the memory queue is full, and the cast must not wait behind the whole
  // prefetch. The other items are issued one after each cast quarter, so the
  // weight stream keeps flowing while the VALU casts.
#pragma unroll
  for (int d = 0; d < PRE; ++d) load_item(d, d);

  // 3. stage activations in LDS, interleaved with the rest of the prefetch
  if constexpr (FUSED) {
    const int G = nblk * M * 4;
#pragma unroll
    for (int c = 0; c < CR; ++c) {
      cast_act_quarters<NT, 1>(G, tid, c * NT, reinterpret_cast<const uint4(&)[1][4]>(xr[c]),
                               act, act_s);
      if (PRE + c < D) load_item(PRE + c, PRE + c);
    }
#pragma unroll
    for (int d = PRE + CR; d < D; ++d) load_item(d, d);
  } else {
    copy_act<NT>(p, kb0, nblk, tid, act, act_s);
#pragma unroll
    for (int d = PRE; d < D; ++d) load_item(d, d);
  }
  store_wscales<NT>(p, nbf, nbr, kb0, nblk, tid, sf, wsl);
  lds_barrier();

  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int d, int i) {
    const int t = i / njw, j = i - t * njw;
    const int kb = wk + j * WK;
    if (kb < nblk) {
      // A 16-row tile may straddle two 128-row scale blocks (row ranges are
      // multiples of 4, not of 16); each lane's four output rows lie in one.
      // this lane's four output rows lie in one 128-row scale block (row
      // ranges are multiples of 4); lanes past the range read a valid entry
      int nbl = (r0 + 16 * t + 4 * g16) / BLK - nbf;
      nbl = nbl < nbr ? nbl : nbr - 1;
      const float sw = wsl[nbl * nblk + kb];
      const i32x8 aop = weight_operand<PK>(wb[d], lo8);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int m = l16 + 16 * mt;
        i32x8 bop = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
        float sa = 0.0f;
        if (m < M) {
          const uint8_t* a = act + (kb * M + m) * ACT_STRIDE + 32 * g16;
          const uint4 lo = *reinterpret_cast<const uint4*>(a);
          const uint4 hi = *reinterpret_cast<const uint4*>(a + 16);
          bop = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                      (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
          sa = act_s[kb * M + m];
        }
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        const f32x4 pb =
            __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop, bop, z, 0, 0, 0, 0, 0, 0);
        const float sc = sa * sw;
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[mt][q] = __builtin_fmaf(pb[q], sc, acc[mt][q]);
      }
    }
    if (j == njw - 1) {
      // end of tile t: partial sums of waves 1..WK-1 through LDS, summed in wave order
      f32x4* rt = red + (t & 1) * (WK - 1) * MT * 64;
      if (wk > 0) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) rt[((wk - 1) * MT + mt) * 64 + lane] = acc[mt];
      }
      lds_barrier();
      if (wk == 0) {
        for (int w = 1; w < WK; ++w)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) acc[mt] += rt[((w - 1) * MT + mt) * 64 + lane];
        const int rl = 16 * t + 4 * g16;  // first of this lane's four rows
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int m = l16 + 16 * mt;
          if (m < M && rl < nrows) {
            if constexpr (SW) {
              stage_y4(ystage, p.rows_per_wg, m, rl, acc[mt][0], acc[mt][1], acc[mt][2],
                       acc[mt][3]);
            } else if constexpr (OUTK == ROWS_OUT_PARTIAL) {
              *reinterpret_cast<float4*>(p.part + ((size_t)blockIdx.y * M + m) * (size_t)p.n +
                                         r0 + rl) =
                  make_float4(acc[mt][0], acc[mt][1], acc[mt][2], acc[mt][3]);
            } else {
              uint2* dst = reinterpret_cast<uint2*>(p.y + (size_t)m * (size_t)p.n + r0 + rl);
              *dst = make_uint2(pack_bf16x2(acc[mt][0], acc[mt][1]),
                                pack_bf16x2(acc[mt][2], acc[mt][3]));
            }
          }
        }
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };

  const int ngrp = (nitem + D - 1) / D;
  for (int g = 0; g + 1 < ngrp; ++g) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      compute(d, g * D + d);
      load_item(d, (g + 1) * D + d);
    }
  }
#pragma unroll
  for (int d = 0; d < D; ++d) {
    const int i = (ngrp - 1) * D + d;
    if (i < nitem) compute(d, i);
  }
  if constexpr (SW) {
    flush_ystage<NT>(p, ystage, r0, nrows, tid);
    swiglu_arrive<NT>(p, r0, r1, p.rows_per_wg, gridDim.x, tid);
  }
}

// ====================================================================
// Row-range kernel with register-resident activations: the work split of
// gemm_rows_kernel (one workgroup per compute unit, a contiguous range of
// output columns over the whole K range, WK waves taking K blocks
// wk, wk + WK, ...), but each wave keeps the activation operands of its own
// NJ K blocks in VGPRs for the whole launch instead of reading them from
// LDS: NJ * MT * 8 dwords per lane (80 at NJ = 5, m <= 32). The multiply
// loop reads only weight scales and the cross-wave exchange area from LDS,
// and the activations of a long K range never limit m. With m <= 16 (or
// codes given) each wave loads and casts its own blocks straight into the
// operand layout (quarter l/16 of row l%16 in lane l; the block amax is
// taken across those four lanes); with 16 < m <= 32 and the cast fused, the
// workgroup casts 16 rows at a time into LDS and each wave copies its
// operands out. Either way the rule and arithmetic are those of every other
// cast, so codes and scales equal fp8bs_quantize_act's. Requires
// kbn <= NJ * WK; waves whose block index passes kbn skip it. Products are accumulated in the same
// order as gemm_rows_kernel with the same WK, and summed across waves in
// wave order.
//
// Weights: wave slot j holds block wk + j WK of the current 16-row tile; it
// is refilled with the next tile's block as soon as it has been multiplied,
// so NJ blocks per wave stay in flight. PRE of them are requested before
// the activation cast.
// ====================================================================

template <int MT, int NJ>
struct RegAct {
  i32x8 op[NJ][MT];  // B operands (zero for rows past m)
  float s[NJ][MT];   // activation scale of row l%16 + 16 mt (0 past m)
};

template <int MT, int WK, int NJ, int PRE, bool FUSED, bool SW = false, bool PK = false>
__global__ __launch_bounds__(64 * WK) void gemm_rows_reg_kernel(GemmParams p) {
  constexpr int NT = 64 * WK;
  extern __shared__ __align__(16) uint8_t lds_all[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wk = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int M = p.m;
  const int nblk = p.kbn;
  const int r0 = blockIdx.x * p.rows_per_wg;
  const int r1 = r0 + p.rows_per_wg < p.n ? r0 + p.rows_per_wg : p.n;
  const int nrows = r1 - r0;
  const int ntile = (nrows + 15) >> 4;
  const int nbf = r0 / BLK, nbr = (r1 - 1) / BLK - nbf + 1;
  float* wsl = reinterpret_cast<float*>(lds_all);
  f32x4* red = reinterpret_cast<f32x4*>(lds_all + lds_wscale_bytes(p.rows_per_wg, nblk));
  // m > 16 with the cast fused: the 16-row cast area (lds_act_bytes(nblk, 16))
  uint8_t* act = reinterpret_cast<uint8_t*>(red) + 2 * (WK - 1) * MT * 64 * 16;
  // SwiGLU epilogue: bf16 outputs staged after the other areas
  uint16_t* ystage =
      reinterpret_cast<uint16_t*>(act + (FUSED && MT == 2 ? lds_act_bytes(nblk, 16) : 0));

  const int l16 = lane & 15, g16 = lane >> 4;
  const int l7 = lane & 7, hb = (lane >> 3) & 1;
  const bool lo8 = hb == 0;

  // block of slot j (clamped for the address; the multiply is skipped)
  auto slot_block = [&](int j) {
    const int kb = wk + j * WK;
    return kb < nblk ? kb : nblk - 1;
  };
  auto act_row = [&](int mt) {
    const int m = l16 + 16 * mt;
    return m < M ? m : M - 1;
  };

  TileLoad wb[NJ];
  auto load_slot = [&](int j, int t) {
    t = t < ntile ? t : ntile - 1;
    if constexpr (PK) {
      int ra = 16 * t + l16;
      ra = ra < nrows ? ra : nrows - 1;
      const uint8_t* a = p.wq + tile_layout_off(r0 + ra, slot_block(j), p.kbn, g16);
      wb[j].p = load_stream16(a);
      wb[j].q = load_stream16(a + 1024);
    } else {
      int ra = 16 * t + l7, rb = 16 * t + 8 + l7;
      ra = ra < nrows ? ra : nrows - 1;
      rb = rb < nrows ? rb : nrows - 1;
      const uint8_t* base = p.wq + (size_t)slot_block(j) * BLK;
      wb[j].p = load_stream16(base + (size_t)(r0 + ra) * (size_t)p.k + 16 * (2 * g16 + hb));
      wb[j].q = load_stream16(base + (size_t)(r0 + rb) * (size_t)p.k + 16 * (2 * g16 + 1 - hb));
    }
  };
  RegAct<MT, NJ> xa;
  ScaleFetch sf;

  if constexpr (FUSED && MT == 2) {
    // Activations cast cooperatively through LDS, 16 rows at a time (the
    // bf16 values of a wave's own blocks would not fit in registers next to
    // the operands): quarter g of a half is (block g / 64, row (g / 4) % 16,
    // quarter g % 4), in the quad layout cast_quarter takes. A thread holds
    // at most NJ quarters per half (kbn <= NJ WK). Both halves are loaded
    // before the first weight slot is requested.
    float* act_s = reinterpret_cast<float*>(act + nblk * 16 * ACT_STRIDE);
    const int G = nblk * 64;
    uint4 xh[2][NJ][4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < NJ; ++i) {
        int g = tid + i * NT;
        g = g < G ? g : G - 1;
        const int bm = g >> 2;
        int m = 16 * h + (bm & 15);
        m = m < M ? m : M - 1;
        const uint4* src = reinterpret_cast<const uint4*>(
            p.x + (size_t)m * (size_t)p.k + (size_t)(bm >> 4) * BLK + 32 * (g & 3));
#pragma unroll
        for (int q = 0; q < 4; ++q) xh[h][i][q] = src[q];
      }
    load_wscales<NT>(p, nbf, nbr, 0, nblk, tid, sf);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < PRE && j < NJ; ++j) load_slot(j, 0);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (h == 1) lds_barrier();  // every wave has read the first half
#pragma unroll
      for (int i = 0; i < NJ; ++i) {
        const int g = tid + i * NT;
        uint32_t c[8];
        const float sc = cast_quarter(xh[h][i], c);  // the whole quad takes part
        if (g < G) {  // G is a multiple of 4: the four lanes of a quad agree
          const int bm = g >> 2;
          uint4* d = reinterpret_cast<uint4*>(act + bm * ACT_STRIDE + (g & 3) * 32);
          d[0] = make_uint4(c[0], c[1], c[2], c[3]);
          d[1] = make_uint4(c[4], c[5], c[6], c[7]);
          if ((g & 3) == 0) act_s[bm] = sc;
        }
        if (h == 0 && PRE + i < NJ) load_slot(PRE + i, 0);
      }
      lds_barrier();
      const bool live = 16 * h + l16 < M;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int bm = slot_block(j) * 16 + l16;
        const uint4* a = reinterpret_cast<const uint4*>(act + bm * ACT_STRIDE + 32 * g16);
        const uint4 lo = a[0], hi = a[1];
        xa.op[j][h] = live ? i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                                   (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w}
                           : i32x8{0, 0, 0, 0, 0, 0, 0, 0};
        xa.s[j][h] = live ? act_s[bm] : 0.0f;
      }
    }
  } else {
    // Each wave loads (and casts) the operands of its own blocks straight
    // into registers: quarter l/16 of row l%16 of each block; the activation
    // loads come before any weight load, so each cast waits for activation
    // loads only.
    uint4 xr[NJ][MT][4];
    float xsr[NJ][MT];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int kb = slot_block(j);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int m = act_row(mt);
        if constexpr (FUSED) {
          const uint4* src = reinterpret_cast<const uint4*>(p.x + (size_t)m * (size_t)p.k +
                                                            (size_t)kb * BLK + 32 * g16);
#pragma unroll
          for (int i = 0; i < 4; ++i) xr[j][mt][i] = src[i];
        } else {
          const uint4* src = reinterpret_cast<const uint4*>(p.xq + (size_t)m * (size_t)p.k +
                                                            (size_t)kb * BLK + 32 * g16);
          xr[j][mt][0] = src[0];
          xr[j][mt][1] = src[1];
          xsr[j][mt] = p.xs[(size_t)m * (size_t)p.kbn + kb];
        }
      }
    }
    load_wscales<NT>(p, nbf, nbr, 0, nblk, tid, sf);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < PRE && j < NJ; ++j) load_slot(j, 0);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const bool live = l16 + 16 * mt < M;
        uint32_t c[8];
        float sc;
        if constexpr (FUSED) {
          sc = cast_quarter_cols(xr[j][mt], c);  // every lane takes part in the shuffles
        } else {
          const uint4 lo = xr[j][mt][0], hi = xr[j][mt][1];
          c[0] = lo.x; c[1] = lo.y; c[2] = lo.z; c[3] = lo.w;
          c[4] = hi.x; c[5] = hi.y; c[6] = hi.z; c[7] = hi.w;
          sc = xsr[j][mt];
        }
        xa.op[j][mt] = live ? i32x8{(int)c[0], (int)c[1], (int)c[2], (int)c[3], (int)c[4],
                                    (int)c[5], (int)c[6], (int)c[7]}
                            : i32x8{0, 0, 0, 0, 0, 0, 0, 0};
        xa.s[j][mt] = live ? sc : 0.0f;
      }
      if (PRE + j < NJ) load_slot(PRE + j, 0);
    }
  }
  store_wscales<NT>(p, nbf, nbr, 0, nblk, tid, sf, wsl);
  lds_barrier();

  // 4. tiles: multiply slot j, refill it with the next tile's block
  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto multiply_tile = [&](int t, auto refill) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int kb = wk + j * WK;
      if (kb < nblk) {
        // this lane's four output rows lie in one 128-row scale block
        int nbl = (r0 + 16 * t + 4 * g16) / BLK - nbf;
        nbl = nbl < nbr ? nbl : nbr - 1;
        const float sw = wsl[nbl * nblk + kb];
        const i32x8 aop = weight_operand<PK>(wb[j], lo8);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const f32x4 z = {0.f, 0.f, 0.f, 0.f};
          const f32x4 pb = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              aop, xa.op[j][mt], z, 0, 0, 0, 0, 0, 0);
          const float sc = xa.s[j][mt] * sw;
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[mt][q] = __builtin_fmaf(pb[q], sc, acc[mt][q]);
        }
      }
      if constexpr (decltype(refill)::value) load_slot(j, t + 1);
    }
    // partial sums of waves 1..WK-1 through LDS, summed in wave order
    f32x4* rt = red + (t & 1) * (WK - 1) * MT * 64;
    if (wk > 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) rt[((wk - 1) * MT + mt) * 64 + lane] = acc[mt];
    }
    lds_barrier();
    if (wk == 0) {
      for (int w = 1; w < WK; ++w)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] += rt[((w - 1) * MT + mt) * 64 + lane];
      const int rl = 16 * t + 4 * g16;  // first of this lane's four rows
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int m = l16 + 16 * mt;
        if (m < M && rl < nrows) {
          if constexpr (SW) {
            stage_y4(ystage, p.rows_per_wg, m, rl, acc[mt][0], acc[mt][1], acc[mt][2],
                     acc[mt][3]);
          } else {
            uint2* dst = reinterpret_cast<uint2*>(p.y + (size_t)m * (size_t)p.n + r0 + rl);
            *dst = make_uint2(pack_bf16x2(acc[mt][0], acc[mt][1]),
                              pack_bf16x2(acc[mt][2], acc[mt][3]));
          }
        }
      }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  };

  for (int t = 0; t + 1 < ntile; ++t) multiply_tile(t, std::true_type{});
  multiply_tile(ntile - 1, std::false_type{});
  if constexpr (SW) {
    flush_ystage<NT>(p, ystage, r0, nrows, tid);
    swiglu_arrive<NT>(p, r0, r1, p.rows_per_wg, gridDim.x, tid);
  }
}

// ====================================================================
// MFMA streaming row-range kernel: the work split of gemm_rows_kernel (one
// workgroup per compute unit, a contiguous range of output columns over the
// whole K range, waves interleaving the K blocks of each 16-row tile), but
// without a staging phase. Wave w is the only reader of the activation
// blocks kb = w, w + WK, ..., so it stages exactly those itself, each one
// when the first tile reaches it: the bf16 block (or its codes and scales)
// is fetched together with the weight tile of that item, cast in registers,
// and kept in LDS for the later tiles. The cast of the whole activation is
// thereby spread over the weight stream instead of delaying its start, and
// each workgroup still casts every activation element once.
//
// Staging layout: a K block of m activation rows is 8m segments of 16
// values; segment task = 8 * row + seg is handled by lane task % 64 of pass
// task / 64, so the 8 segments of one row sit in 8 adjacent lanes and the
// block amax is an 8-lane reduction. Codes go to LDS as 16-byte chunks
// [kb][seg][row], which the MFMA B operand reads back without bank
// conflicts (lane = row, two consecutive segments).
//
// Activation fetches go through a buffer resource: items of later tiles
// issue the same load instructions with an out-of-range offset, which
// return zeros without touching memory, so every item issues the same
// number of loads and the wait counts stay exact.
// ====================================================================

// LDS bytes of the streaming kernel: codes [kbn][8][m] x 16, scales
// [kbn][m] fp32 (padded to 16), tile-sum exchange [2][WK-1][MT][64] x 16.
__host__ __device__ inline int lds_stream_bytes(int kbn, int m, int wk, int mt) {
  return kbn * m * BLK + ((kbn * m * 4 + 15) & ~15) + 2 * (wk - 1) * mt * 64 * 16;
}

constexpr uint32_t BUF_OOB = 0x80000000u;  // an offset past every staged tensor

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float octet_max(float v) {
  v = __builtin_fmaxf(v, dpp_f<DPP_QUAD_XOR1>(v));
  v = __builtin_fmaxf(v, dpp_f<DPP_QUAD_XOR2>(v));
  v = __builtin_fmaxf(v, dpp_f<DPP_ROW_HALF_MIRROR>(v));
  return v;
}

// One K block of activations as fetched by one wave: per pass, 16 bf16
// values (two 16-byte loads) or 16 codes plus the row's scale.
template <int XP>
struct ActFetch {
  uint4 a[XP];
  uint4 b[XP];  // fused: values 8..15; pre-quantized: .x holds the scale bits
};

// XP = staging passes (1, 2, 4): 8 * XP >= m activation rows.
template <int XP, int WK, int D, bool FUSED, bool SW = false, bool PK = false>
__global__ __launch_bounds__(64 * WK) void gemm_stream_kernel(GemmParams p) {
  constexpr int MT = XP > 2 ? 2 : 1;  // 16-row activation tiles of the MFMA B operand
  extern __shared__ __align__(16) uint8_t lds_all[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wk = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int M = p.m;
  const int kbn = p.kbn;
  const int r0 = blockIdx.x * p.rows_per_wg;
  const int r1 = r0 + p.rows_per_wg < p.n ? r0 + p.rows_per_wg : p.n;
  const int nrows = r1 - r0;
  const int ntile = (nrows + 15) >> 4;
  const int njw = (kbn + WK - 1) / WK;  // blocks per tile per wave (same for every wave)
  const int nitem = ntile * njw;

  const int nbf = r0 / BLK, nbr = (r1 - 1) / BLK - nbf + 1;
  float* wsl = reinterpret_cast<float*>(lds_all);
  uint8_t* lds = lds_all + lds_wscale_bytes(p.rows_per_wg, kbn);
  uint4* act = reinterpret_cast<uint4*>(lds);                     // [kbn][8][M] chunks
  float* act_s = reinterpret_cast<float*>(lds + kbn * M * BLK);    // [kbn][M]
  f32x4* red = reinterpret_cast<f32x4*>(lds + kbn * M * BLK + ((kbn * M * 4 + 15) & ~15));
  uint16_t* ystage = reinterpret_cast<uint16_t*>(lds + lds_stream_bytes(kbn, M, WK, MT));

  const int l16 = lane & 15, g16 = lane >> 4;
  const int l7 = lane & 7, hb = (lane >> 3) & 1;
  const bool lo8 = hb == 0;

  // activation sources (byte offsets < 2^31 are guaranteed by the host)
  const __amdgpu_buffer_rsrc_t xr =
      FUSED ? buffer_rsrc(p.x, (uint32_t)M * (uint32_t)p.k * 2u)
            : buffer_rsrc(p.xq, (uint32_t)M * (uint32_t)p.k);
  const __amdgpu_buffer_rsrc_t sr = buffer_rsrc(p.xs, FUSED ? 0u : (uint32_t)M * (uint32_t)kbn * 4u);

  TileLoad wb[D];
  ActFetch<XP> xb[D];
  auto load_item = [&](int d, int i) {
    i = i < nitem ? i : nitem - 1;
    const int t = i / njw, j = i - t * njw;
    int kb = wk + j * WK;
    const bool stage = t == 0 && kb < kbn;
    kb = kb < kbn ? kb : kbn - 1;
    if constexpr (PK) {
      int ra = 16 * t + l16;
      ra = ra < nrows ? ra : nrows - 1;
      const uint8_t* a = p.wq + tile_layout_off(r0 + ra, kb, kbn, g16);
      wb[d].p = load_stream16(a);
      wb[d].q = load_stream16(a + 1024);
    } else {
      int ra = 16 * t + l7, rb = 16 * t + 8 + l7;
      ra = ra < nrows ? ra : nrows - 1;
      rb = rb < nrows ? rb : nrows - 1;
      const uint8_t* base = p.wq + (size_t)kb * BLK;
      wb[d].p = load_stream16(base + (size_t)(r0 + ra) * (size_t)p.k + 16 * (2 * g16 + hb));
      wb[d].q = load_stream16(base + (size_t)(r0 + rb) * (size_t)p.k + 16 * (2 * g16 + 1 - hb));
    }
#pragma unroll
    for (int c = 0; c < XP; ++c) {
      const int task = 64 * c + lane;
      const int m = task >> 3, seg = task & 7;
      const bool live = stage && m < M;
      if constexpr (FUSED) {
        const uint32_t off = live ? ((uint32_t)m * (uint32_t)p.k + (uint32_t)kb * BLK + 16u * seg) * 2u
                                  : BUF_OOB;
        xb[d].a[c] = buffer_load16(xr, off);
        xb[d].b[c] = buffer_load16(xr, off + 16u);
      } else {
        const uint32_t off = live ? (uint32_t)m * (uint32_t)p.k + (uint32_t)kb * BLK + 16u * seg
                                  : BUF_OOB;
        const uint32_t soff = live ? ((uint32_t)m * (uint32_t)kbn + (uint32_t)kb) * 4u : BUF_OOB;
        xb[d].a[c] = buffer_load16(xr, off);
        xb[d].b[c].x = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(sr, soff, 0, 0);
      }
    }
  };

  // Stage K block kb (first tile only): cast or copy into LDS.
  auto stage_block = [&](int d, int kb) {
#pragma unroll
    for (int c = 0; c < XP; ++c) {
      const int task = 64 * c + lane;
      const int m = task >> 3, seg = task & 7;
      if (c > 0 && 64 * c >= 8 * M) break;  // no rows left in this pass (uniform)
      uint4 codes;
      float s;
      if constexpr (FUSED) {
        const uint32_t w[8] = {xb[d].a[c].x, xb[d].a[c].y, xb[d].a[c].z, xb[d].a[c].w,
                               xb[d].b[c].x, xb[d].b[c].y, xb[d].b[c].z, xb[d].b[c].w};
        float x[16];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          x[2 * e] = bf16_lo(w[e]);
          x[2 * e + 1] = bf16_hi(w[e]);
        }
        float am = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) am = __builtin_fmaxf(am, __builtin_fabsf(x[e]));
        am = octet_max(am);
        s = am / 448.0f;
        block_quotients(x, am, s);
        codes = make_uint4(e4m3x4(x[0], x[1], x[2], x[3]), e4m3x4(x[4], x[5], x[6], x[7]),
                           e4m3x4(x[8], x[9], x[10], x[11]), e4m3x4(x[12], x[13], x[14], x[15]));
      } else {
        codes = xb[d].a[c];
        s = __uint_as_float(xb[d].b[c].x);
      }
      if (m < M) {
        act[(kb * 8 + seg) * M + m] = codes;
        if (seg == 0) act_s[kb * M + m] = s;
      }
    }
  };

  ScaleFetch sf;
  load_wscales<64 * WK>(p, nbf, nbr, 0, kbn, tid, sf);
  __builtin_amdgcn_sched_barrier(0);
  // Issue order must match the loop's (item by item) for the wait counts
  // of the loop to be tight: keep the scheduler from interleaving items.
#pragma unroll
  for (int d = 0; d < D; ++d) {
    load_item(d, d);
    __builtin_amdgcn_sched_barrier(0);
  }
  store_wscales<64 * WK>(p, nbf, nbr, 0, kbn, tid, sf, wsl);
  lds_barrier();

  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int d, int i) {
    const int t = i / njw, j = i - t * njw;
    const int kb = wk + j * WK;
    if (kb < kbn) {
      if (t == 0) stage_block(d, kb);
      // this lane's four output rows lie in one 128-row scale block (row
      // ranges are multiples of 4); lanes past the range read a valid entry
      int nbl = (r0 + 16 * t + 4 * g16) / BLK - nbf;
      nbl = nbl < nbr ? nbl : nbr - 1;
      const float sw = wsl[nbl * kbn + kb];
      const i32x8 aop = weight_operand<PK>(wb[d], lo8);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int m = l16 + 16 * mt;
        i32x8 bop = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
        float sa = 0.0f;
        if (m < M) {
          const uint4 lo = act[(kb * 8 + 2 * g16) * M + m];
          const uint4 hi = act[(kb * 8 + 2 * g16 + 1) * M + m];
          bop = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                      (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
          sa = act_s[kb * M + m];
        }
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        const f32x4 pb =
            __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop, bop, z, 0, 0, 0, 0, 0, 0);
        const float sc = sa * sw;
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[mt][q] = __builtin_fmaf(pb[q], sc, acc[mt][q]);
      }
    }
    if (j == njw - 1) {
      f32x4* rt = red + (t & 1) * (WK - 1) * MT * 64;
      if (wk > 0) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) rt[((wk - 1) * MT + mt) * 64 + lane] = acc[mt];
      }
      lds_barrier();
      if (wk == 0) {
        for (int w = 1; w < WK; ++w)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) acc[mt] += rt[((w - 1) * MT + mt) * 64 + lane];
        const int rl = 16 * t + 4 * g16;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int m = l16 + 16 * mt;
          if (m < M && rl < nrows) {
            if constexpr (SW) {
              stage_y4(ystage, p.rows_per_wg, m, rl, acc[mt][0], acc[mt][1], acc[mt][2],
                       acc[mt][3]);
            } else {
              uint2* dst = reinterpret_cast<uint2*>(p.y + (size_t)m * (size_t)p.n + r0 + rl);
              *dst = make_uint2(pack_bf16x2(acc[mt][0], acc[mt][1]),
                                pack_bf16x2(acc[mt][2], acc[mt][3]));
            }
          }
        }
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };

  const int ngrp = (nitem + D - 1) / D;
  for (int g = 0; g + 1 < ngrp; ++g) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      compute(d, g * D + d);
      load_item(d, (g + 1) * D + d);
    }
  }
#pragma unroll
  for (int d = 0; d < D; ++d) {
    const int i = (ngrp - 1) * D + d;
    if (i < nitem) compute(d, i);
  }
  if constexpr (SW) {
    flush_ystage<64 * WK>(p, ystage, r0, nrows, tid);
    swiglu_arrive<64 * WK>(p, r0, r1, p.rows_per_wg, gridDim.x, tid);
  }
}

// ====================================================================
// DOT path (smallest m): lane l handles weight row (l/8) of each 8-row
// group and the 16-byte K segment l%8 of each block; it converts its 16
// codes to fp32 and forms m dot products against the decoded activation
// codes of the same K positions. Per block the lane rescales its partial by
// xs * ws; the 8 lanes of a row are summed once at the end.
// ====================================================================

// Body of the DOT kernel for CR activation-load rounds per thread.
template <int MD, int RT, int WN, int WK, int D, bool FUSED, int CR>
__device__ __forceinline__ void gemm_dot_body(const GemmParams& p, uint8_t* lds_all) {
  constexpr int NT = 64 * WN * WK;
  constexpr int ROWS = 8 * RT * WN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave % WN, wk = wave / WN;
  const int s = blockIdx.y;
  int kb0, kb1;
  split_range(s, p.split, p.kbn, kb0, kb1);
  const int nblk = kb1 - kb0;
  const int M = p.m;

  const int n0 = blockIdx.x * ROWS;
  uint8_t* lds = lds_all;
  uint8_t* act = lds;
  float* act_s = reinterpret_cast<float*>(lds + nblk * M * ACT_STRIDE);
  float* red = reinterpret_cast<float*>(lds + lds_act_bytes(nblk, M));
  const int row0 = n0 + wn * 8 * RT;
  const int r8 = lane >> 3, seg = lane & 7;
  const uint8_t* wrow = p.wq + (size_t)(row0 + r8) * (size_t)p.k + 16 * seg;
  const int nj = nblk > wk ? (nblk - wk + WK - 1) / WK : 0;

  stage_act_tail<NT, CR, FUSED>(p, kb0, nblk, tid, act, act_s);
  uint4 xr[CR][4];
  if constexpr (FUSED) load_act_quarters<NT, CR>(p, kb0, nblk * M * 4, tid, 0, xr);
  __builtin_amdgcn_sched_barrier(0);  // activation loads stay ahead of the weight loads

  uint4 wb[D][RT];
  auto load_block = [&](int d, int j) {
    const int jc = j < nj ? j : (nj > 0 ? nj - 1 : 0);
    int kb = kb0 + wk + jc * WK;
    kb = kb < p.kbn ? kb : p.kbn - 1;
    const uint8_t* src = wrow + (size_t)kb * BLK;
#pragma unroll
    for (int t = 0; t < RT; ++t)
      wb[d][t] = load_stream16(src + (size_t)t * 8 * (size_t)p.k);
  };
  constexpr int PRE = D < 2 ? D : 2;
#pragma unroll
  for (int d = 0; d < PRE; ++d) load_block(d, d);

  stage_act<NT, CR, FUSED>(p, kb0, nblk, tid, xr, act, act_s);
#pragma unroll
  for (int d = PRE; d < D; ++d) load_block(d, d);
  lds_barrier();

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
    const float sw = load_invariant(p.ws, (size_t)(row0 / BLK) * (size_t)p.kbn + kb);
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
          if (p.out == OUT_DIRECT)
            p.y[(size_t)m * (size_t)p.n + n] = (uint16_t)bf16_rne(acc[t][m]);
          else if (p.out == OUT_LAST_ARRIVER)
            __hip_atomic_store(p.part + ((size_t)s * M + m) * (size_t)p.n + n, acc[t][m],
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          else
            p.part[((size_t)s * M + m) * (size_t)p.n + n] = acc[t][m];
        }
      }
    }
  }
  if (p.out == OUT_LAST_ARRIVER) last_arriver_reduce<NT, ROWS>(p, n0, tid);
}

template <int MD, int RT, int WN, int WK, int D, bool FUSED>
__global__ __launch_bounds__(64 * WN * WK) void gemm_dot_kernel(GemmParams p) {
  constexpr int NT = 64 * WN * WK;
  extern __shared__ __align__(16) uint8_t lds_all[];
  if constexpr (FUSED) {
    int kb0, kb1;
    split_range(blockIdx.y, p.split, p.kbn, kb0, kb1);
    const int rounds = act_rounds((kb1 - kb0) * p.m * 4, NT);
    if (rounds == 1)
      gemm_dot_body<MD, RT, WN, WK, D, true, 1>(p, lds_all);
    else if (rounds == 2)
      gemm_dot_body<MD, RT, WN, WK, D, true, 2>(p, lds_all);
    else
      gemm_dot_body<MD, RT, WN, WK, D, true, 3>(p, lds_all);
  } else {
    gemm_dot_body<MD, RT, WN, WK, D, false, 1>(p, lds_all);
  }
}

}  // namespace fp8bs
