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

#include <type_traits>

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


// ---------------------------------------------------------------------------
// Prefill kernel with direct global-to-LDS loads. The same tiles, operand
// layout and rescale as gemm_prefill_kernel, but the K blocks travel from
// memory straight into a ring of S LDS stages (global_load_lds: each
// instruction writes 64 lanes x 16 bytes to 1 KB of consecutive LDS at the
// address in M0; the 4-byte form, 64 x 4 bytes), so no registers hold blocks
// in flight and S - 1 blocks are on their way while one is multiplied.
//
// Stage layout: weight rows [64 WN][128], activation rows [128][128] and
// activation scales [128]. Rows are not padded (each load instruction fills
// 1 KB of consecutive LDS); instead 16-byte segment s of row r sits at
// position s ^ pf_swz(r), which spreads the MFMA operand reads of 16
// consecutive rows over all banks.
//
// The loads are issued from inline assembly so that the compiler does not
// make every LDS read wait for all of them; the waits are explicit. Every
// wave issues the same number of loads per stage (PF_DMA_PER_STAGE), so
// waiting until at most (S - 2) stages' worth of this wave's loads are
// outstanding means its loads of the stage about to be read have landed; the
// barrier after that wait (which also drains this wave's LDS reads) makes the
// whole stage visible and frees the stage read in the previous iteration,
// which is the one refilled next. Blocks past the K range are loaded again
// from the last block into the stage nobody reads, so the count never
// changes; the wave drains its loads before it exits.
__host__ __device__ constexpr int pf_dma_stage_bytes(int wn) {
  return pf_tile_n(wn) * BLK + PF_TILE_M * BLK + PF_TILE_M * 4;
}
__host__ __device__ constexpr int pf_dma_lds_bytes(int wn, int stages) {
  return stages * pf_dma_stage_bytes(wn);
}
// loads per wave and stage: 4 weight, 8 / WN activation, 1 scale
__host__ __device__ constexpr int pf_dma_per_stage(int wn) { return 4 + 8 / wn + 1; }

__device__ __forceinline__ int pf_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// 32 K bytes of swizzled row `row` for lane group g (segments 2g, 2g + 1).
__device__ __forceinline__ i32x8 pf_swz_operand(const uint8_t* rows, int row, int g) {
  const uint8_t* a = rows + row * BLK;
  const int z = pf_swz(row);
  const uint4 lo = *reinterpret_cast<const uint4*>(a + 16 * ((2 * g) ^ z));
  const uint4 hi = *reinterpret_cast<const uint4*>(a + 16 * ((2 * g + 1) ^ z));
  return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>(p);
}

// One 16-byte (or 4-byte) direct load per lane: LDS[m0 + 16 lane] (or 4 lane)
// = global[base + voff].
__device__ __forceinline__ void dma16(uint32_t m0, const void* base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(m0), "v"(voff), "s"(base)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(uint32_t m0, const void* base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
               :
               : "s"(m0), "v"(voff), "s"(base)
               : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_loads_then_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(N) : "memory");
}

// Output tile of this workgroup. Workgroups are dispatched to the 8 XCDs in
// turn (linear id mod 8), and each XCD has its own L2. In dispatch order,
// XCD c gets the weight (n) tiles x = c mod 8 and every activation (m) tile,
// so with many n tiles each activation tile is fetched into all eight L2s.
// For wide unsplit grids (at least 64 n tiles, a multiple of 8 tiles in
// all) the order is remapped so that XCD c takes a contiguous eighth of a
// grouped order: groups of up to 8 m tiles, and inside a group consecutive
// tiles share one n tile. The workgroups resident on one XCD then read a
// few weight and activation tiles in step from that XCD's L2. Measured on
// MI355X: 5-9% faster at N = 34816; slower on 40 n tiles, where the plain
// order already keeps each weight tile on one XCD. The map is a permutation
// of the tiles, so any dispatch order gives the same result.
__device__ __forceinline__ void pf_tile_order(int& bx, int& by) {
  const int gx = gridDim.x, gy = gridDim.y, nxy = gx * gy;
  bx = blockIdx.x;
  by = blockIdx.y;
  if ((nxy & 7) != 0 || gx < 64 || gridDim.z != 1) return;
  const int id = bx + gx * by;
  const int t = (id & 7) * (nxy >> 3) + (id >> 3);
  constexpr int GM = 8;
  const int group = t / (GM * gx);
  const int first = group * GM;
  const int gm = gy - first < GM ? gy - first : GM;
  const int r = t - group * GM * gx;
  by = first + r % gm;
  bx = r / gm;
}

// Blocks kb + I, I = 0 .. S-1, one per ring stage I (compile-time).
template <int I, int S, typename F>
__device__ __forceinline__ void pf_ring_turn(int kb, F& f) {
  if constexpr (I < S) {
    f(kb + I, std::integral_constant<int, I>{});
    pf_ring_turn<I + 1, S>(kb, f);
  }
}
// The blocks kb .. last (fewer than S) left after the whole turns.
template <int I, int S, typename F>
__device__ __forceinline__ void pf_ring_tail(int kb, int last, F& f) {
  if constexpr (I < S - 1) {
    if (kb + I <= last) {
      f(kb + I, std::integral_constant<int, I>{});
      pf_ring_tail<I + 1, S>(kb, last, f);
    }
  }
}

// grid: (n / (64 WN), ceil(m / 128), split); 128 WN threads;
// pf_dma_lds_bytes(WN, S) of dynamic LDS. Otherwise as gemm_prefill_kernel.
//
// EARLY: a stage is refilled as soon as every wave has copied the block's
// operands into registers (a second barrier right after those reads),
// with the block S later, instead of when the next block starts: S blocks
// are then in flight while one is multiplied, from the same LDS.
// Tile-layout weights (PK): a stage's weight rows are 4 WN whole 16-row
// tiles of 2 KB (the tile layout of the codes, see tile_layout_off); load
// instruction q of the stage copies KB q (tile q/2, half q%2) as it is, so
// the stage holds the tiles in operand order and lane l reads the two
// 16-byte halves of its A operand at t*2048 + 16l and t*2048 + 1024 + 16l
// (consecutive lanes, consecutive bytes: no bank conflicts, no swizzle).
__device__ __forceinline__ i32x8 pf_tile_operand(const uint8_t* rows, int t, int lane) {
  const uint4 lo = *reinterpret_cast<const uint4*>(rows + t * 2048 + 16 * lane);
  const uint4 hi = *reinterpret_cast<const uint4*>(rows + t * 2048 + 1024 + 16 * lane);
  return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

template <int WN, int S, bool EARLY = false, bool PK = false>
__global__ __launch_bounds__(128 * WN, WN == 2 ? 2 : 1) void gemm_prefill_dma_kernel(GemmParams p) {
  static_assert(S >= 2 && (S - 1) * pf_dma_per_stage(WN) <= 63, "vmcnt range");
  extern __shared__ __align__(16) uint8_t lds_all[];
  constexpr int STAGE = pf_dma_stage_bytes(WN);
  constexpr int WROWS = pf_tile_n(WN);
  constexpr int XI = 8 / WN;  // activation load instructions per wave and stage
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave % WN, wm = wave / WN;
  int bx, by;
  pf_tile_order(bx, by);
  const int n0 = bx * WROWS, m0 = by * PF_TILE_M;
  const int l16 = lane & 15, g = lane >> 4;
  int kb0, kb1;
  split_range(blockIdx.z, p.split, p.kbn, kb0, kb1);
  const int last = kb1 - 1;
  const float* wsrow = p.ws + (size_t)((n0 + 64 * wn) / BLK) * (size_t)p.kbn;
  const uint32_t lds0 = lds_addr(lds_all);

  // per-lane load offsets (the block's K offset goes into the scalar base)
  uint32_t wo[4], xo[XI];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (PK) {
      const int q = 4 * wave + i;
      wo[i] = (uint32_t)(q >> 1) * (uint32_t)p.kbn * 2048u + (uint32_t)(q & 1) * 1024u +
              16u * (uint32_t)lane;
    } else {
      const int r = 8 * (4 * wave + i) + (lane >> 3);
      wo[i] = (uint32_t)r * (uint32_t)p.k + 16u * (uint32_t)((lane & 7) ^ pf_swz(r));
    }
  }
#pragma unroll
  for (int i = 0; i < XI; ++i) {
    const int r = 8 * (XI * wave + i) + (lane >> 3);
    const int mr = m0 + r < p.m ? r : p.m - 1 - m0;
    xo[i] = (uint32_t)mr * (uint32_t)p.k + 16u * (uint32_t)((lane & 7) ^ pf_swz(r));
  }
  const int sr = 64 * (wave & 1) + lane;  // scale row of this lane
  const uint32_t so = (uint32_t)(m0 + sr < p.m ? sr : p.m - 1 - m0) * (uint32_t)p.kbn * 4u;
  // row-major: row n0, the block's K offset added per block; tile layout:
  // tile n0/16 of K block 0, the block's 2 KB step added per block
  const uint8_t* wbase = PK ? p.wq + (size_t)(n0 >> 4) * (size_t)p.kbn * 2048u
                            : p.wq + (size_t)n0 * (size_t)p.k;
  const uint8_t* xbase = p.xq + (size_t)m0 * (size_t)p.k;
  const float* sbase = p.xs + (size_t)m0 * (size_t)p.kbn;

  auto issue = [&](int kb, int stage) {
    kb = kb < last ? kb : last;
    const uint32_t st = lds0 + (uint32_t)(stage * STAGE);
    const uint8_t* wb = wbase + (size_t)kb * (PK ? 2048u : (size_t)BLK);
    const uint8_t* xb = xbase + (size_t)kb * BLK;
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(st + (uint32_t)(4 * wave + i) * 1024u, wb, wo[i]);
#pragma unroll
    for (int i = 0; i < XI; ++i)
      dma16(st + (uint32_t)(WROWS * BLK) + (uint32_t)(XI * wave + i) * 1024u, xb, xo[i]);
    dma4(st + (uint32_t)(WROWS * BLK + PF_TILE_M * BLK) + (uint32_t)(wave & 1) * 256u,
         sbase + kb, so);
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int s = 0; s < (EARLY ? S : S - 1); ++s) issue(kb0 + s, s);

  // One K block out of stage ST (a compile-time ring position, so every
  // LDS address is a lane base plus an immediate): all operands first, then
  // the 16 products into separate registers, each rescaled into acc a few
  // products later, so no product waits on the one before it.
  auto block = [&](int kb, auto stc) {
    constexpr int ST = decltype(stc)::value;
    wait_loads_then_barrier<(EARLY ? S - 1 : S - 2) * pf_dma_per_stage(WN)>();
    if constexpr (!EARLY) issue(kb + S - 1, (ST + S - 1) % S);
    const uint8_t* st = lds_all + ST * STAGE;
    const uint8_t* wl = st;
    const uint8_t* xl = st + WROWS * BLK;
    const float* sl = reinterpret_cast<const float*>(xl + PF_TILE_M * BLK);
    const float sw = load_invariant(wsrow, (size_t)kb);
    i32x8 aop[4], bop[4];
    float sc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int mr = 64 * wm + 16 * j + l16;
      bop[j] = pf_swz_operand(xl, mr, g);
      if constexpr (PK)
        aop[j] = pf_tile_operand(wl, 4 * wn + j, lane);
      else
        aop[j] = pf_swz_operand(wl, 64 * wn + 16 * j + l16, g);
      sc[j] = sl[mr] * sw;
    }
    if constexpr (EARLY) {
      // every wave holds this block's operands: refill the stage
      lds_barrier();
      issue(kb + S, ST);
    }
    f32x4 pb[4][4];
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      pb[q >> 2][q & 3] =
          __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop[q >> 2], bop[q & 3], z, 0, 0, 0, 0, 0, 0);
      if (q >= 3) {
        const int r = q - 3, t = r >> 2, j = r & 3;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[t][j][i] = __builtin_fmaf(pb[t][j][i], sc[j], acc[t][j][i]);
      }
    }
#pragma unroll
    for (int r = 13; r < 16; ++r) {
      const int t = r >> 2, j = r & 3;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[t][j][i] = __builtin_fmaf(pb[t][j][i], sc[j], acc[t][j][i]);
    }
  };

  // block kb0 + i sits in stage i % S: whole turns of the ring, then the rest
  int kb = kb0;
  for (; kb + S - 1 <= last; kb += S) pf_ring_turn<0, S>(kb, block);
  pf_ring_tail<0, S>(kb, last, block);
  // no load may land in LDS after the workgroup has ended
  asm volatile("s_waitcnt vmcnt(0)" : : : "memory");

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


// Wide wave tiles. In the kernel above each wave owns 64 x 64 outputs, so per
// K block it reads 16 KB of operands out of LDS for 2 MFLOP, and a 128 x 128
// workgroup tile fetches 32 KB from L2 per 4 MFLOP. Here 8 waves, 4 along m
// by 2 along n, own a 256-column tile; each wave owns 16 JM rows (JM = 4 or
// 3 activation subtiles) by 128 columns (8 weight subtiles, one whole weight
// block row, so the weight scale is one value per wave and block). With
// JM = 4, 256 x 256 tiles read 24 KB of LDS per 4 MFLOP and fetch 64 KB per
// 16 MFLOP, half the L2 traffic per product of the 128 x 128 tile; JM = 3
// (192-row tiles) makes 4/3 as many tiles, for shapes where 256-row tiles
// leave compute units idle. One workgroup per compute unit (two stages take
// up to 130 KB of LDS). A workgroup can also take a half tile, 128 columns
// with 16 JM x 64 per wave (the last tile of an odd number of 128-column
// blocks, and the tail of the one-dimensional schedule below). The stages
// are filled by direct loads as in gemm_prefill_dma_kernel, issued by one
// loader wave per SIMD. Per block, a wave reads its activation operands,
// then for each weight subtile one operand and JM MFMAs, and rescales each
// subtile's products into the fp32 accumulators one subtile later; the wait
// and barrier that publish the next block come after the block's last
// operand read, so the last MFMAs run while the waves meet.
constexpr int PFW_TILE_N = 256;  // output columns of a whole tile
constexpr int PFW_NARROW_N = 160;  // output columns of a narrow tile (5 weight subtiles per wave)
constexpr int PF_WIDE = 3;       // tiles_n of a configuration: this kernel, grid schedule
constexpr int PF_WIDE_1D = 4;    // tiles_n of a configuration: this kernel, 1-D schedule
constexpr int PF_WIDE_160 = 5;   // tiles_n of a configuration: narrow tiles, 1-D schedule
// JM: activation subtiles (16 rows) per wave, 4 or 3; 4 waves along m, so
// a tile has 64 JM rows (256 or 192).
__host__ __device__ constexpr int pfw_tile_m(int jm) { return 64 * jm; }
__host__ __device__ constexpr int pfw_stage_bytes(int jm) {
  return PFW_TILE_N * BLK + pfw_tile_m(jm) * BLK + pfw_tile_m(jm) * 4;
}
__host__ __device__ constexpr int pfw_lds_bytes(int jm, int stages) {
  return stages * pfw_stage_bytes(jm);
}
// Waves that issue the stage loads (one per SIMD), and the loads each issues
// per stage with NT weight subtiles per wave (8: whole tile, 4: half tile):
// 4 NT / 4 weight pieces of 1 KB, the activation pieces, one scale piece.
constexpr int PFW_LOADERS = 4;
__host__ __device__ constexpr int pfw_per_stage(int jm, int nt) {
  return 4 * nt / PFW_LOADERS + pfw_tile_m(jm) * BLK / 1024 / PFW_LOADERS + 1;
}

// Tile q of the grouped order -> (n tile, m tile): groups of up to 8 m tiles,
// and inside a group consecutive q share one n tile.
__device__ __forceinline__ void pfw_tile_xy(int q, int tiles_n, int tiles_m, int& bx, int& by) {
  constexpr int GM = 8;
  const int group = q / (GM * tiles_n);
  const int first = group * GM;
  const int gm = tiles_m - first < GM ? tiles_m - first : GM;
  const int r = q - group * GM * tiles_n;
  by = first + r % gm;
  bx = r / gm;
}

// Work of a workgroup: output columns n0 .. n0 + 255 (half: n0 .. n0 + 127),
// rows m0 .., K blocks kb0 .. kb1 - 1.
// Grid schedule (p.pf_1d == 0): grid (ceil(n / 256), ceil(m / (64 JM)),
// split), the tile order of pf_tile_order, split z of K; a tile of one
// 128-column block is a half tile.
// 1-D schedule (p.pf_1d == 1): p.pf_full whole tiles, which fill complete
// rounds of resident workgroups, then two half-tile units for each tile
// left over (too few tiles to occupy every compute unit; each half has the
// whole K range, so halves meet no partial sums). Workgroups are dispatched
// to the 8 XCDs in turn, so whole tile b is taken from the grouped order at
// (b mod 8) * (p.pf_full / 8) + b / 8: each XCD works through its own
// contiguous eighth of it, a few weight and activation tiles at a time. The
// second half of a one-block tile is empty.
struct PfwWork {
  int n0, m0, kb0, kb1;
  bool half;
};
template <int TM>
__device__ __forceinline__ PfwWork pfw_work(const GemmParams& p) {
  PfwWork w;
  int bx, by;
  if (p.pf_1d == 0) {
    pf_tile_order(bx, by);
    split_range(blockIdx.z, p.split, p.kbn, w.kb0, w.kb1);
    w.n0 = bx * PFW_TILE_N;
    w.m0 = by * TM;
    w.half = w.n0 + BLK >= p.n;
    return w;
  }
  const int tiles_n = (p.n + PFW_TILE_N - 1) / PFW_TILE_N, tiles_m = (p.m + TM - 1) / TM;
  const int b = blockIdx.x, full = p.pf_full;
  w.kb0 = 0;
  w.kb1 = p.kbn;
  if (b < full) {
    pfw_tile_xy((full & 7) == 0 ? (b & 7) * (full >> 3) + (b >> 3) : b, tiles_n, tiles_m, bx, by);
    w.n0 = bx * PFW_TILE_N;
    w.half = w.n0 + BLK >= p.n;
  } else {
    const int u = b - full;
    pfw_tile_xy(full + (u >> 1), tiles_n, tiles_m, bx, by);
    w.n0 = bx * PFW_TILE_N + (u & 1) * BLK;
    w.half = true;
  }
  w.m0 = by * TM;
  return w;
}

// Work of a workgroup on narrow tiles (n a multiple of 160): whole tiles
// only, one per workgroup of the 1-D grid, in the grouped order with each
// XCD taking a contiguous eighth of it (as pfw_work's whole tiles).
template <int TM>
__device__ __forceinline__ PfwWork pfw_work_narrow(const GemmParams& p) {
  PfwWork w;
  int bx, by;
  const int tiles_n = p.n / PFW_NARROW_N, tiles_m = (p.m + TM - 1) / TM;
  const int b = blockIdx.x, full = p.pf_full;
  pfw_tile_xy((full & 7) == 0 ? (b & 7) * (full >> 3) + (b >> 3) : b, tiles_n, tiles_m, bx, by);
  w.n0 = bx * PFW_NARROW_N;
  w.m0 = by * TM;
  w.kb0 = 0;
  w.kb1 = p.kbn;
  w.half = false;
  return w;
}

// f(integral_constant<I>) for I = I0 .. N-1, in order.
template <int I, int N, typename F>
__device__ __forceinline__ void pf_static_for(F& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    pf_static_for<I + 1, N>(f);
  }
}

// One unit (whole tile, NT = 8; half tile, NT = 4; narrow tile, NT = 5) of
// the kernel below.
template <int JM, int S, bool PK, int NT, bool LOADER>
__device__ __forceinline__ void pfw_unit(const GemmParams& p, uint8_t* lds_all, const PfwWork& work) {
  constexpr int STAGE = pfw_stage_bytes(JM);
  constexpr int TM = pfw_tile_m(JM);
  constexpr int WR = 16 * JM;               // activation rows of a wave
  constexpr int LW = PFW_LOADERS;
  constexpr int WQ = 4 * NT / LW;           // weight pieces (1 KB) per loader and stage
  constexpr int XQ = TM * BLK / 1024 / LW;  // activation pieces per loader and stage
  constexpr int PER = pfw_per_stage(JM, NT);
  static_assert(PER == WQ + XQ + 1 && TM * BLK % (1024 * LW) == 0, "equal loads per loader");
  static_assert(TM * 4 == 256 * JM && JM <= LW, "at most one 256-byte scale piece per loader");
  constexpr int WCOLS = 16 * NT;         // output columns of a wave
  constexpr int XOFF = PFW_TILE_N * BLK;  // activation rows within a stage
  constexpr int SOFF = XOFF + TM * BLK;   // activation scales within a stage
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave & 1, wm = wave >> 1;
  const int n0 = work.n0, m0 = work.m0;
  const int l16 = lane & 15, g = lane >> 4;
  const int kb0 = work.kb0, last = work.kb1 - 1;
  // a whole tile holds two weight blocks, one per wave column; a half tile
  // one; a narrow tile's wave column (80 columns from any multiple of 16)
  // lies in one block or straddles two (nbw, nbw1: the block of its first
  // and of its last column)
  const int nbw = NT == 5 ? (n0 + WCOLS * wn) / BLK : n0 / BLK + (NT == 8 ? wn : 0);
  const float* wsrow = p.ws + (size_t)nbw * (size_t)p.kbn;
  const int nbw1 = NT == 5 ? (n0 + WCOLS * wn + WCOLS - 1) / BLK : nbw;
  const float* wsrow1 = p.ws + (size_t)nbw1 * (size_t)p.kbn;
  const uint32_t lds0 = lds_addr(lds_all);

  // Loader wave w < LW copies pieces q = w + LW i of the stage's weight rows
  // (1 KB: rows 8q .. 8q+7, or half q % 2 of 2 KB tile q / 2) and of its
  // activation rows, and scale piece w (rows 64 w ..; with JM = 3 pieces,
  // loader 3 loads piece 2 again, the same bytes). Every piece q a
  // loader takes has q % 2 = w % 2, so one lane offset serves all of them:
  // row 8q + lane / 8, 16-byte segment (lane % 8) ^ (lane / 8) ^ (q % 2)
  // (the swizzle of pf_swz); the rest of each weight offset is uniform and
  // goes into the scalar base. Activation rows past m (last m tile) are
  // clamped per lane.
  const uint32_t xseg = 16u * (uint32_t)((lane & 7) ^ (lane >> 3) ^ (wave & 1));
  const uint32_t wlo = PK ? 16u * (uint32_t)lane : (uint32_t)(lane >> 3) * (uint32_t)p.k + xseg;
  const int xlim = p.m - 1 - m0;  // last activation row of the tile
  const int sq = wave < JM ? wave : JM - 1;  // scale piece of this loader
  const int sr = 64 * sq + lane;
  const uint32_t so = (uint32_t)(sr <= xlim ? sr : xlim) * (uint32_t)p.kbn * 4u;
  const uint8_t* wbase = PK ? p.wq + (size_t)(n0 >> 4) * (size_t)p.kbn * 2048u
                            : p.wq + (size_t)n0 * (size_t)p.k;
  const uint8_t* xbase = p.xq + (size_t)m0 * (size_t)p.k;
  const float* sbase = p.xs + (size_t)m0 * (size_t)p.kbn;

  // The loads of block kb into a stage, by the loaders (LOADER: this wave
  // is one; the kernel runs this function in two copies, so neither has a
  // branch in its loop): WQ weight pieces, XQ activation pieces, the scale
  // piece (PER in all). The other waves load nothing, so only the loaders
  // can stall on a full memory queue, and on every SIMD the other wave keeps
  // the matrix core busy meanwhile.
  auto issue = [&](int kb, int stage) {
    if constexpr (LOADER) {
      kb = kb < last ? kb : last;
      const uint32_t st = lds0 + (uint32_t)(stage * STAGE);
      const uint8_t* wb = wbase + (size_t)kb * (PK ? 2048u : (size_t)BLK);
      const uint8_t* xb = xbase + (size_t)kb * BLK;
#pragma unroll
      for (int i = 0; i < WQ; ++i) {
        const int q = wave + LW * i;
        const size_t off = PK ? (size_t)(q >> 1) * (size_t)p.kbn * 2048u + (size_t)(q & 1) * 1024u
                              : (size_t)(8 * q) * (size_t)p.k;
        dma16(st + (uint32_t)q * 1024u, wb + off, wlo);
      }
      // the clamped offsets are recomputed per block (a few VALU operations)
      // rather than held in registers across the loop
      int lr = lane >> 3;
      asm volatile("" : "+v"(lr));
#pragma unroll
      for (int i = 0; i < XQ; ++i) {
        const int q = wave + LW * i;
        const int r = 8 * q + lr;
        const uint32_t off = (uint32_t)(r <= xlim ? r : xlim) * (uint32_t)p.k + xseg;
        dma16(st + (uint32_t)XOFF + (uint32_t)q * 1024u, xb, off);
      }
      dma4(st + (uint32_t)SOFF + (uint32_t)sq * 256u, sbase + kb, so);
    }
  };

  f32x4 acc[NT][JM];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int j = 0; j < JM; ++j) acc[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // The activation operands and the scale products of block kb, from its
  // stage. Narrow tiles keep the activation scales and both weight scales
  // of the wave column, and form each subtile's products where it is
  // rescaled (the same fp32 product sa * sw).
  i32x8 bop[JM];
  float sc[JM];
  float sw0 = 0.0f, sw1 = 0.0f;
  auto read_x = [&](const uint8_t* st) {
#pragma unroll
    for (int j = 0; j < JM; ++j) bop[j] = pf_swz_operand(st + XOFF, WR * wm + 16 * j + l16, g);
  };
  auto read_sc = [&](int kb, const uint8_t* st) {
    const float* sl = reinterpret_cast<const float*>(st + SOFF);
    if constexpr (NT == 5) {
      sw0 = load_invariant(wsrow, (size_t)kb);
      sw1 = load_invariant(wsrow1, (size_t)kb);
#pragma unroll
      for (int j = 0; j < JM; ++j) sc[j] = sl[WR * wm + 16 * j + l16];
    } else {
      const float sw = load_invariant(wsrow, (size_t)kb);
#pragma unroll
      for (int j = 0; j < JM; ++j) sc[j] = sl[WR * wm + 16 * j + l16] * sw;
    }
  };
  // the scale product of subtile T and activation subtile j
  auto scale = [&](int T, int j) {
    if constexpr (NT == 5) {
      const bool first = (n0 + WCOLS * wn + 16 * T) / BLK == nbw;  // wave-uniform
      return sc[j] * (first ? sw0 : sw1);
    } else {
      return sc[j];
    }
  };

  // S - 1 stages in flight (block kb0 + S - 1 is loaded during block kb0),
  // then the first block's activation operands
#pragma unroll
  for (int s = 0; s < S - 1; ++s) issue(kb0 + s, s);
  wait_loads_then_barrier<(S - 2) * PER>();
  read_x(lds_all);
  read_sc(kb0, lds_all);

  // One K block out of stage ST (a compile-time ring position). The wait
  // and barrier that publish the next block's stage and free this one come
  // after this block's last LDS read and last MFMA issue, so the matrix
  // cores still work on the last products while the waves meet, refill the
  // stage with the block S ahead and read the next block's activations.
  // One K block out of stage ST (a compile-time ring position). The loads
  // of block kb + S - 1 go into the stage the last barrier freed. The wait
  // and barrier that publish the next block's
  // stage and free this one come after this block's last LDS read and last
  // MFMA issue, so the matrix cores still work on the last products while
  // the waves meet and read the next block's activations.
  auto block = [&](int kb, auto stc) {
    constexpr int ST = decltype(stc)::value;
    constexpr int SP = (ST + S - 1) % S;
    const uint8_t* wl = lds_all + ST * STAGE;
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    f32x4 pb[2][JM];
    auto sub = [&](auto tc) {
      constexpr int T = decltype(tc)::value;
      if constexpr (T == 0) issue(kb + S - 1, SP);
      const i32x8 aop = PK ? pf_tile_operand(wl, NT * wn + T, lane)
                           : pf_swz_operand(wl, WCOLS * wn + 16 * T + l16, g);
#pragma unroll
      for (int j = 0; j < JM; ++j)
        pb[T & 1][j] =
            __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop, bop[j], z, 0, 0, 0, 0, 0, 0);
      if constexpr (T > 0) {
#pragma unroll
        for (int j = 0; j < JM; ++j) {
          const float sj = scale(T - 1, j);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[T - 1][j][i] = __builtin_fmaf(pb[(T - 1) & 1][j][i], sj, acc[T - 1][j][i]);
        }
      }
    };
    pf_static_for<0, NT>(sub);
    wait_loads_then_barrier<(S - 2) * PER>();
    const uint8_t* next = lds_all + ((ST + 1) % S) * STAGE;
    read_x(next);
#pragma unroll
    for (int j = 0; j < JM; ++j) {
      const float sj = scale(NT - 1, j);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[NT - 1][j][i] = __builtin_fmaf(pb[(NT - 1) & 1][j][i], sj, acc[NT - 1][j][i]);
    }
    read_sc(kb + 1 < last ? kb + 1 : last, next);
  };

  int kb = kb0;
  for (; kb + S - 1 <= last; kb += S) pf_ring_turn<0, S>(kb, block);
  pf_ring_tail<0, S>(kb, last, block);
  // every load of this wave has landed; after the barrier, every load and
  // every operand read of the workgroup is done and the LDS is free
  asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
  lds_barrier();

  if (p.out == OUT_PARTIAL) {
#pragma unroll
    for (int j = 0; j < JM; ++j) {
      const int m = m0 + WR * wm + 16 * j + l16;
      if (m < p.m) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const int n = n0 + WCOLS * wn + 16 * t + 4 * g;
          *reinterpret_cast<float4*>(p.part + ((size_t)blockIdx.z * p.m + m) * (size_t)p.n + n) =
              make_float4(acc[t][j][0], acc[t][j][1], acc[t][j][2], acc[t][j][3]);
        }
      }
    }
    return;
  }
  // bf16 output: each wave stages its WR x WCOLS part in its own LDS
  // (row r: 2 WCOLS bytes in U = 2 NT 16-byte units, unit u at
  // u ^ (r mod U), or (u + r) mod U when U is not a power of two, so both
  // the 8-byte writes of 16 rows and the 16-byte reads of whole rows spread
  // over the banks), then writes whole row segments of 2 WCOLS bytes, 1 KB
  // per store instruction (lane l of instruction i: unit 64 i + l of the
  // wave's WR U units, row by row), instead of 32-byte pieces of 16 rows.
  constexpr int U = 2 * NT;  // 16-byte units per staged row
  auto slot = [](int u, int r) {
    if constexpr ((U & (U - 1)) == 0)
      return u ^ (r % U);
    else
      return (u + r) % U;
  };
  uint8_t* ob = lds_all + wave * (WR * 16 * U);
#pragma unroll
  for (int j = 0; j < JM; ++j) {
    const int r = 16 * j + l16;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int u = 2 * t + (g >> 1);
      *reinterpret_cast<uint2*>(ob + r * 16 * U + 16 * slot(u, r) + 8 * (g & 1)) =
          make_uint2(pack_bf16x2(acc[t][j][0], acc[t][j][1]),
                     pack_bf16x2(acc[t][j][2], acc[t][j][3]));
    }
  }
  // the wave reads back only what it wrote itself (LDS accesses of one wave
  // complete in order)
#pragma unroll
  for (int i = 0; i < (WR * U + 63) / 64; ++i) {
    const int f = 64 * i + lane;
    const int r = f / U, u = f - (f / U) * U;
    const int m = m0 + WR * wm + r;
    if (f < WR * U) {
      const uint4 v = *reinterpret_cast<const uint4*>(ob + r * 16 * U + 16 * slot(u, r));
      if (m < p.m) {
        typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
        __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w},
                                    reinterpret_cast<u32x4*>(p.y + (size_t)m * (size_t)p.n + n0 +
                                                             WCOLS * wn + 8 * u));
      }
    }
  }
}

// pfw_lds_bytes(JM, S) of dynamic LDS; 512 threads (8 waves: 4 along m,
// 2 along n); grid as pfw_work, or (TW = 160, narrow tiles) pfw_work_narrow.
template <int JM, int S, bool PK = false, int TW = PFW_TILE_N>
__global__ __launch_bounds__(512, 1) void gemm_prefill_wide_kernel(GemmParams p) {
  static_assert(JM == 3 || JM == 4, "48 or 64 activation rows per wave");
  static_assert(TW == PFW_TILE_N || TW == PFW_NARROW_N, "256- or 160-column tiles");
  static_assert(8 * 16 * JM * 256 <= pfw_lds_bytes(JM, S), "output staging fits in the stages");
  static_assert(S >= 2 && (S - 1) * pfw_per_stage(JM, 8) <= 63, "vmcnt range");
  extern __shared__ __align__(16) uint8_t lds_all[];
  const bool loader = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) < PFW_LOADERS;
  if constexpr (TW == PFW_NARROW_N) {
    const PfwWork work = pfw_work_narrow<pfw_tile_m(JM)>(p);
    if (loader)
      pfw_unit<JM, S, PK, 5, true>(p, lds_all, work);
    else
      pfw_unit<JM, S, PK, 5, false>(p, lds_all, work);
    return;
  }
  const PfwWork work = pfw_work<pfw_tile_m(JM)>(p);
  if (work.n0 >= p.n) return;  // the empty second half of a one-block tile
  if (work.half) {
    if (loader)
      pfw_unit<JM, S, PK, 4, true>(p, lds_all, work);
    else
      pfw_unit<JM, S, PK, 4, false>(p, lds_all, work);
  } else {
    if (loader)
      pfw_unit<JM, S, PK, 8, true>(p, lds_all, work);
    else
      pfw_unit<JM, S, PK, 8, false>(p, lds_all, work);
  }
}

}  // namespace fp8bs
