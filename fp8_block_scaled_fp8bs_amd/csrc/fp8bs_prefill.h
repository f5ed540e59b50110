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

}  // namespace fp8bs
