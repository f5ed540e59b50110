// Stream-K decode GEMM: every compute unit streams an equal share of the
// weight units in one launch, whatever the number of 16-row tiles.
//
// The work partition (fp8bs_skplan.h) gives P = 256 workgroups equal runs of
// (16-row tile, 128-deep K block) units. Where the tiles do not divide
// evenly among the workgroups, a few tiles are cut into pieces computed by
// different workgroups; the pieces of such a tile are added in a fixed
// order by the workgroup that completes the set, so the result is
// deterministic ("A 23% faster GPU kernel, and a model that did not move",
// section "Why this shape is hard": split the long dimension across the
// units and reduce deterministically; there the units were an H100's SMs).
//
// A workgroup has WK streaming waves and one output wave:
//   * The streaming waves interleave the K blocks of each segment (wave wk
//     takes blocks b0 + wk, b0 + wk + WK, ...), keeping D weight tiles in
//     flight per wave across segment ends, and run one FP8 MFMA per tile and
//     block with the per-block fp32 rescale. They never store to global
//     memory or wait on anything but their own loads: at the end of a
//     segment each writes its fp32 partial to an LDS buffer and bumps that
//     buffer's arrival count.
//   * The output wave waits for the WK partials of each segment, adds them
//     in wave order, and either writes the bf16 outputs (a tile with one
//     piece) or stores the piece to the workspace and arrives on the tile's
//     counter; the arrival that completes the count adds all the tile's
//     pieces in plan order and writes the bf16 outputs. Its stores, waits
//     and counter updates therefore never hold up the weight stream (the
//     wait counter of a wave covers loads and stores alike).
// Each workgroup computes its pieces first, so the cross-workgroup additions
// happen while the rest of the weights stream in.
//
// Cross-workgroup hand-off (the protocol of the split-K helpers in
// fp8bs_gemm.h): the 8 XCDs have separate L2 caches, so a piece is written
// with device-coherent stores (agent-scope atomic stores, which write
// through the writer's L2), the output wave waits until its own stores are
// performed (on this architecture the vmcnt counter covers stores), and
// only then arrives: an agent-scope integer read-modify-write on the tile's
// counter. The arrival that completes the count reads the pieces with
// device-coherent loads, which are not served from a stale line of its own
// L2. No cache-wide write-back or invalidate is issued: with agent-scope
// release/acquire fences around the arrival instead (an L2 write-back and
// an L2 invalidate each time), this kernel took 18.5 us for the square
// projection at m = 8 on MI355X, 2.4x the grid kernel, and 50 us for the
// MLP down projection, whose workgroups arrive five times each. The counter carries a per-launch epoch (see arrive()), so it
// needs no initialization and is left at zero for graph replays.
#pragma once

#include "fp8bs_gemm.h"
#include "fp8bs_skplan.h"

namespace fp8bs {

constexpr int SK_NBUF = 4;  // LDS partial-sum buffers between streaming and output waves

// The hand-off between the waves of one workgroup goes through LDS only.
// LDS performs each wave's operations in issue order, so a data write
// issued before a counter update is visible to any wave that has read the
// updated counter; the accesses only must not be reordered by the compiler
// (a signal fence), and need no hardware wait. The counters are addressed
// as LDS so that their atomics are LDS instructions: on a generic address
// an atomic would also wait for the wave's outstanding weight loads.
typedef __attribute__((address_space(3))) int lds_int;

__device__ __forceinline__ void lds_signal_add(lds_int* c) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __hip_atomic_fetch_add(c, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_signal_set(lds_int* c, int v) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __hip_atomic_store(c, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_wait_at_least(lds_int* c, int target) {
  while (__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < target)
    __builtin_amdgcn_s_sleep(1);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Dynamic LDS: staged activations of one chunk (codes + scales), then
// SK_NBUF buffers of WK wave partials.
__host__ __device__ inline int lds_streamk_bytes(int kc, int m, int wk, int mt) {
  return lds_act_bytes(kc, m) + SK_NBUF * wk * mt * 64 * 16;
}

// Workspace: piece slots of MT KB each, then one 64-bit counter per tile.
__host__ __device__ inline int64_t sk_slot_count(const SkPlan& q) {
  return q.dp_slots + (int64_t)q.P * SK_MAXSK;
}
__host__ __device__ inline int64_t sk_workspace_bytes(const SkPlan& q, int mt) {
  if (q.whole && q.S == 1) return 0;  // no tile is cut: no pieces, no counters
  return sk_slot_count(q) * mt * 1024 + (int64_t)q.ntiles * 8;
}

// Position in the item sequence of a streaming wave: item j of segment s.
struct SkCursor {
  int s, j, nj;     // segment, item within it, items of the segment per wave
  int tile, kbase;  // weight tile; first absolute K block of the chunk
  int b0, b1;       // blocks [b0, b1) of the chunk
};

template <int MT, int WK, int D, int PRE, bool FUSED, int CR, bool PK>
__device__ __forceinline__ void gemm_streamk_body(const GemmParams& p, uint8_t* lds_all,
                                                  lds_int* s_arrived, lds_int* s_consumed) {
  constexpr int NT = 64 * (WK + 1);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int M = p.m;
  const SkPlan q = sk_plan(p.n >> 4, p.kbn, p.split, (int)gridDim.x, p.sk_whole);
  const int w = blockIdx.x;
  int nsk;
  const int nseg = sk_segments(q, w, &nsk);
  const int kx0 = sk_chunk_of(q, w) * q.kc;  // staged activations: K blocks [kx0, kx0 + kc)
  const int nblk = q.kc;

  uint8_t* act = lds_all;
  float* act_s = reinterpret_cast<float*>(lds_all + nblk * M * ACT_STRIDE);
  f32x4* red = reinterpret_cast<f32x4*>(lds_all + lds_act_bytes(nblk, M));
  const int l16 = lane & 15, g16 = lane >> 4;
  const int l7 = lane & 7, hb = (lane >> 3) & 1;
  const bool lo8 = hb == 0;
  const bool streaming = wave < WK;

  if (tid == 0) {
#pragma unroll
    for (int b = 0; b < SK_NBUF; ++b) s_arrived[b] = 0;
    *s_consumed = 0;
  }

  // 1. activation loads first (the tail loop, if any, before anything else)
  stage_act_tail<NT, CR, FUSED>(p, kx0, nblk, tid, act, act_s);
  uint4 xr[CR][4];
  if constexpr (FUSED) load_act_quarters<NT, CR>(p, kx0, nblk * M * 4, tid, 0, xr);
  __builtin_amdgcn_sched_barrier(0);  // activation loads stay ahead of the weight loads

  // 2. weight stream of a streaming wave: items in segment order; blocks
  //    past a segment's end, and items past the last segment, load through
  //    an out-of-range buffer offset (zeros, no memory traffic), so every
  //    item issues the same loads and the wait counts stay exact.
  const __amdgpu_buffer_rsrc_t wr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.wq), (short)0,
                                        (int)((int64_t)p.n * p.k), 0x00020000);
  const int wk = streaming ? wave : 0;
  auto seg_at = [&](SkCursor& c) {
    if (c.s < nseg) {
      const SkSegment sg = sk_segment(q, w, nsk, c.s);
      c.tile = sg.tile;
      c.kbase = sg.chunk * q.kc;
      c.b0 = sg.b0;
      c.b1 = sg.b1;
      c.nj = (sg.b1 - sg.b0 + WK - 1) / WK;
    } else {
      c.tile = 0;
      c.kbase = 0;
      c.b0 = c.b1 = 0;
      c.nj = 1 << 30;
    }
  };
  auto advance = [&](SkCursor& c) {
    if (++c.j == c.nj) {
      c.j = 0;
      ++c.s;
      seg_at(c);
    }
  };
  SkCursor lc{0, 0, 0, 0, 0, 0, 0};
  seg_at(lc);
  TileLoad wb[D];
  auto load_next = [&](int d) {
    const int kb = lc.b0 + wk + lc.j * WK;  // block within the chunk
    const bool valid = lc.s < nseg && kb < lc.b1;
    const int ka = lc.kbase + kb;
    uint32_t op, oq;
    if constexpr (PK) {
      op = (uint32_t)(((uint32_t)lc.tile * (uint32_t)p.kbn + (uint32_t)ka) * 2048u +
                      (uint32_t)((16 * g16 + l16) * 16));
      oq = op + 1024u;
    } else {
      const uint32_t r0 = (uint32_t)(16 * lc.tile + l7);
      op = r0 * (uint32_t)p.k + (uint32_t)ka * BLK + 16u * (2 * g16 + hb);
      oq = (r0 + 8u) * (uint32_t)p.k + (uint32_t)ka * BLK + 16u * (2 * g16 + 1 - hb);
    }
    if (!valid) op = oq = BUF_OOB;
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(wr, op, 0, 2);  // nt: streamed once
    const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(wr, oq, 0, 2);
    wb[d].p = make_uint4(a.x, a.y, a.z, a.w);
    wb[d].q = make_uint4(b.x, b.y, b.z, b.w);
    advance(lc);
  };
  if (streaming) {
#pragma unroll
    for (int d = 0; d < PRE; ++d) load_next(d);
  }

  // 3. activations to LDS (every wave casts), then the rest of the prefetch
  stage_act<NT, CR, FUSED>(p, kx0, nblk, tid, xr, act, act_s);
  if (streaming) {
#pragma unroll
    for (int d = PRE; d < D; ++d) load_next(d);
  }
  lds_barrier();

  if (streaming) {
    // 4. stream: compute item i from slot i % D, then refill the slot
    SkCursor cc{0, 0, 0, 0, 0, 0, 0};
    seg_at(cc);
    // items per wave: the stream-K segments, then the whole cells
    int c0;
    int items = sk_cells(q, w, &c0) * ((q.kc + WK - 1) / WK);
    for (int s = 0; s < nsk; ++s) {
      const SkSegment sg = sk_segment(q, w, nsk, s);
      items += (sg.b1 - sg.b0 + WK - 1) / WK;
    }
    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](int d) {
      const int kb = cc.b0 + wk + cc.j * WK;
      if (kb < cc.b1) {
        const int ka = cc.kbase + kb;
        const float sw = load_invariant(p.ws, (size_t)(cc.tile >> 3) * (size_t)p.kbn + ka);
        const i32x8 aop = weight_operand<PK>(wb[d], lo8);
        const int kl = ka - kx0;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int m = l16 + 16 * mt;
          i32x8 bop = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
          float sa = 0.0f;
          if (m < M) {
            const uint8_t* a = act + (kl * M + m) * ACT_STRIDE + 32 * g16;
            const uint4 lo = *reinterpret_cast<const uint4*>(a);
            const uint4 hi = *reinterpret_cast<const uint4*>(a + 16);
            bop = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                        (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            sa = act_s[kl * M + m];
          }
          const f32x4 z = {0.f, 0.f, 0.f, 0.f};
          const f32x4 pb =
              __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop, bop, z, 0, 0, 0, 0, 0, 0);
          const float sc = sa * sw;
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[mt][i] = __builtin_fmaf(pb[i], sc, acc[mt][i]);
        }
      }
      if (cc.j == cc.nj - 1) {
        // end of segment cc.s: hand the partial to the output wave
        const int buf = cc.s % SK_NBUF;
        if (cc.s >= SK_NBUF) lds_wait_at_least(s_consumed, cc.s - SK_NBUF + 1);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          red[((buf * WK + wk) * MT + mt) * 64 + lane] = acc[mt];
          acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        if (lane == 0) lds_signal_add(&s_arrived[buf]);
      }
      advance(cc);
    };
    const int ngrp = (items + D - 1) / D;
    for (int g = 0; g + 1 < ngrp; ++g) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        compute(d);
        load_next(d);
      }
    }
#pragma unroll
    for (int d = 0; d < D; ++d)
      if ((ngrp - 1) * D + d < items) compute(d);
    return;
  }

  // 5. output wave
  const int64_t nslots = sk_slot_count(q);
  float* pieces = p.part;
  uint64_t* counters = reinterpret_cast<uint64_t*>(pieces + nslots * MT * 256);
  auto store_out = [&](int tile, const f32x4 (&v)[MT]) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = l16 + 16 * mt;
      if (m < M) {
        uint2* dst = reinterpret_cast<uint2*>(p.y + (size_t)m * (size_t)p.n + 16 * tile + 4 * g16);
        *dst = make_uint2(pack_bf16x2(v[mt][0], v[mt][1]), pack_bf16x2(v[mt][2], v[mt][3]));
      }
    }
  };
  for (int s = 0; s < nseg; ++s) {
    const int buf = s % SK_NBUF;
    const int target = WK * (s / SK_NBUF + 1);
    lds_wait_at_least(&s_arrived[buf], target);
    f32x4 v[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      v[mt] = red[((buf * WK) * MT + mt) * 64 + lane];
      for (int k = 1; k < WK; ++k) v[mt] += red[((buf * WK + k) * MT + mt) * 64 + lane];
    }
    if (lane == 0) lds_signal_set(s_consumed, s + 1);
    const SkSegment sg = sk_segment(q, w, nsk, s);
    int64_t slots[SK_MAXPIECES];
    const int np = sk_tile_pieces(q, sg.tile, slots);
    if (np == 1) {
      store_out(sg.tile, v);
      continue;
    }
    // a piece: to the workspace with device-coherent stores, then arrive on
    // the tile's counter once they are performed
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      float* dst = pieces + ((sg.slot * MT + mt) * 64 + lane) * 4;
      store_coherent64(dst, (uint64_t)__float_as_uint(v[mt][0]) |
                                ((uint64_t)__float_as_uint(v[mt][1]) << 32));
      store_coherent64(dst + 2, (uint64_t)__float_as_uint(v[mt][2]) |
                                    ((uint64_t)__float_as_uint(v[mt][3]) << 32));
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    int last = 0;
    if (lane == 0) last = arrive(counters + sg.tile, p.epoch, (uint64_t)np) ? 1 : 0;
    last = __builtin_amdgcn_readfirstlane(last);
    if (!last) continue;
    // every piece of the tile requested at once (coherent loads; slots past
    // the count read the first piece again and are not added), then added
    // in plan order
    uint64_t pv[SK_MAXPIECES][MT][2];
#pragma unroll
    for (int i = 0; i < SK_MAXPIECES; ++i)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const float* src = pieces + (((i < np ? slots[i] : slots[0]) * MT + mt) * 64 + lane) * 4;
        pv[i][mt][0] = load_coherent64(src);
        pv[i][mt][1] = load_coherent64(src + 2);
      }
    f32x4 sum[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int i = 0; i < SK_MAXPIECES; ++i) {
        const f32x4 e = {__uint_as_float((uint32_t)pv[i][mt][0]),
                         __uint_as_float((uint32_t)(pv[i][mt][0] >> 32)),
                         __uint_as_float((uint32_t)pv[i][mt][1]),
                         __uint_as_float((uint32_t)(pv[i][mt][1] >> 32))};
        if (i == 0)
          sum[mt] = e;
        else if (i < np)
          sum[mt] += e;
      }
    }
    store_out(sg.tile, sum);
  }
}

template <int MT, int WK, int D, int PRE, bool FUSED, bool PK>
__global__ __launch_bounds__(64 * (WK + 1)) void gemm_streamk_kernel(GemmParams p) {
  extern __shared__ __align__(16) uint8_t lds_all[];
  __shared__ int s_flags[SK_NBUF + 1];  // arrivals per buffer, then segments consumed
  lds_int* s_arrived = (lds_int*)s_flags;
  lds_int* s_consumed = s_arrived + SK_NBUF;
  if constexpr (FUSED) {
    // one body with three activation-load rounds: the path is selected only
    // explicitly, so it is not specialised per size like the table's kernels
    gemm_streamk_body<MT, WK, D, PRE, true, 3, PK>(p, lds_all, s_arrived, s_consumed);
  } else {
    gemm_streamk_body<MT, WK, D, PRE, false, 1, PK>(p, lds_all, s_arrived, s_consumed);
  }
}

}  // namespace fp8bs
