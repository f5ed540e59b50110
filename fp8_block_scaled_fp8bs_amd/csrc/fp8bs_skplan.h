// Work partition of the stream-K decode GEMM, shared by the kernel and the
// host (launch checks, workspace size, and the plan self-check that the
// C ABI exposes for tests). Plain integer arithmetic only.
//
// The product is streamed as (16-row weight tile, 128-deep K block) units.
// The pages' kernel splits the long K dimension across the compute units and
// reduces the partial results in a fixed order ("A 23% faster GPU kernel,
// and a model that did not move", section "Why this shape is hard"). Here a
// fixed number P of workgroups (one per compute unit of a full MI355X) each
// take an equal share of the units:
//
//   * K is cut into S chunks of kc = kbn / S blocks. A cell is one tile over
//     one chunk: cell z = c * ntiles + t (chunk-major), kc units.
//   * Data-parallel part: R = floor(C / P) whole cells per workgroup
//     (C = ntiles * S cells), workgroup w taking cells w*R .. w*R + R - 1.
//   * Stream-K part: the remaining C - R*P cells, laid end to end as units,
//     are split evenly: workgroup w takes units [Usk*w/P, Usk*(w+1)/P).
//     A cell of this part may be shared by several workgroups.
//   * Whole-cell mode (S = 1 only): no stream-K part; workgroup w takes the
//     whole cells [C*w/P, C*(w+1)/P), so the counts differ by at most one
//     cell and no tile is ever cut. Where the cells do not divide evenly, a
//     few workgroups stream one more tile than the rest, in exchange for no
//     hand-off between workgroups at all.
//
// Each maximal run of a workgroup's units inside one cell is a segment. The
// fp32 sum of a segment is a "piece" of its tile's output. A tile whose only
// piece is a whole cell with S = 1 is written directly; the pieces of every
// other tile go to the workspace and are added in a fixed order -- chunk c
// ascending, then the workgroups sharing a cell in K order -- by whichever
// contributing workgroup arrives last, so the bits never depend on timing.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define FP8BS_HD __host__ __device__
#else
#define FP8BS_HD
#endif

namespace fp8bs {

constexpr int SK_MAXSK = 4;       // stream-K segments of one workgroup, at most
constexpr int SK_MAXPIECES = 8;   // pieces of one tile, at most

struct SkPlan {
  int ntiles;   // n / 16
  int kbn;      // K blocks
  int S;        // K chunks
  int kc;       // blocks per chunk
  int P;        // workgroups
  int R;        // whole cells per workgroup (data-parallel part)
  int64_t C;    // cells
  int64_t Usk;  // units of the stream-K part
  int64_t dp_slots;  // workspace piece slots of data-parallel cells (S > 1)
  int whole;         // whole-cell mode
};

FP8BS_HD inline SkPlan sk_plan(int ntiles, int kbn, int S, int P, int whole = 0) {
  SkPlan q;
  q.whole = whole;
  q.ntiles = ntiles;
  q.kbn = kbn;
  q.S = S;
  q.kc = S > 0 ? kbn / S : 0;
  q.P = P;
  q.C = (int64_t)ntiles * S;
  q.R = P > 0 ? (int)(q.C / P) : 0;
  q.Usk = whole ? 0 : (q.C - (int64_t)q.R * P) * q.kc;
  q.dp_slots = S > 1 ? (int64_t)q.R * P : 0;
  return q;
}

// Whole cells of workgroup w: [*c0, *c0 + count).
FP8BS_HD inline int sk_cells(const SkPlan& q, int w, int* c0) {
  if (q.whole) {
    const int a = (int)(q.C * w / q.P), b = (int)(q.C * (w + 1) / q.P);
    *c0 = a;
    return b - a;
  }
  *c0 = w * q.R;
  return q.R;
}

// First stream-K unit of workgroup w (w = P gives the end).
FP8BS_HD inline int64_t sk_begin(const SkPlan& q, int w) { return q.Usk * w / q.P; }

// The workgroup whose stream-K units contain unit u (0 <= u < Usk).
FP8BS_HD inline int sk_owner(const SkPlan& q, int64_t u) {
  return (int)(((u + 1) * q.P - 1) / q.Usk);
}

// Workspace slot of the piece of stream-K cell zz (index within the
// stream-K part) computed by workgroup w.
FP8BS_HD inline int64_t sk_slot(const SkPlan& q, int w, int64_t zz) {
  return q.dp_slots + (int64_t)w * SK_MAXSK + (zz - sk_begin(q, w) / q.kc);
}

struct SkSegment {
  int tile;    // 16-row weight tile
  int chunk;   // K chunk: absolute K blocks chunk * kc + [b0, b1)
  int b0, b1;  // blocks within the chunk
  int64_t slot;  // workspace piece slot (if the tile is reduced)
};

// Segment i of workgroup w, in processing order: its stream-K segments
// first (their pieces reach the workspace early), then its whole cells.
// Returns the number of stream-K segments in *nsk and the total count.
FP8BS_HD inline int sk_segments(const SkPlan& q, int w, int* nsk) {
  int n = 0;
  if (q.Usk > 0) {
    const int64_t ua = sk_begin(q, w), ub = sk_begin(q, w + 1);
    n = ub > ua ? (int)((ub - 1) / q.kc - ua / q.kc + 1) : 0;
  }
  *nsk = n;
  int c0;
  return n + sk_cells(q, w, &c0);
}

FP8BS_HD inline SkSegment sk_segment(const SkPlan& q, int w, int nsk, int i) {
  SkSegment s;
  if (i < nsk) {
    const int64_t ua = sk_begin(q, w), ub = sk_begin(q, w + 1);
    const int64_t zz = ua / q.kc + i;
    const int64_t lo = zz * q.kc > ua ? zz * q.kc : ua;
    const int64_t hi = zz * q.kc + q.kc < ub ? zz * q.kc + q.kc : ub;
    const int64_t z = (int64_t)q.R * q.P + zz;
    s.tile = (int)(z % q.ntiles);
    s.chunk = (int)(z / q.ntiles);
    s.b0 = (int)(lo - zz * q.kc);
    s.b1 = (int)(hi - zz * q.kc);
    s.slot = sk_slot(q, w, zz);
  } else {
    // C < 2^31 in a valid plan: 32-bit arithmetic
    int c0;
    sk_cells(q, w, &c0);
    const int z = c0 + (i - nsk);
    s.tile = z % q.ntiles;
    s.chunk = z / q.ntiles;
    s.b0 = 0;
    s.b1 = q.kc;
    s.slot = q.S > 1 ? z : -1;  // with S = 1 a whole cell is a whole tile, written directly
  }
  return s;
}

// The pieces of tile t in summation order: their workspace slots (up to
// SK_MAXPIECES; the count is returned even when it exceeds that).
FP8BS_HD inline int sk_tile_pieces(const SkPlan& q, int t, int64_t* slots) {
  int np = 0;
  for (int c = 0; c < q.S; ++c) {
    const int64_t z = (int64_t)c * q.ntiles + t;
    if (q.whole || z < (int64_t)q.R * q.P) {
      if (np < SK_MAXPIECES) slots[np] = q.S > 1 ? z : -1;  // S = 1: the whole tile, no slot
      ++np;
    } else {
      const int64_t zz = z - (int64_t)q.R * q.P;
      const int w0 = sk_owner(q, zz * q.kc), w1 = sk_owner(q, zz * q.kc + q.kc - 1);
      for (int w = w0; w <= w1; ++w) {
        if (np < SK_MAXPIECES) slots[np] = sk_slot(q, w, zz);
        ++np;
      }
    }
  }
  return np;
}

// K blocks a workgroup stages activations for: the chunks of its cells.
// Valid plans keep every workgroup inside one chunk (S = 1, or whole cells
// only with R dividing ntiles), so this is one chunk: [chunk * kc, +kc).
FP8BS_HD inline int sk_chunk_of(const SkPlan& q, int w) {
  int nsk;
  sk_segments(q, w, &nsk);
  return sk_segment(q, w, nsk, 0).chunk;
}

// Whether the plan is one the kernel supports: S divides kbn; with S = 1 at
// most SK_MAXSK stream-K segments per workgroup; with S > 1 no stream-K
// part and each workgroup's cells inside one chunk; every tile at most
// SK_MAXPIECES pieces; at least one segment per workgroup.
FP8BS_HD inline bool sk_plan_ok(const SkPlan& q) {
  if (q.S < 1 || q.P < 1 || q.kbn < 1 || q.ntiles < 1 || q.kbn % q.S) return false;
  if (q.C >= ((int64_t)1 << 31) || q.C * q.P >= ((int64_t)1 << 62)) return false;
  if (q.whole) return q.S == 1 && q.C >= q.P;
  if (q.S > SK_MAXPIECES) return false;
  if (q.S > 1 && (q.Usk != 0 || q.R < 1 || q.ntiles % q.R)) return false;
  if (q.Usk > 0) {
    // longest stream-K run, and the pieces a stream-K cell can be cut into
    const int64_t lmax = (q.Usk + q.P - 1) / q.P;
    const int64_t lmin = q.Usk / q.P;
    if (lmin < 1) return false;
    if ((lmax + q.kc - 1) / q.kc + 1 > SK_MAXSK) return false;
    if ((q.kc + lmin - 1) / lmin + 1 > SK_MAXPIECES) return false;
  } else if (q.R < 1) {
    return false;
  }
  return true;
}

}  // namespace fp8bs
