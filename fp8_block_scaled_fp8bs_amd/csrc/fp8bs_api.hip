// C ABI of the library: argument checks, the fixed configuration table,
// kernel launches and launch counters. Every kernel runs on the caller's
// stream; nothing here allocates, frees or synchronizes.
#include <algorithm>
#include <atomic>
#include <cstring>
#include <mutex>
#include <vector>

#include "fp8bs.h"
#include "fp8bs_diag.h"
#include "fp8bs_prefill.h"
#include "fp8bs_quant.h"
#include "fp8bs_reduce.h"
#include "fp8bs_registry.h"
#include "fp8bs_streamk.h"

using namespace fp8bs;

namespace {

std::atomic<uint64_t> g_counts[9];
std::atomic<uint64_t> g_epoch{1};  // launch tags for the last-arriver counters (never 0)

enum {
  CNT_QW = 0, CNT_QA = 1, CNT_MFMA = 2, CNT_DOT = 3, CNT_RED = 4, CNT_ENC = 5, CNT_DIAG = 6,
  CNT_SWIGLU = 7, CNT_PACK = 8
};

constexpr int kMaxDevices = 64;
struct DeviceInfo {
  bool checked = false;
  bool ok = false;
  int max_lds = 0;
  int num_cu = 0;
  int index = 0;
};
DeviceInfo g_dev[kMaxDevices];
std::mutex g_dev_mu;

// The current device must be a gfx950. Result cached per device.
fp8bs_status current_device(DeviceInfo* out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return FP8BS_ERR_DEVICE;
  }
  std::lock_guard<std::mutex> lk(g_dev_mu);
  DeviceInfo& d = g_dev[dev];
  if (!d.checked) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return FP8BS_ERR_DEVICE;
    }
    d.ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    d.index = dev;
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess)
      d.max_lds = v;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
      d.num_cu = v;
    d.checked = true;
  }
  if (!d.ok) return FP8BS_ERR_DEVICE;
  if (out) *out = d;
  return FP8BS_OK;
}

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Kernels that take more than 64 KB of dynamic LDS need the per-function
// limit raised once per device: to the device maximum less the kernel's
// static LDS. A bit per device records that it was done, so a launch pays
// for it only the first time.
constexpr int kMaxKernels = 4096;
std::atomic<uint64_t> g_lds_raised[kMaxKernels];

fp8bs_status raise_lds_limit(const void* fn, int slot, const DeviceInfo& dev, size_t need) {
  if (slot < 0 || slot >= kMaxKernels) return FP8BS_ERR_LAUNCH;
  const uint64_t bit = uint64_t(1) << dev.index;
  if (g_lds_raised[slot].load(std::memory_order_acquire) & bit) return FP8BS_OK;
  hipFuncAttributes attr;
  if (hipFuncGetAttributes(&attr, fn) != hipSuccess) {
    (void)hipGetLastError();
    return FP8BS_ERR_LAUNCH;
  }
  const int limit = dev.max_lds - (int)attr.sharedSizeBytes;
  if (limit < (int)need) return FP8BS_ERR_CONFIG;
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, limit) != hipSuccess) {
    (void)hipGetLastError();
    return FP8BS_ERR_LAUNCH;
  }
  g_lds_raised[slot].fetch_or(bit, std::memory_order_acq_rel);
  return FP8BS_OK;
}

fp8bs_status launch(const void* fn, dim3 grid, dim3 block, size_t lds, void* stream, void** args) {
  const hipError_t e = hipLaunchKernel(fn, grid, block, args, lds, as_stream(stream));
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return FP8BS_ERR_LAUNCH;
  }
  return FP8BS_OK;
}

// ----------------------------------------------------------- GEMM configs ---

// Fixed device scratch of fp8bs_gemm_noalloc: every GPU the library runs on
// holds its own copy from load until the process ends. Host code never uses
// the array's name as an address: its device address is looked up once per
// device (hipGetSymbolAddress, with that device current) and kept.
constexpr size_t kNoAllocScratchBytes = (size_t)8 << 20;

}  // namespace

namespace fp8bs {
__device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];
}  // namespace fp8bs

namespace {

void* g_scratch_ptr[kMaxDevices];
bool g_scratch_ok[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of this device's scratch (nullptr on failure).
void* scratch_address(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ok[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
    g_scratch_ok[dev] = true;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

namespace fp8bs {
std::vector<KernelEntry>& kernel_registry() {
  static std::vector<KernelEntry> r;
  return r;
}
}  // namespace fp8bs

namespace {

constexpr int64_t kMaxDecodeM = 32;       // activation rows of the decode kernels (paths 1-4, 6)
constexpr int64_t kMaxM = (int64_t)1 << 20;  // activation rows of the prefill path
// Compute units the configuration table, the row-range split and the
// stream-K partition assume (a full MI355X). Launch geometry never depends on
// the device's own count, so a shape runs the same kernel with the same
// work split, and gives the same bits, on a partitioned device too (more
// rounds of workgroups there).
constexpr int kTableCUs = 256;

// Row-range paths: one workgroup per compute unit, n split over them.
inline bool is_row_range(int path) {
  return path == FP8BS_PATH_MFMA_ROWS || path == FP8BS_PATH_MFMA_STREAM ||
         path == FP8BS_PATH_MFMA_ROWS_REG || path == FP8BS_PATH_MFMA_ROWS_DMA;
}

// The streaming kernel addresses activations with 32-bit buffer offsets
// and marks unused fetches with offset 2^31: every byte offset of the bf16
// activations must stay below that.
inline bool stream_offsets_fit(int64_t m, int64_t k) { return m * k * 2 < ((int64_t)1 << 31); }

// The register-activation row-range kernel holds depth K blocks per wave:
// the K range must fit in waves_k * depth blocks, without a split.
inline bool rows_reg_fits(const fp8bs_gemm_config& c, int kbn) {
  return c.split_k == 1 && kbn <= c.waves_k * c.depth;
}

// swiglu: the row-range kernels instantiated with the SwiGLU epilogue.
const KernelEntry* find_kernel(const fp8bs_gemm_config& c, int m, bool fused,
                               bool swiglu = false) {
  int mt;
  if (c.path == FP8BS_PATH_MFMA || c.path == FP8BS_PATH_MFMA_ROWS ||
      c.path == FP8BS_PATH_MFMA_ROWS_REG) {
    mt = m <= 16 ? 1 : 2;
  } else if (c.path == FP8BS_PATH_MFMA_ROWS_DMA) {
    if (m > 16 || swiglu) return nullptr;
    mt = 1;
  } else if (c.path == FP8BS_PATH_MFMA_STREAMK) {
    if (swiglu) return nullptr;  // the epilogue runs in a second kernel
    mt = m <= 16 ? 1 : 2;
  } else if (c.path == FP8BS_PATH_MFMA_STREAM) {
    if (c.tiles_n != 1) return nullptr;
    mt = m <= 8 ? 1 : (m <= 16 ? 2 : 4);  // staging passes
  } else if (c.path == FP8BS_PATH_DOT) {
    if (m > 4) return nullptr;
    mt = m <= 1 ? 1 : (m <= 2 ? 2 : 4);
  } else if (c.path == FP8BS_PATH_PREFILL) {
    // one kernel; it reads activation codes (the fused call casts them first)
    for (const KernelEntry& e : kernel_registry())
      if (e.path == FP8BS_PATH_PREFILL && !swiglu && e.wn == c.waves_n && e.wk == c.waves_k &&
          e.d == c.depth && e.tn == c.tiles_n && e.layout == c.weight_layout)
        return &e;
    return nullptr;
  } else {
    return nullptr;
  }
  // waves_n is unused by the row-range paths and a partition mode of stream-K
  const bool rows = is_row_range(c.path);
  const bool any_wn = rows || c.path == FP8BS_PATH_MFMA_STREAMK;
  const int variant = rows ? (swiglu ? 1 : (c.split_k > 1 ? 2 : 0)) : 0;
  for (const KernelEntry& e : kernel_registry())
    if (e.path == c.path && e.mt == mt && e.tn == c.tiles_n && (any_wn || e.wn == c.waves_n) &&
        e.wk == c.waves_k && e.d == c.depth && e.fused == (int)fused && e.variant == variant &&
        e.layout == c.weight_layout)
      return &e;
  return nullptr;
}

// The wide prefill kernel, grid or 1-D schedule, whole or narrow tiles.
bool pfw_config(const fp8bs_gemm_config& c) {
  return c.path == FP8BS_PATH_PREFILL &&
         (c.tiles_n == PF_WIDE || c.tiles_n == PF_WIDE_1D || c.tiles_n == PF_WIDE_160);
}

// 1-D schedule of the wide prefill kernel (tiles_n PF_WIDE_1D): whole
// 256 x 256 tiles in complete rounds of kTableCUs workgroups; the tiles left
// over run as two 128-column halves each when those fit in half a round,
// else as whole tiles in a last, partly filled round.
struct PfwPlan {
  int64_t full, units;
};
PfwPlan pfw_plan(int waves_m, int64_t m, int64_t n) {
  const int64_t tm = pfw_tile_m(waves_m);
  const int64_t tiles = ((n + PFW_TILE_N - 1) / PFW_TILE_N) * ((m + tm - 1) / tm);
  PfwPlan q;
  q.full = tiles / kTableCUs * kTableCUs;
  const int64_t rem = tiles - q.full;
  if (rem > 0 && 2 * rem <= kTableCUs) {
    q.units = q.full + 2 * rem;
  } else {
    q.full = tiles;
    q.units = tiles;
  }
  return q;
}

// Narrow tiles (tiles_n PF_WIDE_160, n a multiple of 160): every tile is a
// unit of the 1-D grid.
PfwPlan pfw_plan_narrow(int waves_m, int64_t m, int64_t n) {
  const int64_t tm = pfw_tile_m(waves_m);
  PfwPlan q;
  q.full = (n / PFW_NARROW_N) * ((m + tm - 1) / tm);
  q.units = q.full;
  return q;
}

// Output columns per workgroup of a grid configuration (the row-range
// path divides n by the compute-unit count at launch instead).
int config_rows(const fp8bs_gemm_config& c) {
  if (is_row_range(c.path)) return 4;
  if (c.path == FP8BS_PATH_MFMA_STREAMK) return 16;
  if (c.path == FP8BS_PATH_PREFILL)
    return pfw_config(c) ? (c.tiles_n == PF_WIDE_160 ? PFW_NARROW_N : BLK) : pf_tile_n(c.waves_n);
  return (c.path == FP8BS_PATH_DOT ? 8 : 16) * c.tiles_n * c.waves_n;
}

// Row range per workgroup of the row-range path: n split over the compute
// units, rounded up to a multiple of 4 (the last workgroup may get fewer).
// On tile-layout weights the ranges start on 16-row tiles (a multiple of
// 16), so no 2 KB tile is fetched in two parts by two workgroups, unless
// that rounding would leave more than 2% of the compute units without a
// range (34816 rows: 144-row ranges would idle 14 of 256 units). Measured
// on MI355X: tile-aligned ranges are needed on long ranges (972 rows of the
// vocabulary layer: 211 against 240-290 us at m = 16-32); on 136-row
// ranges the unaligned split is 1-2.5% faster than the aligned one.
int rows_per_workgroup(int64_t n, int num_cu, int layout = FP8BS_LAYOUT_ROWS) {
  const int64_t cu = num_cu > 0 ? num_cu : 1;
  const int64_t r = (n + cu - 1) / cu;
  const int64_t r4 = (r + 3) / 4 * 4;
  if (layout != FP8BS_LAYOUT_TILES) return (int)r4;
  const int64_t r16 = (r + 15) / 16 * 16;
  return 50 * ((n + r16 - 1) / r16) >= 49 * cu ? (int)r16 : (int)r4;
}

size_t config_lds_bytes(const fp8bs_gemm_config& c, int m, int64_t n, int kbn, int num_cu,
                        bool swiglu = false) {
  if (c.path == FP8BS_PATH_PREFILL) {
    if (pfw_config(c)) return (size_t)pfw_lds_bytes(c.waves_k, c.depth);
    return (size_t)(c.depth > 1 ? pf_dma_lds_bytes(c.waves_n, c.depth) : pf_lds_bytes(c.waves_n));
  }
  const int mt = m <= 16 ? 1 : 2;
  if (c.path == FP8BS_PATH_MFMA_STREAMK)
    return (size_t)lds_streamk_bytes(c.split_k > 0 ? kbn / c.split_k : kbn, m, c.waves_k, mt);
  if (c.path == FP8BS_PATH_MFMA_ROWS_DMA)
    return (size_t)rd_lds_bytes(rows_per_workgroup(n, num_cu, FP8BS_LAYOUT_TILES), kbn, m, c.depth);
  if (is_row_range(c.path)) {
    // weight scales of the row range first, then the kernel's own layout,
    // then (SwiGLU epilogue) the staged outputs
    // (split: the longest K range of a workgroup)
    const int rows = rows_per_workgroup(n, num_cu, c.weight_layout);
    const int nblk = (kbn + c.split_k - 1) / c.split_k;
    const size_t ws = (size_t)lds_wscale_bytes(rows, nblk);
    const size_t ys = swiglu ? (size_t)lds_ystage_bytes(m, rows) : 0;
    if (c.path == FP8BS_PATH_MFMA_STREAM)
      return ws + (size_t)lds_stream_bytes(kbn, m, c.waves_k, mt) + ys;
    if (c.path == FP8BS_PATH_MFMA_ROWS_REG)  // m > 16: 16 rows at a time cast through LDS
      return ws + (size_t)2 * (c.waves_k - 1) * mt * 64 * 16 +
             (mt == 2 ? (size_t)lds_act_bytes(kbn, 16) : 0) + ys;
    return ws + (size_t)lds_act_bytes(nblk, m) + (size_t)2 * (c.waves_k - 1) * mt * 64 * 16 + ys;
  }
  const int nblk = (kbn + c.split_k - 1) / c.split_k;
  size_t red = 0;
  if (c.waves_k > 1) {
    if (c.path == FP8BS_PATH_MFMA) {
      red = (size_t)(c.waves_k - 1) * c.waves_n * c.tiles_n * mt * 64 * 16;
    } else {
      const int md = m <= 1 ? 1 : (m <= 2 ? 2 : 4);
      red = (size_t)(c.waves_k - 1) * c.waves_n * c.tiles_n * md * 64 * 4;
    }
  }
  return (size_t)lds_act_bytes(nblk, m) + red;
}

constexpr size_t kLdsLimit = 160 * 1024;  // one workgroup per CU at most

// The stream-K plan of a configuration (workgroups: the table's compute units).
SkPlan streamk_plan(const fp8bs_gemm_config& c, int64_t n, int64_t k) {
  return sk_plan((int)(n / 16), (int)(k / BLK), c.split_k, kTableCUs, c.waves_n == 2 ? 1 : 0);
}

// Whether a stream-K configuration can run this shape: a supported plan,
// weight offsets within a 31-bit buffer range, one workgroup per CU.
bool streamk_fits(const fp8bs_gemm_config& c, int64_t m, int64_t n, int64_t k) {
  if (c.waves_n < 1 || c.waves_n > 2 || c.waves_k < 1 || c.waves_k > 15 || c.split_k < 1)
    return false;
  if (m > kMaxDecodeM || n * k >= ((int64_t)1 << 31)) return false;
  return sk_plan_ok(streamk_plan(c, n, k));
}


fp8bs_gemm_config make_cfg(int path, int tn, int wn, int wk, int d, int split) {
  fp8bs_gemm_config c;
  std::memset(&c, 0, sizeof(c));
  c.path = path;
  c.tiles_n = tn;
  c.waves_n = wn;
  c.waves_k = wk;
  c.depth = d;
  c.split_k = split;
  c.reduce = FP8BS_REDUCE_KERNEL;
  return c;
}

struct Candidate {
  int path, tn, wn, wk, d, split, reduce;
};

constexpr int LA = FP8BS_REDUCE_LAST_ARRIVER;
constexpr int RK = FP8BS_REDUCE_KERNEL;
constexpr int MF = FP8BS_PATH_MFMA;
constexpr int DT = FP8BS_PATH_DOT;
constexpr int RW = FP8BS_PATH_MFMA_ROWS;
constexpr int ST = FP8BS_PATH_MFMA_STREAM;
constexpr int RR = FP8BS_PATH_MFMA_ROWS_REG;
constexpr int SK = FP8BS_PATH_MFMA_STREAMK;
constexpr int RD = FP8BS_PATH_MFMA_ROWS_DMA;

// Configurations the SwiGLU call accepts. With the separate epilogue:
// everything but the last-arriver reduce (the split sum carries the
// epilogue, or a second kernel runs it). Inside the GEMM: unsplit MFMA grid
// and the row-range kernels compiled with the epilogue.
bool swiglu_supported(const fp8bs_gemm_config& c, int m) {
  if (c.epilogue == FP8BS_EPILOGUE_SEPARATE)
    return c.split_k == 1 || c.reduce == FP8BS_REDUCE_KERNEL;
  if (c.epilogue != FP8BS_EPILOGUE_IN_GEMM || c.split_k != 1) return false;
  if (is_row_range(c.path)) return find_kernel(c, m, true, true) != nullptr;
  return c.path == FP8BS_PATH_MFMA;
}

bool candidate_fits(const Candidate& cd, int64_t m, int64_t n, int kbn, fp8bs_gemm_config* out,
                    int layout = FP8BS_LAYOUT_ROWS) {
  fp8bs_gemm_config c = make_cfg(cd.path, cd.tn, cd.wn, cd.wk, cd.d, cd.split);
  c.reduce = cd.split > 1 ? cd.reduce : RK;
  c.weight_layout = layout;
  // the tile layout is compiled for the kernels the table selects with it
  if (layout != FP8BS_LAYOUT_ROWS && !find_kernel(c, (int)m, true)) return false;
  if (n % config_rows(c) != 0) return false;
  if (cd.path == DT && m > 4) return false;
  if (c.split_k > kbn) return false;
  if (cd.path == ST && !stream_offsets_fit(m, (int64_t)kbn * BLK)) return false;
  if (cd.path == RR && !rows_reg_fits(c, kbn)) return false;
  if (cd.path == SK && !streamk_fits(c, m, n, (int64_t)kbn * BLK)) return false;
  if (kbn > 0 && config_lds_bytes(c, (int)m, n, kbn, kTableCUs) > kLdsLimit) return false;
  *out = c;
  return true;
}

// The fixed configuration table. A pure function of (m, n, k): no timing,
// no device state, so a shape always runs the same kernel and gives the
// same bits. Shapes fall in five classes by their extents (square-like,
// deep K, wide N in one round of 128-row workgroups, wide N, vocabulary-wide
// N) and six classes of m; each cell lists
// candidates in order of preference, measured on MI355X with graph-replayed
// launches over a rotating 1 GiB weight pool. The first candidate that fits
// the shape (rows dividing n, split not above the number of K blocks,
// staged activations within the LDS budget, the K range within the
// registers of the register-activation kernel) is used; on wide shapes with
// 17-32 rows the LDS row-range kernel fits up to about 22 rows at k = 5120
// and the register-activation kernel takes the rest; a fallback list with
// growing split catches everything else. The SwiGLU call (swiglu set) uses
// the same choice with the separate epilogue, so its y equals fp8bs_gemm's.
//
// With the tile layout (layout = FP8BS_LAYOUT_TILES) a second table of the
// same classes applies, measured the same way on tile-layout weights. The
// grid kernels stream that layout faster than row-major weights (each load
// instruction reads one contiguous KB), while the one-workgroup-per-CU
// kernels on long row ranges do not, so this table takes the grid kernels
// wherever they win; candidates without a tile-layout kernel are passed
// over. Prefill sizes take the direct-load kernel in either layout.
// Vocabulary-wide shapes at m = 9-16 on tile-layout weights take the
// row-range kernel with the weight stream through LDS (3 stages): 248320 x
// 5120 at m = 9 / 12 / 16: 190.0 / 194.6 / 201.0 us against 197.9 / 202.7 /
// 207.9 us for the row-range kernel.
// Deep K (MLP down, 17408 -> 5120) from m = 5 splits K over 5 or 6
// workgroups per 128-column group (200 or 240 workgroups): tile layout
// m = 8 18.5 against 19.2 us with 4, m = 16 19.5 against 21.4 us, m = 32
// 23.6 against 25.6 us; row-major m = 16 20.9 against 21.9 us.
bool select_config(int64_t m, int64_t n, int64_t k, fp8bs_gemm_config* out, bool swiglu = false,
                   int layout = FP8BS_LAYOUT_ROWS) {
  if (m < 0 || m > kMaxM || n < 0 || k < 0 || n % BLK || k % BLK) return false;
  if (swiglu && n % (2 * BLK)) return false;
  if (m > kMaxDecodeM && n > 0 && k > 0) {
    // prefill sizes with at least 150 256 x 256 output tiles (m n >= about
    // 9.8 M): the wide kernel (8 waves, 16 JM x 128 outputs each) on the 1-D
    // schedule. Measured on MI355X at m = 128 .. 8192 on the square, MLP-up
    // and MLP-down weights: faster than the 128 x 128 kernel from 160 tiles
    // up (square m = 2048: 70 against 84 us; m = 8192: 214 against 260 us),
    // slower at 136 and fewer (MLP up m = 128: 80 against 71 us). Between
    // 256-row (JM = 4) and 192-row (JM = 3) tiles, the one with fewer rounds
    // of 256 workgroups, a 192-row tile counted as 0.8 of a 256-row one and
    // a round of half tiles as 0.6 of a round (the measured ratios): 192 rows
    // at square and MLP-down m = 2048 (70 against 74 us, 208 against
    // 226 us), 256 rows at m = 8192 and on MLP up.
    // Narrow tiles ((64 JM) x 160, n a multiple of 640) where they make
    // one round that occupies at least three quarters of the compute units
    // (256-row tiles first): one 160-column tile does about 15% less work
    // per unit of time than a wide one, but leaves fewer units idle.
    // Measured on MI355X at n = 5120, against the table's choice without
    // them: square m = 1024 50.6 against 52.0 us (192-row narrow tiles
    // against the 128 x 128 kernel), m = 2048 69.0 against 70.1 us (256-row
    // narrow tiles against 192 x 256 tiles); MLP down m = 1024 148.2 against
    // 152.0 us, m = 2048 204.6 against 212.8 us; at m = 4096 (not one round)
    // the two tie, at m = 8192 narrow tiles take 17% longer.
    // Deep K (k >= 12288) with too few wide tiles to occupy the compute
    // units: the wide kernel on the grid schedule with K split over s
    // workgroups, s the largest that keeps tiles x s within one round of
    // kTableCUs workgroups, when that round is at least three quarters full
    // and each split keeps at least 8 K blocks (256-row tiles first); the
    // fp32 partials are summed by the reduce kernel. Measured on MI355X on
    // MLP down (17408 -> 5120): m = 1024 110 against 148 us (80 tiles,
    // split 3), m = 512 74 against 88 us (40 tiles, split 6), m = 256 52
    // against 64 us, m = 128 41 against 44 us (20 tiles, split 12); at
    // m = 64 the 128 x 128 kernel stays (34 against 38 us: three quarters
    // of a 256-row tile would be padding).
    const int64_t kbn_p = k / BLK;
    if (kbn_p >= 96 && m > 64) {
      for (int jm = 4; jm >= 3; --jm) {
        const int64_t tm = pfw_tile_m(jm);
        const int64_t tiles = ((n + PFW_TILE_N - 1) / PFW_TILE_N) * ((m + tm - 1) / tm);
        if (tiles >= kTableCUs) break;
        int64_t sp = kTableCUs / tiles;
        sp = sp < kbn_p / 8 ? sp : kbn_p / 8;
        sp = sp < 64 ? sp : 64;
        if (sp >= 2 && 4 * tiles * sp >= 3 * kTableCUs) {
          *out = make_cfg(FP8BS_PATH_PREFILL, PF_WIDE, 2, jm, 2, (int)sp);
          out->weight_layout = layout;
          return true;
        }
      }
    }
    if (n % (5 * BLK) == 0) {
      for (int njm = 4; njm >= 3; --njm) {
        const int64_t t = pfw_plan_narrow(njm, m, n).units;
        if (4 * t >= 3 * kTableCUs && t <= kTableCUs) {
          *out = make_cfg(FP8BS_PATH_PREFILL, PF_WIDE_160, 2, njm, 2, 1);
          out->weight_layout = layout;
          return true;
        }
      }
    }
    // (also from 128 tiles whose rows are at least 90% filled: MLP up at
    // m = 256, 136 tiles, 83.9 against 103.3 us with the 128 x 128 kernel)
    const int64_t wtiles = ((n + PFW_TILE_N - 1) / PFW_TILE_N) * ((m + 255) / 256);
    const bool full_rows = 10 * m >= 9 * ((m + 255) / 256) * 256;
    if (wtiles >= 150 || (wtiles >= 128 && full_rows)) {
      auto cost = [&](int jm) {
        const int64_t tm = pfw_tile_m(jm);
        const int64_t tiles = ((n + PFW_TILE_N - 1) / PFW_TILE_N) * ((m + tm - 1) / tm);
        const int64_t full = tiles / kTableCUs * kTableCUs, rem = tiles - full;
        double r = (double)(full / kTableCUs);
        if (rem > 0) r += 2 * rem <= kTableCUs ? 0.6 : 1.0;
        return jm == 3 ? 0.8 * r : r;
      };
      const int jm = cost(3) < cost(4) ? 3 : 4;
      // (the grid schedule where the 1-D grid would pass 2^31 workgroups)
      const bool one_d = pfw_plan(jm, m, n).units <= INT32_MAX;
      *out = make_cfg(FP8BS_PATH_PREFILL, one_d ? PF_WIDE_1D : PF_WIDE, 2, jm, 2, 1);
      out->weight_layout = layout;
      return true;
    }
    // fewer tiles: the tiled kernel with 4 waves on 128 x 128 output tiles
    // and two LDS stages filled by direct loads (two workgroups per compute
    // unit), with K split when the tiles alone cannot fill the compute units
    // (each split keeps at least two K blocks). Measured on MI355X at
    // m = 512 .. 8192 against the register-pipelined kernels and deeper
    // stage rings (one workgroup per unit), which it beats at every size.
    const int64_t mtiles = (m + PF_TILE_M - 1) / PF_TILE_M;
    const int wn = 2;
    const int64_t tiles = (n / pf_tile_n(wn)) * mtiles;
    int64_t split = (kTableCUs + tiles - 1) / tiles;
    const int64_t kblocks = k / BLK;
    const int64_t max_split = kblocks / 2 < 16 ? kblocks / 2 : 16;
    split = split < max_split ? split : max_split;
    split = split < 1 ? 1 : split;
    *out = make_cfg(FP8BS_PATH_PREFILL, 1, wn, 2, 2, (int)split);
    out->weight_layout = layout;
    return true;
  }
  const int kbn = (int)(k / BLK);
  const int64_t nbn = n / BLK;
  if (m == 0 || n == 0 || kbn == 0) {
    *out = make_cfg(MF, 1, 1, 4, 5, 1);
    out->weight_layout = layout;
    return true;
  }
  struct Cell {
    Candidate c[3];
    int n;
  };
  // [shape class][m class]: m = 1, 2, 3-4, 5-8, 9-16, 17-32; each candidate
  // is {path, tiles_n, waves_n, waves_k, depth, split_k, reduce}
  static const Cell table[5][6] = {
      // square-like: n < 25600, k <= 6144
      {{{{DT, 2, 2, 4, 4, 1, RK}, {MF, 1, 2, 4, 5, 1, RK}}, 2},
       {{{MF, 1, 2, 4, 5, 1, RK}}, 1},
       {{{MF, 1, 2, 4, 5, 1, RK}, {MF, 1, 5, 1, 5, 4, RK}}, 2},
       {{{MF, 1, 2, 4, 5, 1, RK}, {MF, 1, 5, 1, 5, 4, RK}}, 2},
       {{{MF, 1, 5, 1, 5, 4, RK}, {MF, 1, 5, 2, 5, 4, RK}}, 2},
       {{{MF, 1, 5, 2, 5, 4, RK}, {MF, 1, 8, 1, 5, 4, RK}}, 2}},
      // deep K: n < 25600, k > 6144
      {{{{DT, 2, 2, 4, 4, 1, RK}, {MF, 1, 5, 2, 2, 4, RK}}, 2},
       {{{MF, 1, 5, 1, 5, 4, RK}, {MF, 1, 5, 2, 2, 4, RK}}, 2},
       {{{MF, 1, 5, 1, 5, 4, RK}, {MF, 1, 5, 2, 2, 4, RK}}, 2},
       {{{MF, 1, 8, 1, 5, 6, RK}, {MF, 1, 5, 2, 5, 4, RK}}, 2},
       {{{MF, 1, 8, 1, 5, 6, RK}, {MF, 1, 5, 2, 5, 4, RK}}, 2},
       {{{MF, 1, 8, 1, 5, 6, RK}, {MF, 2, 5, 1, 5, 8, RK}}, 2}},
      // wide N: 256 < n/128 < 512 (32768 < n < 65536)
      {{{{MF, 1, 1, 4, 5, 1, RK}, {MF, 1, 1, 8, 5, 1, RK}}, 2},
       {{{RW, 4, 1, 8, 4, 1, RK}, {RW, 1, 1, 8, 3, 1, RK}}, 2},
       {{{RW, 1, 1, 8, 3, 1, RK}, {RW, 2, 1, 8, 6, 1, RK}}, 2},
       {{{RW, 2, 1, 8, 6, 1, RK}, {RW, 1, 1, 8, 3, 1, RK}}, 2},
       {{{RW, 4, 1, 8, 4, 1, RK}, {RW, 2, 1, 8, 6, 1, RK}}, 2},
       {{{RW, 2, 1, 8, 6, 1, RK}, {RR, 1, 1, 8, 5, 1, RK}, {MF, 1, 8, 1, 5, 4, RK}}, 3}},
      // vocabulary-wide N: n >= 65536
      {{{{MF, 1, 2, 4, 2, 1, RK}, {MF, 1, 2, 4, 5, 1, RK}}, 2},
       {{{MF, 1, 2, 4, 5, 1, RK}, {MF, 1, 1, 8, 5, 1, RK}}, 2},
       {{{MF, 4, 1, 4, 2, 1, RK}, {MF, 1, 8, 1, 5, 1, RK}}, 2},
       {{{ST, 1, 1, 8, 6, 1, RK}, {RW, 2, 1, 8, 6, 1, RK}}, 2},
       {{{RW, 1, 1, 8, 3, 1, RK}, {RW, 2, 1, 8, 6, 1, RK}}, 2},
       {{{RW, 2, 1, 8, 6, 1, RK}, {RR, 1, 1, 8, 5, 1, RK}, {MF, 1, 8, 1, 5, 2, RK}}, 3}},
      // wide N in one round of 128-row workgroups: 200 <= n/128 <= 256 (one
      // GPU's 8-way column share of the vocabulary layer, 31104 x 5120: 8
      // waves along N, 128 output columns per workgroup, at most one per
      // compute unit; at m = 3-24, 26.2-33.1 us against 27.4-37.2 us for the
      // wide-N choices)
      {{{{MF, 1, 1, 4, 5, 1, RK}, {MF, 1, 1, 8, 5, 1, RK}}, 2},
       {{{MF, 1, 8, 1, 5, 1, RK}, {RW, 4, 1, 8, 4, 1, RK}}, 2},
       {{{MF, 1, 8, 1, 5, 1, RK}, {RW, 1, 1, 8, 3, 1, RK}}, 2},
       {{{MF, 1, 8, 1, 5, 1, RK}, {RW, 2, 1, 8, 6, 1, RK}}, 2},
       {{{MF, 1, 8, 1, 5, 1, RK}, {RW, 4, 1, 8, 4, 1, RK}}, 2},
       {{{MF, 1, 8, 1, 5, 1, RK}, {RW, 2, 1, 8, 6, 1, RK}, {RR, 1, 1, 8, 5, 1, RK}}, 3}}};
  static const Candidate fallback[] = {{MF, 1, 1, 4, 5, 1, RK}, {MF, 1, 1, 4, 5, 2, RK},
                                       {MF, 1, 1, 4, 5, 4, RK}, {MF, 1, 1, 4, 5, 8, RK},
                                       {MF, 1, 1, 4, 5, 16, RK}, {MF, 1, 1, 4, 5, 32, RK},
                                       {MF, 1, 1, 4, 5, 64, RK}};
  static const Cell table_tiles[5][6] = {
      // square-like
      {{{{MF, 1, 2, 4, 5, 1, RK}}, 1},
       {{{MF, 1, 2, 4, 5, 1, RK}}, 1},
       {{{MF, 1, 2, 4, 5, 1, RK}, {MF, 1, 5, 1, 5, 4, RK}}, 2},
       {{{MF, 1, 2, 4, 5, 1, RK}, {MF, 1, 5, 1, 5, 4, RK}}, 2},
       {{{MF, 1, 8, 1, 5, 4, RK}, {MF, 1, 5, 1, 5, 4, RK}}, 2},
       {{{MF, 1, 8, 1, 5, 4, RK}, {MF, 1, 5, 2, 5, 4, RK}}, 2}},
      // deep K (m = 1-2: no K split, so no second kernel; MLP down
      // 17408 -> 5120 at m = 1 / 2: 16.2 / 16.8 us against 17.5 / 17.8 us
      // with K split in four)
      {{{{MF, 1, 2, 4, 5, 1, RK}, {MF, 1, 5, 2, 2, 4, RK}, {MF, 1, 5, 1, 5, 4, RK}}, 3},
       {{{MF, 1, 2, 4, 5, 1, RK}, {MF, 1, 5, 1, 5, 4, RK}, {MF, 1, 5, 2, 2, 4, RK}}, 3},
       {{{MF, 1, 5, 1, 5, 4, RK}, {MF, 1, 5, 2, 2, 4, RK}}, 2},
       {{{MF, 1, 8, 1, 5, 5, RK}, {MF, 1, 8, 1, 5, 4, RK}}, 2},
       {{{MF, 1, 8, 1, 5, 6, RK}, {MF, 1, 8, 1, 5, 4, RK}}, 2},
       {{{MF, 1, 8, 1, 5, 6, RK}, {MF, 2, 5, 1, 5, 8, RK}}, 2}},
      // wide N (256 < n/128 < 512)
      {{{{MF, 1, 1, 4, 5, 1, RK}, {MF, 1, 1, 8, 5, 1, RK}}, 2},
       {{{MF, 1, 1, 8, 5, 1, RK}, {MF, 1, 1, 4, 5, 1, RK}}, 2},
       {{{RW, 1, 1, 8, 3, 1, RK}, {MF, 1, 1, 8, 5, 1, RK}}, 2},
       {{{RW, 1, 1, 8, 3, 1, RK}, {RW, 2, 1, 8, 6, 1, RK}}, 2},
       {{{RW, 1, 1, 8, 3, 1, RK}, {RW, 2, 1, 8, 6, 1, RK}}, 2},
       {{{RW, 2, 1, 8, 6, 1, RK}, {RR, 1, 1, 8, 5, 1, RK}, {MF, 1, 8, 1, 5, 4, RK}}, 3}},
      // vocabulary-wide N
      {{{{MF, 1, 1, 8, 5, 1, RK}, {MF, 1, 2, 4, 2, 1, RK}}, 2},
       {{{MF, 1, 2, 4, 2, 1, RK}, {MF, 1, 1, 8, 5, 1, RK}}, 2},
       {{{MF, 1, 2, 4, 2, 1, RK}, {MF, 1, 2, 4, 5, 1, RK}}, 2},
       {{{MF, 1, 8, 1, 5, 1, RK}, {MF, 1, 2, 4, 5, 1, RK}}, 2},
       {{{RD, 1, 1, 8, 3, 1, RK}, {RW, 1, 1, 8, 3, 1, RK}, {MF, 1, 8, 1, 5, 1, RK}}, 3},
       {{{RW, 1, 1, 8, 3, 1, RK}, {RR, 1, 1, 8, 5, 1, RK}, {MF, 1, 8, 1, 5, 2, RK}}, 3}},
      // wide N in one round of 128-row workgroups (31104 x 5120 at m = 3-4:
      // 24.7-25.3 us with 2 x 4 waves against 33.0-33.1; m = 5-24: 8 waves
      // along N, 26.4-32.9 us against 34.0-42.4; m = 32: the same with K
      // split in two, 39.4 against 43.5 us)
      {{{{MF, 1, 2, 4, 5, 1, RK}, {MF, 1, 1, 4, 5, 1, RK}}, 2},
       {{{MF, 1, 2, 4, 5, 1, RK}, {MF, 1, 8, 1, 5, 1, RK}}, 2},
       {{{MF, 1, 2, 4, 5, 1, RK}, {MF, 1, 8, 1, 5, 1, RK}}, 2},
       {{{MF, 1, 8, 1, 5, 1, RK}, {MF, 1, 2, 4, 5, 1, RK}}, 2},
       {{{MF, 1, 8, 1, 5, 1, RK}, {RD, 1, 1, 8, 3, 1, RK}, {RW, 1, 1, 8, 3, 1, RK}}, 3},
       {{{MF, 1, 8, 1, 5, 1, RK}, {MF, 1, 8, 1, 5, 2, RK}, {RW, 2, 1, 8, 6, 1, RK}}, 3}}};
  // shape class: 3 vocabulary-wide, 2 wide N, 4 wide N whose 128-row blocks
  // fill at most one round of compute units, 1 deep K, 0 square-like
  const int shape = nbn >= 512 ? 3
                    : nbn > kTableCUs ? 2
                    : nbn >= 200 ? 4
                    : (kbn > 48 ? 1 : 0);
  const int mc = m == 1 ? 0 : (m == 2 ? 1 : (m <= 4 ? 2 : (m <= 8 ? 3 : (m <= 16 ? 4 : 5))));
  const Cell& cell = layout == FP8BS_LAYOUT_ROWS ? table[shape][mc] : table_tiles[shape][mc];
  for (int i = 0; i < cell.n; ++i)
    if (candidate_fits(cell.c[i], m, n, kbn, out, layout)) return true;
  for (const Candidate& cd : fallback)
    if (candidate_fits(cd, m, n, kbn, out, layout)) return true;
  return false;
}

// Workspace layout: fp32 partials [split][m][n], then (last-arriver reduce)
// one 64-bit arrival counter per row group.
size_t cfg_partial_bytes(const fp8bs_gemm_config& c, int64_t m, int64_t n) {
  return c.split_k > 1 ? (size_t)c.split_k * (size_t)m * (size_t)n * sizeof(float) : 0;
}

// Prefill path, fused cast: the activation codes [m][k] and scales [m][k/128]
// are written to the workspace first.
size_t prefill_x_bytes(int64_t m, int64_t k) {
  return (size_t)((m * k + 255) / 256 * 256) + (size_t)((m * (k / BLK) * 4 + 15) / 16 * 16);
}

// Prefill workspace: the cast activations (fused call), then the split
// partials.
size_t prefill_workspace(const fp8bs_gemm_config& c, int64_t m, int64_t n, int64_t k, bool fused) {
  return (fused ? prefill_x_bytes(m, k) : 0) + cfg_partial_bytes(c, m, n);
}

size_t cfg_workspace(const fp8bs_gemm_config& c, int64_t m, int64_t n, int64_t k, bool fused) {
  if (c.path == FP8BS_PATH_PREFILL) return prefill_workspace(c, m, n, k, fused);
  if (c.path == FP8BS_PATH_MFMA_STREAMK)
    return (size_t)sk_workspace_bytes(streamk_plan(c, n, k), m <= 16 ? 1 : 2);
  size_t b = cfg_partial_bytes(c, m, n);
  if (c.split_k > 1 && c.reduce == FP8BS_REDUCE_LAST_ARRIVER) {
    const int rows = config_rows(c);
    b += (size_t)((n / rows) * sizeof(uint64_t) + 15) / 16 * 16;
  }
  return b;
}

// SwiGLU workspace: the split partials, or (epilogue inside the GEMM) one
// 64-bit arrival counter per 128-column block of h.
size_t swiglu_workspace(const fp8bs_gemm_config& c, int64_t m, int64_t n, int64_t k, bool fused) {
  if (c.path == FP8BS_PATH_PREFILL) return prefill_workspace(c, m, n, k, fused);
  if (c.path == FP8BS_PATH_MFMA_STREAMK) return cfg_workspace(c, m, n, k, fused);
  if (c.split_k > 1) return cfg_partial_bytes(c, m, n);
  if (c.epilogue != FP8BS_EPILOGUE_IN_GEMM) return 0;
  return (size_t)((n / (2 * BLK)) * sizeof(uint64_t) + 15) / 16 * 16;
}

// The standalone MLP epilogue launch (also used by the fused call when k == 0).
fp8bs_status launch_swiglu_quant(const void* y_bf16, int64_t m, int64_t inter, uint8_t* h_fp8,
                                 float* h_scale, void* stream) {
  const uint16_t* y = static_cast<const uint16_t*>(y_bf16);
  int64_t in = inter;
  void* args[] = {&y, &in, &h_fp8, &h_scale};
  g_counts[CNT_SWIGLU]++;
  return launch(reinterpret_cast<const void*>(swiglu_quant_kernel),
                dim3((unsigned)(inter / BLK), (unsigned)m), dim3(64), 0, stream, args);
}


// Shape limits of every GEMM entry point: n and k whole blocks; n below
// 2^31 (the kernels index columns in 32 bits), k/128 at most 2^20; m up to
// 2^20 (the SwiGLU call: 65535, one epilogue wave row per activation row);
// the prefill kernel (m > 32) forms 32-bit offsets within a 256-row slab of
// W, so there k < 2^24.
bool gemm_shape_ok(int64_t m, int64_t n, int64_t k, bool swiglu) {
  if (m < 0 || m > kMaxM || n < 0 || k < 0 || n % BLK || k % BLK) return false;
  if (n / BLK >= (int64_t)1 << 24 || k / BLK > (int64_t)1 << 20) return false;
  if (swiglu && (n % (2 * BLK) || m > 65535)) return false;
  if (m > kMaxDecodeM && (int64_t)256 * k >= ((int64_t)1 << 32)) return false;
  return true;
}

// The GEMM, optionally with the SwiGLU epilogue (swiglu: h_fp8 and h_scale
// receive the re-quantized SwiGLU output). fused: the activations are bf16
// x_bf16 (cast in the kernel), else codes x_fp8 and scales x_scale.
// Checks run in the documented order -- shape, NULL pointers, alignment,
// configuration, workspace, device -- and all of them before any launch.
fp8bs_status gemm_impl(bool fused, const void* x_bf16, const uint8_t* x_fp8,
                       const float* x_scale, int64_t m, const uint8_t* w_fp8,
                       const float* w_scale, int64_t n, int64_t k, void* y_bf16, void* workspace,
                       size_t workspace_bytes, const fp8bs_gemm_config* cfg_in, void* stream,
                       bool swiglu = false, uint8_t* h_fp8 = nullptr, float* h_scale = nullptr,
                       int layout = FP8BS_LAYOUT_ROWS) {
  // shapes (an empty output is a no-op whatever the pointers)
  if (!gemm_shape_ok(m, n, k, swiglu)) return FP8BS_ERR_SHAPE;
  if (m == 0 || n == 0) return FP8BS_OK;
  // pointers
  if (!y_bf16) return FP8BS_ERR_NULL;
  if (swiglu && (!h_fp8 || !h_scale)) return FP8BS_ERR_NULL;
  if (k > 0) {
    if (!w_fp8 || !w_scale) return FP8BS_ERR_NULL;
    if (fused ? !x_bf16 : (!x_fp8 || !x_scale)) return FP8BS_ERR_NULL;
  }
  // alignment
  if (!aligned(y_bf16, 16)) return FP8BS_ERR_ALIGN;
  if (swiglu && (!aligned(h_fp8, 16) || !aligned(h_scale, 4))) return FP8BS_ERR_ALIGN;
  if (k > 0) {
    if (!aligned(w_fp8, 16) || !aligned(w_scale, 4)) return FP8BS_ERR_ALIGN;
    if (fused ? !aligned(x_bf16, 16) : (!aligned(x_fp8, 16) || !aligned(x_scale, 4)))
      return FP8BS_ERR_ALIGN;
  }
  if (k == 0) {
    DeviceInfo dev;
    const fp8bs_status st = current_device(&dev);
    if (st != FP8BS_OK) return st;
    const int64_t n8 = m * n / 4;
    uint2* y = static_cast<uint2*>(y_bf16);
    int64_t n8v = n8;
    void* args[] = {&y, &n8v};
    g_counts[CNT_RED]++;
    const fp8bs_status zs = launch(reinterpret_cast<const void*>(zero_fill_kernel),
                                   dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, stream, args);
    if (zs != FP8BS_OK || !swiglu) return zs;
    return launch_swiglu_quant(y_bf16, m, n / 2, h_fp8, h_scale, stream);
  }
  const int kbn = (int)(k / BLK);
  // configuration
  fp8bs_gemm_config c;
  if (cfg_in) {
    c = *cfg_in;
  } else if (!select_config(m, n, k, &c, swiglu, layout)) {
    return FP8BS_ERR_SHAPE;
  }
  // tile layout: plain kernels only (the SwiGLU epilogue runs after the split
  // sum or in a second kernel)
  if (c.weight_layout != FP8BS_LAYOUT_ROWS &&
      (c.weight_layout != FP8BS_LAYOUT_TILES || (swiglu && c.epilogue != FP8BS_EPILOGUE_SEPARATE)))
    return FP8BS_ERR_CONFIG;
  // the prefill kernel forms its per-lane weight offsets in 32 bits (up to
  // 256 rows times k, or 16 tiles times k/128 times 2 KB): an explicit
  // prefill configuration needs the prefill shape limit too
  if (c.path == FP8BS_PATH_PREFILL && (int64_t)256 * k >= ((int64_t)1 << 32))
    return FP8BS_ERR_CONFIG;
  if (c.split_k < 1 || c.split_k > 64 || c.split_k > kbn) return FP8BS_ERR_CONFIG;
  if (c.path == FP8BS_PATH_PREFILL ? c.reduce != FP8BS_REDUCE_KERNEL : m > kMaxDecodeM)
    return FP8BS_ERR_CONFIG;
  // the 1-D schedule runs every tile over the whole K range, one workgroup
  // per whole or half tile on a one-dimensional grid
  if (c.path == FP8BS_PATH_PREFILL && c.tiles_n == PF_WIDE_1D &&
      (c.split_k != 1 || pfw_plan(c.waves_k, m, n).units > INT32_MAX))
    return FP8BS_ERR_CONFIG;
  if (c.path == FP8BS_PATH_PREFILL && c.tiles_n == PF_WIDE_160 &&
      (c.split_k != 1 || n % PFW_NARROW_N || pfw_plan_narrow(c.waves_k, m, n).units > INT32_MAX))
    return FP8BS_ERR_CONFIG;
  // row-range paths: split only on MFMA_ROWS, with the reduce kernel
  if (is_row_range(c.path) &&
      (c.waves_n != 1 ||
       (c.split_k != 1 && (c.path != FP8BS_PATH_MFMA_ROWS || c.reduce != FP8BS_REDUCE_KERNEL))))
    return FP8BS_ERR_CONFIG;
  if (c.path == FP8BS_PATH_MFMA_STREAM && !stream_offsets_fit(m, k)) return FP8BS_ERR_CONFIG;
  if (c.path == FP8BS_PATH_MFMA_ROWS_REG && !rows_reg_fits(c, kbn)) return FP8BS_ERR_CONFIG;
  if (c.path == FP8BS_PATH_MFMA_ROWS_DMA &&
      (c.weight_layout != FP8BS_LAYOUT_TILES || c.split_k != 1 || c.tiles_n != 1 || m > 16))
    return FP8BS_ERR_CONFIG;
  const bool streamk = c.path == FP8BS_PATH_MFMA_STREAMK;
  if (streamk && (!streamk_fits(c, m, n, k) || c.reduce != FP8BS_REDUCE_KERNEL))
    return FP8BS_ERR_CONFIG;
  if (c.reduce != FP8BS_REDUCE_KERNEL && c.reduce != FP8BS_REDUCE_LAST_ARRIVER)
    return FP8BS_ERR_CONFIG;
  if (swiglu && !swiglu_supported(c, (int)m)) return FP8BS_ERR_CONFIG;
  const bool in_gemm = swiglu && c.epilogue == FP8BS_EPILOGUE_IN_GEMM;
  const bool split = c.split_k > 1 && !streamk;  // stream-K: split_k counts K chunks
  const bool last_arriver = split && c.reduce == FP8BS_REDUCE_LAST_ARRIVER;
  const bool prefill = c.path == FP8BS_PATH_PREFILL;
  const KernelEntry* ke = find_kernel(c, (int)m, fused && !prefill, in_gemm);
  if (!ke) return FP8BS_ERR_CONFIG;
  const int rows = config_rows(c);
  if (n % rows) return FP8BS_ERR_CONFIG;
  // workspace
  const size_t need =
      swiglu ? swiglu_workspace(c, m, n, k, fused) : cfg_workspace(c, m, n, k, fused);
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return FP8BS_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return FP8BS_ERR_ALIGN;
  }
  // device
  DeviceInfo dev;
  const fp8bs_status st = current_device(&dev);
  if (st != FP8BS_OK) return st;
  const size_t lds = config_lds_bytes(c, (int)m, n, kbn, kTableCUs, in_gemm);
  if (lds > (size_t)dev.max_lds) return FP8BS_ERR_CONFIG;
  if (lds > 64 * 1024) {
    const fp8bs_status ls = raise_lds_limit(reinterpret_cast<const void*>(ke->fn),
                                            (int)(ke - kernel_registry().data()), dev, lds);
    if (ls != FP8BS_OK) return ls;
  }

  GemmParams p;
  p.x = static_cast<const uint16_t*>(x_bf16);
  p.xq = x_fp8;
  p.xs = x_scale;
  p.wq = w_fp8;
  p.ws = w_scale;
  p.y = static_cast<uint16_t*>(y_bf16);
  p.part = static_cast<float*>(workspace);
  p.counters = last_arriver ? reinterpret_cast<uint64_t*>(static_cast<uint8_t*>(workspace) +
                                                          cfg_partial_bytes(c, m, n))
                            : nullptr;
  if (in_gemm) p.counters = static_cast<uint64_t*>(workspace);
  p.hq = h_fp8;
  p.hs = h_scale;
  p.epoch = g_epoch.fetch_add(1) & ((uint64_t(1) << 56) - 1);
  p.sk_whole = streamk && c.waves_n == 2 ? 1 : 0;
  p.pf_full = 0;
  p.pf_1d = 0;
  p.rows_per_wg = 0;
  p.m = (int)m;
  p.n = (int)n;
  p.k = (int)k;
  p.kbn = kbn;
  p.split = c.split_k;
  p.out = !split ? (in_gemm ? OUT_SWIGLU : OUT_DIRECT)
                 : (last_arriver ? OUT_LAST_ARRIVER : OUT_PARTIAL);
  void* args[] = {&p};
  dim3 grid((unsigned)(n / rows), (unsigned)c.split_k);
  if (is_row_range(c.path)) {
    p.rows_per_wg = rows_per_workgroup(n, kTableCUs, c.weight_layout);
    grid = dim3((unsigned)((n + p.rows_per_wg - 1) / p.rows_per_wg), (unsigned)c.split_k);
  }
  // the SwiGLU epilogue arrives on each (side, 128-column block) pair of a
  // workgroup's range at once, one lane per pair
  if (in_gemm && 2 * ((is_row_range(c.path) ? p.rows_per_wg : rows) / BLK + 2) >
                     SWIGLU_MAX_ARRIVALS)
    return FP8BS_ERR_CONFIG;
  dim3 block(64 * (is_row_range(c.path) ? 1 : c.waves_n) * c.waves_k);
  if (c.path == FP8BS_PATH_MFMA_ROWS_DMA) block = dim3(64 * (RD_WK + RD_LOADERS));
  if (streamk) {
    grid = dim3((unsigned)kTableCUs);
    block = dim3(64 * (c.waves_k + 1));
  }
  if (prefill) {
    if (pfw_config(c)) {
      const int64_t tm = pfw_tile_m(c.waves_k);
      grid = dim3((unsigned)((n + PFW_TILE_N - 1) / PFW_TILE_N), (unsigned)((m + tm - 1) / tm),
                  (unsigned)c.split_k);
      block = dim3(512);  // 8 waves; waves_k gives the rows per wave (16 waves_k)
      if (c.tiles_n == PF_WIDE_1D || c.tiles_n == PF_WIDE_160) {
        const PfwPlan q = c.tiles_n == PF_WIDE_1D ? pfw_plan(c.waves_k, m, n)
                                                  : pfw_plan_narrow(c.waves_k, m, n);
        grid = dim3((unsigned)q.units);
        p.pf_full = (int)q.full;
        p.pf_1d = 1;
      }
    } else {
      grid = dim3((unsigned)(n / pf_tile_n(c.waves_n)),
                  (unsigned)((m + PF_TILE_M - 1) / PF_TILE_M), (unsigned)c.split_k);
      block = dim3(128 * c.waves_n);
    }
    p.part = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) +
                                      (fused ? prefill_x_bytes(m, k) : 0));
    if (fused) {
      // cast the activations into the workspace: codes, then scales
      uint8_t* xq = static_cast<uint8_t*>(workspace);
      float* xs = reinterpret_cast<float*>(xq + (m * k + 255) / 256 * 256);
      const uint16_t* xb = static_cast<const uint16_t*>(x_bf16);
      int64_t nb = m * kbn, kk = k;
      void* qargs[] = {&xb, &nb, &kk, &xq, &xs};
      g_counts[CNT_QA]++;
      const fp8bs_status qs = launch(reinterpret_cast<const void*>(quant_act_kernel),
                                     dim3((unsigned)((nb * 4 + 255) / 256)), dim3(256), 0, stream,
                                     qargs);
      if (qs != FP8BS_OK) return qs;
      p.x = nullptr;
      p.xq = xq;
      p.xs = xs;
    }
  }
  g_counts[c.path == FP8BS_PATH_DOT ? CNT_DOT : CNT_MFMA]++;
  fp8bs_status ls = launch(reinterpret_cast<const void*>(ke->fn), grid, block, lds, stream, args);
  if (ls != FP8BS_OK || last_arriver || in_gemm) return ls;
  if (!split) return swiglu ? launch_swiglu_quant(y_bf16, m, n / 2, h_fp8, h_scale, stream) : ls;
  if (swiglu) {
    const float* part = p.part;
    int sk = c.split_k, mm = (int)m, nn = (int)n;
    uint16_t* y = p.y;
    void* sargs[] = {&part, &sk, &mm, &nn, &y, &h_fp8, &h_scale};
    g_counts[CNT_RED]++;
    return launch(reinterpret_cast<const void*>(splitk_reduce_swiglu_kernel),
                  dim3((unsigned)(n / (2 * BLK)), (unsigned)m), dim3(64), 0, stream, sargs);
  }
  const float* part = p.part;
  int sk = c.split_k;
  int64_t mn4 = m * n / 4;
  uint16_t* y = p.y;
  void* rargs[] = {&part, &sk, &mn4, &y};
  g_counts[CNT_RED]++;
  return launch(reinterpret_cast<const void*>(splitk_reduce_kernel),
                dim3((unsigned)((mn4 + 255) / 256)), dim3(256), 0, stream, rargs);
}

}  // namespace

extern "C" {

fp8bs_status fp8bs_quantize_weight(const void* w_bf16, int64_t n, int64_t k, uint8_t* w_fp8,
                                   float* w_scale, void* stream) {
  if (n < 0 || k < 0 || n % BLK || k % BLK) return FP8BS_ERR_SHAPE;
  if (n / BLK > 0x7FFFFFFF || k / BLK > 65535) return FP8BS_ERR_SHAPE;
  if (n == 0 || k == 0) return FP8BS_OK;
  if (!w_bf16 || !w_fp8 || !w_scale) return FP8BS_ERR_NULL;
  if (!aligned(w_bf16, 16) || !aligned(w_fp8, 16) || !aligned(w_scale, 4)) return FP8BS_ERR_ALIGN;
  const fp8bs_status st = current_device(nullptr);
  if (st != FP8BS_OK) return st;
  const uint16_t* w = static_cast<const uint16_t*>(w_bf16);
  int64_t kk = k;
  void* args[] = {&w, &kk, &w_fp8, &w_scale};
  g_counts[CNT_QW]++;
  return launch(reinterpret_cast<const void*>(quant_weight_kernel),
                dim3((unsigned)(n / BLK), (unsigned)(k / BLK)), dim3(256), 0, stream, args);
}

fp8bs_status fp8bs_quantize_act(const void* x_bf16, int64_t m, int64_t k, uint8_t* x_fp8,
                                float* x_scale, void* stream) {
  if (m < 0 || k < 0 || k % BLK) return FP8BS_ERR_SHAPE;
  if (m == 0 || k == 0) return FP8BS_OK;
  const int64_t nblocks = m * (k / BLK);
  if (nblocks > ((int64_t)1 << 36)) return FP8BS_ERR_SHAPE;
  if (!x_bf16 || !x_fp8 || !x_scale) return FP8BS_ERR_NULL;
  if (!aligned(x_bf16, 16) || !aligned(x_fp8, 16) || !aligned(x_scale, 4)) return FP8BS_ERR_ALIGN;
  const fp8bs_status st = current_device(nullptr);
  if (st != FP8BS_OK) return st;
  const uint16_t* x = static_cast<const uint16_t*>(x_bf16);
  int64_t nb = nblocks, kk = k;
  void* args[] = {&x, &nb, &kk, &x_fp8, &x_scale};
  g_counts[CNT_QA]++;
  return launch(reinterpret_cast<const void*>(quant_act_kernel),
                dim3((unsigned)((nblocks * 4 + 255) / 256)), dim3(256), 0, stream, args);
}

fp8bs_status fp8bs_gemm(const void* x_bf16, int64_t m, const uint8_t* w_fp8, const float* w_scale,
                        int64_t n, int64_t k, void* y_bf16, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return gemm_impl(true, x_bf16, nullptr, nullptr, m, w_fp8, w_scale, n, k, y_bf16, workspace,
                   workspace_bytes, nullptr, stream);
}

fp8bs_status fp8bs_gemm_noalloc(const void* x_bf16, int64_t m, const uint8_t* w_fp8,
                                const float* w_scale, int64_t n, int64_t k, void* y_bf16,
                                void* stream) {
  // the same checks as fp8bs_gemm, in the same order; the workspace is the
  // library's fixed scratch, so a configuration needing more is rejected
  // (FP8BS_ERR_WORKSPACE) before anything is launched
  if (!gemm_shape_ok(m, n, k, false)) return FP8BS_ERR_SHAPE;
  if (m == 0 || n == 0) return FP8BS_OK;
  if (!y_bf16 || (k > 0 && (!x_bf16 || !w_fp8 || !w_scale))) return FP8BS_ERR_NULL;
  fp8bs_gemm_config c;
  if (k > 0) {
    if (!select_config(m, n, k, &c)) return FP8BS_ERR_SHAPE;
    if (cfg_workspace(c, m, n, k, true) > kNoAllocScratchBytes) return FP8BS_ERR_WORKSPACE;
  }
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return FP8BS_ERR_DEVICE;
  }
  const fp8bs_status st = current_device(nullptr);
  if (st != FP8BS_OK) return st;
  void* ws = scratch_address(dev);
  if (!ws) return FP8BS_ERR_DEVICE;
  return gemm_impl(true, x_bf16, nullptr, nullptr, m, w_fp8, w_scale, n, k, y_bf16, ws,
                   kNoAllocScratchBytes, nullptr, stream);
}

size_t fp8bs_gemm_noalloc_max_scratch(void) { return kNoAllocScratchBytes; }

fp8bs_status fp8bs_gemm_q(const uint8_t* x_fp8, const float* x_scale, int64_t m,
                          const uint8_t* w_fp8, const float* w_scale, int64_t n, int64_t k,
                          void* y_bf16, void* workspace, size_t workspace_bytes, void* stream) {
  return gemm_impl(false, nullptr, x_fp8, x_scale, m, w_fp8, w_scale, n, k, y_bf16, workspace,
                   workspace_bytes, nullptr, stream);
}

size_t fp8bs_gemm_workspace_bytes(int64_t m, int64_t n, int64_t k) {
  fp8bs_gemm_config c;
  if (!select_config(m, n, k, &c)) return 0;
  if (m == 0 || n == 0 || k == 0) return 0;
  size_t need = cfg_workspace(c, m, n, k, true);
  // enough for the tile-layout calls as well (they may select a split grid)
  if (select_config(m, n, k, &c, false, FP8BS_LAYOUT_TILES)) {
    const size_t t = cfg_workspace(c, m, n, k, true);
    need = t > need ? t : need;
  }
  return need;
}

fp8bs_status fp8bs_gemm_select_config(int64_t m, int64_t n, int64_t k, fp8bs_gemm_config* out) {
  if (!out) return FP8BS_ERR_NULL;
  if (!select_config(m, n, k, out)) return FP8BS_ERR_SHAPE;
  return FP8BS_OK;
}

size_t fp8bs_gemm_config_workspace_bytes(const fp8bs_gemm_config* cfg, int64_t m, int64_t n,
                                         int64_t k) {
  if (!cfg || m <= 0 || n <= 0 || k <= 0) return 0;
  return cfg_workspace(*cfg, m, n, k, true);
}

fp8bs_status fp8bs_gemm_ex(const void* x_bf16, const uint8_t* x_fp8, const float* x_scale,
                           int64_t m, const uint8_t* w_fp8, const float* w_scale, int64_t n,
                           int64_t k, void* y_bf16, void* workspace, size_t workspace_bytes,
                           const fp8bs_gemm_config* cfg, void* stream) {
  if (!gemm_shape_ok(m, n, k, false)) return FP8BS_ERR_SHAPE;
  if (!cfg) return FP8BS_ERR_NULL;
  return gemm_impl(x_bf16 != nullptr, x_bf16, x_fp8, x_scale, m, w_fp8, w_scale, n, k, y_bf16,
                   workspace, workspace_bytes, cfg, stream);
}

fp8bs_status fp8bs_pack_weight(const uint8_t* w_fp8, int64_t n, int64_t k, uint8_t* w_tiles,
                               void* stream) {
  if (n < 0 || k < 0 || n % BLK || k % BLK) return FP8BS_ERR_SHAPE;
  if (n / BLK >= (int64_t)1 << 24 || k / BLK > (int64_t)1 << 20) return FP8BS_ERR_SHAPE;
  if (n == 0 || k == 0) return FP8BS_OK;
  // one thread per 16 bytes, 256 per workgroup: the grid must fit in 2^31 - 1
  if ((n / 16) * (k / 256) > (int64_t)0x7FFFFFFF) return FP8BS_ERR_SHAPE;
  if (!w_fp8 || !w_tiles) return FP8BS_ERR_NULL;
  if (!aligned(w_fp8, 16) || !aligned(w_tiles, 16)) return FP8BS_ERR_ALIGN;
  const fp8bs_status st = current_device(nullptr);
  if (st != FP8BS_OK) return st;
  const uint4* src = reinterpret_cast<const uint4*>(w_fp8);
  uint4* dst = reinterpret_cast<uint4*>(w_tiles);
  int64_t chunks = n * k / 16, kc = k / 16, kbn = k / BLK;
  void* args[] = {&src, &chunks, &kc, &kbn, &dst};
  g_counts[CNT_PACK]++;
  return launch(reinterpret_cast<const void*>(pack_weight_kernel),
                dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, stream, args);
}

fp8bs_status fp8bs_gemm_tiles(const void* x_bf16, int64_t m, const uint8_t* w_tiles,
                              const float* w_scale, int64_t n, int64_t k, void* y_bf16,
                              void* workspace, size_t workspace_bytes, void* stream) {
  return gemm_impl(true, x_bf16, nullptr, nullptr, m, w_tiles, w_scale, n, k, y_bf16, workspace,
                   workspace_bytes, nullptr, stream, false, nullptr, nullptr, FP8BS_LAYOUT_TILES);
}

fp8bs_status fp8bs_gemm_q_tiles(const uint8_t* x_fp8, const float* x_scale, int64_t m,
                                const uint8_t* w_tiles, const float* w_scale, int64_t n,
                                int64_t k, void* y_bf16, void* workspace, size_t workspace_bytes,
                                void* stream) {
  return gemm_impl(false, nullptr, x_fp8, x_scale, m, w_tiles, w_scale, n, k, y_bf16, workspace,
                   workspace_bytes, nullptr, stream, false, nullptr, nullptr, FP8BS_LAYOUT_TILES);
}

fp8bs_status fp8bs_gemm_tiles_select_config(int64_t m, int64_t n, int64_t k,
                                            fp8bs_gemm_config* out) {
  if (!out) return FP8BS_ERR_NULL;
  if (!select_config(m, n, k, out, false, FP8BS_LAYOUT_TILES)) return FP8BS_ERR_SHAPE;
  return FP8BS_OK;
}

fp8bs_status fp8bs_swiglu_quant(const void* y_bf16, int64_t m, int64_t inter, uint8_t* h_fp8,
                               float* h_scale, void* stream) {
  if (m < 0 || inter < 0 || inter % BLK) return FP8BS_ERR_SHAPE;
  if (m == 0 || inter == 0) return FP8BS_OK;
  if (inter / BLK > 0x7FFFFFFF || m > 65535) return FP8BS_ERR_SHAPE;
  if (!y_bf16 || !h_fp8 || !h_scale) return FP8BS_ERR_NULL;
  if (!aligned(y_bf16, 16) || !aligned(h_fp8, 16) || !aligned(h_scale, 4)) return FP8BS_ERR_ALIGN;
  const fp8bs_status st = current_device(nullptr);
  if (st != FP8BS_OK) return st;
  return launch_swiglu_quant(y_bf16, m, inter, h_fp8, h_scale, stream);
}

fp8bs_status fp8bs_gemm_swiglu(const void* x_bf16, int64_t m, const uint8_t* w_fp8,
                               const float* w_scale, int64_t n, int64_t k, void* y_bf16,
                               uint8_t* h_fp8, float* h_scale, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return gemm_impl(true, x_bf16, nullptr, nullptr, m, w_fp8, w_scale, n, k, y_bf16, workspace,
                   workspace_bytes, nullptr, stream, true, h_fp8, h_scale);
}

fp8bs_status fp8bs_gemm_swiglu_tiles(const void* x_bf16, int64_t m, const uint8_t* w_tiles,
                                     const float* w_scale, int64_t n, int64_t k, void* y_bf16,
                                     uint8_t* h_fp8, float* h_scale, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  return gemm_impl(true, x_bf16, nullptr, nullptr, m, w_tiles, w_scale, n, k, y_bf16, workspace,
                   workspace_bytes, nullptr, stream, true, h_fp8, h_scale, FP8BS_LAYOUT_TILES);
}

fp8bs_status fp8bs_gemm_swiglu_ex(const void* x_bf16, const uint8_t* x_fp8, const float* x_scale,
                                  int64_t m, const uint8_t* w_fp8, const float* w_scale,
                                  int64_t n, int64_t k, void* y_bf16, uint8_t* h_fp8,
                                  float* h_scale, void* workspace, size_t workspace_bytes,
                                  const fp8bs_gemm_config* cfg, void* stream) {
  if (!gemm_shape_ok(m, n, k, true)) return FP8BS_ERR_SHAPE;
  if (!cfg) return FP8BS_ERR_NULL;
  return gemm_impl(x_bf16 != nullptr, x_bf16, x_fp8, x_scale, m, w_fp8, w_scale, n, k, y_bf16,
                   workspace, workspace_bytes, cfg, stream, true, h_fp8, h_scale);
}

fp8bs_status fp8bs_gemm_swiglu_select_config(int64_t m, int64_t n, int64_t k,
                                             fp8bs_gemm_config* out) {
  if (!out) return FP8BS_ERR_NULL;
  if (!select_config(m, n, k, out, true)) return FP8BS_ERR_SHAPE;
  return FP8BS_OK;
}

size_t fp8bs_gemm_swiglu_workspace_bytes(const fp8bs_gemm_config* cfg, int64_t m, int64_t n,
                                         int64_t k) {
  fp8bs_gemm_config c;
  if (cfg) {
    c = *cfg;
  } else if (!select_config(m, n, k, &c, true)) {
    return 0;
  }
  if (m <= 0 || n <= 0 || k <= 0 || n % (2 * BLK)) return 0;
  return swiglu_workspace(c, m, n, k, true);
}

fp8bs_status fp8bs_encode_e4m3(const float* in, int64_t count, uint8_t* out, int32_t mode,
                               void* stream) {
  if (count < 0 || mode < 0 || mode > 2) return FP8BS_ERR_SHAPE;
  if (count == 0) return FP8BS_OK;
  if (!in || !out) return FP8BS_ERR_NULL;
  if (!aligned(in, 4) || !aligned(out, 4)) return FP8BS_ERR_ALIGN;
  const fp8bs_status st = current_device(nullptr);
  if (st != FP8BS_OK) return st;
  int64_t cnt = count;
  int md = mode;
  void* args[] = {&in, &cnt, &out, &md};
  g_counts[CNT_ENC]++;
  return launch(reinterpret_cast<const void*>(encode_kernel),
                dim3((unsigned)(((count + 3) / 4 + 255) / 256)), dim3(256), 0, stream, args);
}

int32_t fp8bs_streamk_plan_check(int64_t n, int64_t k, int32_t split, int32_t workgroups,
                                 int32_t whole) {
  if (n <= 0 || k <= 0 || n % BLK || k % BLK || workgroups < 1 || split < 1) return 1;
  if (n / 16 > 0x7FFFFFFF || k / BLK > 0x7FFFFFFF || whole < 0 || whole > 1) return 1;
  const SkPlan q = sk_plan((int)(n / 16), (int)(k / BLK), split, workgroups, whole);
  if (!sk_plan_ok(q)) return 1;
  const int64_t units = (int64_t)q.ntiles * q.kbn;
  if (units > ((int64_t)1 << 28)) return 1;  // keep the check's own memory small
  std::vector<uint8_t> cover((size_t)units, 0);
  // per tile: (first absolute K block, slot) of each segment
  std::vector<std::vector<std::pair<int, int64_t>>> segs((size_t)q.ntiles);
  const int64_t nslots = sk_slot_count(q);
  for (int w = 0; w < q.P; ++w) {
    int nsk;
    const int nseg = sk_segments(q, w, &nsk);
    if (nseg < 1) return 2;
    const int chunk = sk_chunk_of(q, w);
    for (int i = 0; i < nseg; ++i) {
      const SkSegment g = sk_segment(q, w, nsk, i);
      if (g.chunk != chunk) return 3;  // staged activations cover one chunk
      if (g.b0 < 0 || g.b1 > q.kc || g.b0 >= g.b1 || g.tile < 0 || g.tile >= q.ntiles) return 4;
      if (g.slot >= nslots) return 5;
      for (int b = g.b0; b < g.b1; ++b) {
        uint8_t& c = cover[(size_t)g.tile * q.kbn + (size_t)g.chunk * q.kc + b];
        if (c) return 6;  // a unit computed twice
        c = 1;
      }
      segs[g.tile].push_back({g.chunk * q.kc + g.b0, g.slot});
    }
  }
  for (uint8_t c : cover)
    if (!c) return 7;  // a unit never computed
  std::vector<uint8_t> used((size_t)nslots, 0);
  for (int t = 0; t < q.ntiles; ++t) {
    std::vector<std::pair<int, int64_t>>& v = segs[t];
    std::sort(v.begin(), v.end());
    int64_t slots[SK_MAXPIECES];
    const int np = sk_tile_pieces(q, t, slots);
    if (np != (int)v.size() || np > SK_MAXPIECES) return 8;
    if (np == 1 && (q.S != 1 || v[0].first != 0)) return 9;  // written directly: a whole tile
    for (int i = 0; i < np; ++i) {
      if (slots[i] != v[i].second) return 10;  // summation order = K order
      if (np > 1) {
        if (slots[i] < 0 || slots[i] >= nslots) return 5;
        if (used[(size_t)slots[i]]) return 11;  // two pieces in one slot
        used[(size_t)slots[i]] = 1;
      }
    }
  }
  return 0;
}

const char* fp8bs_status_string(fp8bs_status s) {
  switch (s) {
    case FP8BS_OK: return "FP8BS_OK";
    case FP8BS_ERR_NULL: return "FP8BS_ERR_NULL: a required pointer is NULL";
    case FP8BS_ERR_SHAPE: return "FP8BS_ERR_SHAPE: unsupported shape (n, k must be multiples of 128; an extent is negative or beyond its documented limit)";
    case FP8BS_ERR_ALIGN: return "FP8BS_ERR_ALIGN: pointer misaligned";
    case FP8BS_ERR_WORKSPACE: return "FP8BS_ERR_WORKSPACE: workspace missing or too small";
    case FP8BS_ERR_DEVICE: return "FP8BS_ERR_DEVICE: no current HIP device or not gfx950";
    case FP8BS_ERR_LAUNCH: return "FP8BS_ERR_LAUNCH: kernel launch failed";
    case FP8BS_ERR_CONFIG: return "FP8BS_ERR_CONFIG: kernel configuration invalid for this shape";
  }
  return "FP8BS_ERR_UNKNOWN";
}

uint64_t fp8bs_launch_count(int32_t which) {
  if (which < 0 || which >= 9) return 0;
  return g_counts[which].load();
}

#ifndef FP8BS_BUILD_FLAGS
#define FP8BS_BUILD_FLAGS "unknown"
#endif

const char* fp8bs_build_info(void) {
#if FP8BS_ENCODER_SW
#define FP8BS_ENC_NAME "software"
#else
#define FP8BS_ENC_NAME "hardware"
#endif
  return "fp8bs gfx950; encoder=" FP8BS_ENC_NAME "; flags=" FP8BS_BUILD_FLAGS;
}

fp8bs_status fp8bs_diag_read(const void* src, size_t bytes, void* sink, int32_t blocks,
                             void* stream) {
  if (bytes % 16 || blocks < 0) return FP8BS_ERR_SHAPE;
  if (bytes == 0) return FP8BS_OK;
  if (!src || !sink) return FP8BS_ERR_NULL;
  if (!aligned(src, 16) || !aligned(sink, 16)) return FP8BS_ERR_ALIGN;
  DeviceInfo dev;
  const fp8bs_status st = current_device(&dev);
  if (st != FP8BS_OK) return st;
  const uint4* s = static_cast<const uint4*>(src);
  int64_t n16 = (int64_t)(bytes / 16);
  uint32_t* sk = static_cast<uint32_t*>(sink);
  int64_t want = (n16 + 1023) / 1024;  // about 4 loads per lane
  const int64_t cap = (int64_t)dev.num_cu * 16;
  if (want > cap) want = cap;
  if (want < 1) want = 1;
  if (blocks > 0) want = blocks;
  void* args[] = {&s, &n16, &sk};
  g_counts[CNT_DIAG]++;
  return launch(reinterpret_cast<const void*>(diag_read_kernel), dim3((unsigned)want), dim3(256),
                0, stream, args);
}

fp8bs_status fp8bs_diag_stream(const void* src, size_t bytes, void* sink, int32_t blocks,
                               int32_t depth, void* stream) {
  if (bytes % 16 || blocks < 1 || (depth != 0 && depth != 4 && depth != 8 && depth != 16))
    return FP8BS_ERR_SHAPE;
  if (bytes == 0) return FP8BS_OK;
  const int64_t per = ((int64_t)bytes / 16 + blocks - 1) / blocks * 16;
  if (per >= ((int64_t)1 << 31) - (int64_t)3 * 512 * 16 * 16) return FP8BS_ERR_SHAPE;
  if (!src || !sink) return FP8BS_ERR_NULL;
  if (!aligned(src, 16) || !aligned(sink, 16)) return FP8BS_ERR_ALIGN;
  const fp8bs_status st = current_device(nullptr);
  if (st != FP8BS_OK) return st;
  const uint8_t* s8 = static_cast<const uint8_t*>(src);
  int64_t nb = (int64_t)bytes, pr = per;
  uint32_t* sk = static_cast<uint32_t*>(sink);
  if (depth == 0) {
    void* largs[] = {&s8, &nb, &pr};
    g_counts[CNT_DIAG]++;
    return launch(reinterpret_cast<const void*>(diag_stream_lds_kernel), dim3((unsigned)blocks),
                  dim3(256), 0, stream, largs);
  }
  void* args[] = {&s8, &nb, &pr, &sk};
  const void* fn = depth == 4 ? reinterpret_cast<const void*>(diag_stream_kernel<4>)
                   : depth == 8 ? reinterpret_cast<const void*>(diag_stream_kernel<8>)
                                : reinterpret_cast<const void*>(diag_stream_kernel<16>);
  g_counts[CNT_DIAG]++;
  return launch(fn, dim3((unsigned)blocks), dim3(512), 0, stream, args);
}

fp8bs_status fp8bs_diag_timestamp(uint64_t* out, void* stream) {
  if (!out) return FP8BS_ERR_NULL;
  if (!aligned(out, 8)) return FP8BS_ERR_ALIGN;
  const fp8bs_status st = current_device(nullptr);
  if (st != FP8BS_OK) return st;
  unsigned long long* o = reinterpret_cast<unsigned long long*>(out);
  void* args[] = {&o};
  g_counts[CNT_DIAG]++;
  return launch(reinterpret_cast<const void*>(diag_timestamp_kernel), dim3(1), dim3(64), 0,
                stream, args);
}

uint64_t fp8bs_diag_timestamp_hz(void) {
  int dev = -1, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return (uint64_t)khz * 1000u;
}

fp8bs_status fp8bs_diag_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (bytes % 16) return FP8BS_ERR_SHAPE;
  if (bytes == 0) return FP8BS_OK;
  if (!src || !dst) return FP8BS_ERR_NULL;
  if (!aligned(src, 16) || !aligned(dst, 16)) return FP8BS_ERR_ALIGN;
  DeviceInfo dev;
  const fp8bs_status st = current_device(&dev);
  if (st != FP8BS_OK) return st;
  const uint4* s = static_cast<const uint4*>(src);
  uint4* d = static_cast<uint4*>(dst);
  int64_t n16 = (int64_t)(bytes / 16);
  int64_t want = (n16 + 255) / 256;
  const int64_t cap = (int64_t)dev.num_cu * 16;
  if (want > cap) want = cap;
  void* args[] = {&s, &d, &n16};
  g_counts[CNT_DIAG]++;
  return launch(reinterpret_cast<const void*>(diag_copy_kernel), dim3((unsigned)want), dim3(256),
                0, stream, args);
}

}  // extern "C"
