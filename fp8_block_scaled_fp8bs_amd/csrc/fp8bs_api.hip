// C ABI of the library: argument checks, the fixed configuration table,
// kernel launches and launch counters. Every kernel runs on the caller's
// stream; nothing here allocates, frees or synchronizes.
#include <atomic>
#include <cstring>
#include <mutex>

#include "fp8bs.h"
#include "fp8bs_diag.h"
#include "fp8bs_quant.h"
#include "fp8bs_reduce.h"
#include "fp8bs_registry.h"

using namespace fp8bs;

namespace {

std::atomic<uint64_t> g_counts[8];

enum { CNT_QW = 0, CNT_QA = 1, CNT_MFMA = 2, CNT_DOT = 3, CNT_RED = 4, CNT_ENC = 5, CNT_DIAG = 6 };

constexpr int kMaxDevices = 64;
struct DeviceInfo {
  bool checked = false;
  bool ok = false;
  int max_lds = 0;
  int num_cu = 0;
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

fp8bs_status launch(const void* fn, dim3 grid, dim3 block, size_t lds, void* stream, void** args) {
  const hipError_t e = hipLaunchKernel(fn, grid, block, args, lds, as_stream(stream));
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return FP8BS_ERR_LAUNCH;
  }
  return FP8BS_OK;
}

// ----------------------------------------------------------- GEMM configs ---

const KernelEntry* find_kernel(const fp8bs_gemm_config& c, int m, bool fused, bool split) {
  if (c.path == FP8BS_PATH_MFMA) {
    const int mt = m <= 16 ? 1 : 2;
    for (int i = 0; i < g_mfma_count; ++i) {
      const KernelEntry& e = g_mfma_entries[i];
      if (e.mt == mt && e.tn == c.tiles_n && e.wn == c.waves_n && e.wk == c.waves_k &&
          e.d == c.depth && e.fused == (int)fused && e.split == (int)split)
        return &e;
    }
  } else if (c.path == FP8BS_PATH_DOT) {
    const int md = m <= 1 ? 1 : (m <= 2 ? 2 : 4);
    if (m > 4) return nullptr;
    for (int i = 0; i < g_dot_count; ++i) {
      const KernelEntry& e = g_dot_entries[i];
      if (e.mt == md && e.tn == c.tiles_n && e.wn == c.waves_n && e.wk == c.waves_k &&
          e.d == c.depth && e.fused == (int)fused && e.split == (int)split)
        return &e;
    }
  }
  return nullptr;
}

int config_rows(const fp8bs_gemm_config& c) {
  return (c.path == FP8BS_PATH_DOT ? 8 : 16) * c.tiles_n * c.waves_n;
}

size_t config_lds_bytes(const fp8bs_gemm_config& c, int m, int kbn) {
  const int nblk = (kbn + c.split_k - 1) / c.split_k;
  size_t red = 0;
  if (c.waves_k > 1) {
    if (c.path == FP8BS_PATH_MFMA) {
      const int mt = m <= 16 ? 1 : 2;
      red = (size_t)(c.waves_k - 1) * c.waves_n * c.tiles_n * mt * 64 * 16;
    } else {
      const int md = m <= 1 ? 1 : (m <= 2 ? 2 : 4);
      red = (size_t)(c.waves_k - 1) * c.waves_n * c.tiles_n * md * 64 * 4;
    }
  }
  return (size_t)lds_act_bytes(nblk, m) + red;
}

constexpr size_t kAutoLdsLimit = 96 * 1024;

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

// Smallest split that keeps the staged activations within the LDS limit.
int min_split_for_lds(const fp8bs_gemm_config& c, int m, int kbn) {
  fp8bs_gemm_config t = c;
  for (int s = 1; s <= kbn && s <= 64; ++s) {
    t.split_k = s;
    if (config_lds_bytes(t, m, kbn) <= kAutoLdsLimit) return s;
  }
  return -1;
}

// The fixed configuration table. A pure function of (m, n, k): no timing,
// no device state, so a shape always runs the same kernel and gives the
// same bits.
bool select_config(int64_t m, int64_t n, int64_t k, fp8bs_gemm_config* out) {
  if (m < 0 || m > 32 || n < 0 || k < 0 || n % BLK || k % BLK) return false;
  const int kbn = (int)(k / BLK);
  const int64_t nbn = n / BLK;
  fp8bs_gemm_config c;
  if (m <= 2) {
    // per-lane dot products: m multiply-adds per weight byte fit the VALU
    c = (nbn >= 256) ? make_cfg(FP8BS_PATH_DOT, 2, 4, 1, 4, 1) : make_cfg(FP8BS_PATH_DOT, 2, 1, 8, 5, 1);
  } else if (nbn >= 512) {
    c = make_cfg(FP8BS_PATH_MFMA, 2, 4, 1, 4, 1);   // 128 rows per workgroup
  } else if (nbn >= 200) {
    c = make_cfg(FP8BS_PATH_MFMA, 2, 2, 2, 4, 1);   // 64 rows, two waves over K
  } else if (kbn <= 48) {
    c = make_cfg(FP8BS_PATH_MFMA, 1, 1, 8, 5, 1);   // 16 rows, eight waves over K
  } else {
    // long K, few rows: split K across workgroups
    c = make_cfg(FP8BS_PATH_MFMA, 1, 4, 2, 4, 1);
    int s = (kbn + 7) / 8;
    if (s > 64) s = 64;
    c.split_k = s;
  }
  if (kbn > 0 && m > 0) {
    if (c.split_k > kbn) c.split_k = kbn;
    if (config_lds_bytes(c, (int)m, kbn) > kAutoLdsLimit) {
      const int s = min_split_for_lds(c, (int)m, kbn);
      if (s < 0) return false;
      c.split_k = s;
    }
  }
  if (c.split_k < 1) c.split_k = 1;
  *out = c;
  return true;
}

size_t cfg_workspace(const fp8bs_gemm_config& c, int64_t m, int64_t n) {
  return c.split_k > 1 ? (size_t)c.split_k * (size_t)m * (size_t)n * sizeof(float) : 0;
}

fp8bs_status gemm_impl(const void* x_bf16, const uint8_t* x_fp8, const float* x_scale, int64_t m,
                       const uint8_t* w_fp8, const float* w_scale, int64_t n, int64_t k,
                       void* y_bf16, void* workspace, size_t workspace_bytes,
                       const fp8bs_gemm_config* cfg_in, void* stream) {
  // shapes
  if (m < 0 || m > 32 || n < 0 || k < 0 || n % BLK || k % BLK) return FP8BS_ERR_SHAPE;
  if (n / BLK > (int64_t)1 << 24 || k / BLK > (int64_t)1 << 20) return FP8BS_ERR_SHAPE;
  if (m == 0 || n == 0) return FP8BS_OK;
  const bool fused = x_bf16 != nullptr;
  // pointers
  if (!y_bf16) return FP8BS_ERR_NULL;
  if (k > 0) {
    if (!w_fp8 || !w_scale) return FP8BS_ERR_NULL;
    if (!fused && (!x_fp8 || !x_scale)) return FP8BS_ERR_NULL;
  }
  // alignment
  if (!aligned(y_bf16, 16)) return FP8BS_ERR_ALIGN;
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
    return launch(reinterpret_cast<const void*>(zero_fill_kernel),
                  dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, stream, args);
  }
  const int kbn = (int)(k / BLK);
  // configuration
  fp8bs_gemm_config c;
  if (cfg_in) {
    c = *cfg_in;
  } else if (!select_config(m, n, k, &c)) {
    return FP8BS_ERR_SHAPE;
  }
  if (c.split_k < 1 || c.split_k > 64 || c.split_k > kbn) return FP8BS_ERR_CONFIG;
  if (c.reduce != FP8BS_REDUCE_KERNEL) return FP8BS_ERR_CONFIG;
  const bool split = c.split_k > 1;
  const KernelEntry* ke = find_kernel(c, (int)m, fused, split);
  if (!ke) return FP8BS_ERR_CONFIG;
  const int rows = config_rows(c);
  if (n % rows) return FP8BS_ERR_CONFIG;
  const size_t lds = config_lds_bytes(c, (int)m, kbn);
  // workspace
  const size_t need = cfg_workspace(c, m, n);
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return FP8BS_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return FP8BS_ERR_ALIGN;
  }
  // device
  DeviceInfo dev;
  const fp8bs_status st = current_device(&dev);
  if (st != FP8BS_OK) return st;
  if (lds > (size_t)dev.max_lds) return FP8BS_ERR_CONFIG;
  if (lds > 64 * 1024) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(ke->fn),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess) {
      (void)hipGetLastError();
      return FP8BS_ERR_LAUNCH;
    }
  }

  GemmParams p;
  p.x = static_cast<const uint16_t*>(x_bf16);
  p.xq = x_fp8;
  p.xs = x_scale;
  p.wq = w_fp8;
  p.ws = w_scale;
  p.y = static_cast<uint16_t*>(y_bf16);
  p.part = static_cast<float*>(workspace);
  p.m = (int)m;
  p.n = (int)n;
  p.k = (int)k;
  p.kbn = kbn;
  p.split = c.split_k;
  void* args[] = {&p};
  const dim3 grid((unsigned)(n / rows), (unsigned)c.split_k);
  const dim3 block(64 * c.waves_n * c.waves_k);
  g_counts[c.path == FP8BS_PATH_MFMA ? CNT_MFMA : CNT_DOT]++;
  fp8bs_status ls = launch(reinterpret_cast<const void*>(ke->fn), grid, block, lds, stream, args);
  if (ls != FP8BS_OK || !split) return ls;
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
  if (!x_bf16 && m > 0 && n > 0 && k > 0) {
    // the shape checks come first; a NULL activation pointer is a NULL error
    if (m > 32 || n % BLK || k % BLK) return FP8BS_ERR_SHAPE;
    return FP8BS_ERR_NULL;
  }
  return gemm_impl(x_bf16, nullptr, nullptr, m, w_fp8, w_scale, n, k, y_bf16, workspace,
                   workspace_bytes, nullptr, stream);
}

fp8bs_status fp8bs_gemm_q(const uint8_t* x_fp8, const float* x_scale, int64_t m,
                          const uint8_t* w_fp8, const float* w_scale, int64_t n, int64_t k,
                          void* y_bf16, void* workspace, size_t workspace_bytes, void* stream) {
  return gemm_impl(nullptr, x_fp8, x_scale, m, w_fp8, w_scale, n, k, y_bf16, workspace,
                   workspace_bytes, nullptr, stream);
}

size_t fp8bs_gemm_workspace_bytes(int64_t m, int64_t n, int64_t k) {
  fp8bs_gemm_config c;
  if (!select_config(m, n, k, &c)) return 0;
  return cfg_workspace(c, m, n);
}

fp8bs_status fp8bs_gemm_select_config(int64_t m, int64_t n, int64_t k, fp8bs_gemm_config* out) {
  if (!out) return FP8BS_ERR_NULL;
  if (!select_config(m, n, k, out)) return FP8BS_ERR_SHAPE;
  return FP8BS_OK;
}

size_t fp8bs_gemm_config_workspace_bytes(const fp8bs_gemm_config* cfg, int64_t m, int64_t n,
                                         int64_t k) {
  (void)k;
  if (!cfg || m < 0 || n < 0) return 0;
  return cfg_workspace(*cfg, m, n);
}

fp8bs_status fp8bs_gemm_ex(const void* x_bf16, const uint8_t* x_fp8, const float* x_scale,
                           int64_t m, const uint8_t* w_fp8, const float* w_scale, int64_t n,
                           int64_t k, void* y_bf16, void* workspace, size_t workspace_bytes,
                           const fp8bs_gemm_config* cfg, void* stream) {
  if (!cfg) return FP8BS_ERR_NULL;
  return gemm_impl(x_bf16, x_fp8, x_scale, m, w_fp8, w_scale, n, k, y_bf16, workspace,
                   workspace_bytes, cfg, stream);
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

const char* fp8bs_status_string(fp8bs_status s) {
  switch (s) {
    case FP8BS_OK: return "FP8BS_OK";
    case FP8BS_ERR_NULL: return "FP8BS_ERR_NULL: a required pointer is NULL";
    case FP8BS_ERR_SHAPE: return "FP8BS_ERR_SHAPE: unsupported shape (n, k must be multiples of 128; gemm m in 0..32)";
    case FP8BS_ERR_ALIGN: return "FP8BS_ERR_ALIGN: pointer misaligned";
    case FP8BS_ERR_WORKSPACE: return "FP8BS_ERR_WORKSPACE: workspace missing or too small";
    case FP8BS_ERR_DEVICE: return "FP8BS_ERR_DEVICE: no current HIP device or not gfx950";
    case FP8BS_ERR_LAUNCH: return "FP8BS_ERR_LAUNCH: kernel launch failed";
    case FP8BS_ERR_CONFIG: return "FP8BS_ERR_CONFIG: kernel configuration invalid for this shape";
  }
  return "FP8BS_ERR_UNKNOWN";
}

uint64_t fp8bs_launch_count(int32_t which) {
  if (which < 0 || which >= 8) return 0;
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
