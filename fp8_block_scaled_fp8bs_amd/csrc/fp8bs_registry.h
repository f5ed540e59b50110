// Table of the compiled GEMM kernel variants. Each instantiation unit adds
// its kernels at load time; the host code looks a configuration up here.
#pragma once

#include <vector>

#include "fp8bs_gemm.h"
#include "fp8bs_rows_dma.h"
#include "fp8bs_streamk.h"

namespace fp8bs {

struct KernelEntry {
  int path;    // 1 = MFMA grid, 2 = DOT grid, 3 = MFMA row range (one workgroup per CU),
               // 4 = MFMA streaming row range, 5 = prefill-size tiled MFMA GEMM,
               // 6 = MFMA row range with register-resident activations, 7 = stream-K,
               // 8 = MFMA row range with the weight stream through LDS
  int mt;      // MFMA: 16-row activation tiles (1: m <= 16, 2: m <= 32); DOT: max m
  int tn;      // MFMA: 16-row weight tiles per wave; DOT: 8-row groups per wave
  int wn, wk, d;
  int fused;   // activations cast in the kernel (1) or given as codes and scales (0)
  void (*fn)(GemmParams);
  int variant = 0;  // row-range kernels: 1 = SwiGLU epilogue, 2 = K split (fp32 partials)
  int layout = 0;   // weight codes: 0 = row-major [n][k], 1 = tile layout (fp8bs_pack_weight)
};

std::vector<KernelEntry>& kernel_registry();

struct KernelRegistrar {
  KernelRegistrar(std::initializer_list<KernelEntry> l) {
    for (const KernelEntry& e : l) kernel_registry().push_back(e);
  }
};

}  // namespace fp8bs

#define FP8BS_MFMA_ENTRY(TN, WN, WK, D)                                   \
  {1, 1, TN, WN, WK, D, 1, gemm_mfma_kernel<1, TN, WN, WK, D, true>},     \
  {1, 2, TN, WN, WK, D, 1, gemm_mfma_kernel<2, TN, WN, WK, D, true>},     \
  {1, 1, TN, WN, WK, D, 0, gemm_mfma_kernel<1, TN, WN, WK, D, false>},    \
  {1, 2, TN, WN, WK, D, 0, gemm_mfma_kernel<2, TN, WN, WK, D, false>},

// The same kernels reading weights in the tile layout.
#define FP8BS_MFMA_TILES_ENTRY(TN, WN, WK, D)                                            \
  {1, 1, TN, WN, WK, D, 1, gemm_mfma_kernel<1, TN, WN, WK, D, true, true>, 0, 1},        \
  {1, 2, TN, WN, WK, D, 1, gemm_mfma_kernel<2, TN, WN, WK, D, true, true>, 0, 1},        \
  {1, 1, TN, WN, WK, D, 0, gemm_mfma_kernel<1, TN, WN, WK, D, false, true>, 0, 1},       \
  {1, 2, TN, WN, WK, D, 0, gemm_mfma_kernel<2, TN, WN, WK, D, false, true>, 0, 1},

// Row-range kernel with the weight stream through LDS (tile layout, m <= 16):
// the config's depth field holds the ring's stages.
#define FP8BS_ROWS_DMA_ENTRY(S)                                          \
  {8, 1, 1, 1, RD_WK, S, 1, gemm_rows_dma_kernel<S, true>, 0, 1},        \
  {8, 1, 1, 1, RD_WK, S, 0, gemm_rows_dma_kernel<S, false>, 0, 1},

#define FP8BS_DOT_ENTRY(RT, WN, WK, D)                                    \
  {2, 1, RT, WN, WK, D, 1, gemm_dot_kernel<1, RT, WN, WK, D, true>},      \
  {2, 2, RT, WN, WK, D, 1, gemm_dot_kernel<2, RT, WN, WK, D, true>},      \
  {2, 4, RT, WN, WK, D, 1, gemm_dot_kernel<4, RT, WN, WK, D, true>},      \
  {2, 1, RT, WN, WK, D, 0, gemm_dot_kernel<1, RT, WN, WK, D, false>},     \
  {2, 2, RT, WN, WK, D, 0, gemm_dot_kernel<2, RT, WN, WK, D, false>},     \
  {2, 4, RT, WN, WK, D, 0, gemm_dot_kernel<4, RT, WN, WK, D, false>},

// Row-range kernel: (waves along K, tiles in flight, of which issued before
// the activation cast). The config's tiles_n field selects the pre-cast count.
#define FP8BS_ROWS_ENTRY(WK, D, PRE)                                         \
  {3, 1, PRE, 1, WK, D, 1, gemm_rows_kernel<1, WK, D, PRE, true>},           \
  {3, 2, PRE, 1, WK, D, 1, gemm_rows_kernel<2, WK, D, PRE, true>},           \
  {3, 1, PRE, 1, WK, D, 0, gemm_rows_kernel<1, WK, D, PRE, false>},          \
  {3, 2, PRE, 1, WK, D, 0, gemm_rows_kernel<2, WK, D, PRE, false>},

#define FP8BS_ROWS_TILES_ENTRY(WK, D, PRE)                                                      \
  {3, 1, PRE, 1, WK, D, 1, gemm_rows_kernel<1, WK, D, PRE, true, ROWS_OUT_BF16, true>, 0, 1},   \
  {3, 2, PRE, 1, WK, D, 1, gemm_rows_kernel<2, WK, D, PRE, true, ROWS_OUT_BF16, true>, 0, 1},   \
  {3, 1, PRE, 1, WK, D, 0, gemm_rows_kernel<1, WK, D, PRE, false, ROWS_OUT_BF16, true>, 0, 1},  \
  {3, 2, PRE, 1, WK, D, 0, gemm_rows_kernel<2, WK, D, PRE, false, ROWS_OUT_BF16, true>, 0, 1},

// Row-range kernels with the SwiGLU epilogue, for the configurations the
// fused up/gate call selects.
#define FP8BS_ROWS_SWIGLU_ENTRY(WK, D, PRE)                                            \
  {3, 1, PRE, 1, WK, D, 1, gemm_rows_kernel<1, WK, D, PRE, true, ROWS_OUT_SWIGLU>, 1},   \
  {3, 2, PRE, 1, WK, D, 1, gemm_rows_kernel<2, WK, D, PRE, true, ROWS_OUT_SWIGLU>, 1},   \
  {3, 1, PRE, 1, WK, D, 0, gemm_rows_kernel<1, WK, D, PRE, false, ROWS_OUT_SWIGLU>, 1},  \
  {3, 2, PRE, 1, WK, D, 0, gemm_rows_kernel<2, WK, D, PRE, false, ROWS_OUT_SWIGLU>, 1},

// Row-range kernels with K split over grid.y (fp32 partials), for m where
// one workgroup's activations of the whole K range do not fit in LDS.
#define FP8BS_ROWS_SPLIT_ENTRY(WK, D, PRE)                                              \
  {3, 1, PRE, 1, WK, D, 1, gemm_rows_kernel<1, WK, D, PRE, true, ROWS_OUT_PARTIAL>, 2},   \
  {3, 2, PRE, 1, WK, D, 1, gemm_rows_kernel<2, WK, D, PRE, true, ROWS_OUT_PARTIAL>, 2},   \
  {3, 1, PRE, 1, WK, D, 0, gemm_rows_kernel<1, WK, D, PRE, false, ROWS_OUT_PARTIAL>, 2},  \
  {3, 2, PRE, 1, WK, D, 0, gemm_rows_kernel<2, WK, D, PRE, false, ROWS_OUT_PARTIAL>, 2},

// Row-range kernel with register-resident activations: (waves along K,
// K blocks per wave, weight slots requested before the cast). The config's
// depth field holds the blocks per wave, tiles_n the pre-cast count.
#define FP8BS_ROWS_REG_ENTRY(WK, NJ, PRE)                                    \
  {6, 1, PRE, 1, WK, NJ, 1, gemm_rows_reg_kernel<1, WK, NJ, PRE, true>},     \
  {6, 2, PRE, 1, WK, NJ, 1, gemm_rows_reg_kernel<2, WK, NJ, PRE, true>},     \
  {6, 1, PRE, 1, WK, NJ, 0, gemm_rows_reg_kernel<1, WK, NJ, PRE, false>},    \
  {6, 2, PRE, 1, WK, NJ, 0, gemm_rows_reg_kernel<2, WK, NJ, PRE, false>},

#define FP8BS_ROWS_REG_SWIGLU_ENTRY(WK, NJ, PRE)                                        \
  {6, 1, PRE, 1, WK, NJ, 1, gemm_rows_reg_kernel<1, WK, NJ, PRE, true, true>, 1},        \
  {6, 2, PRE, 1, WK, NJ, 1, gemm_rows_reg_kernel<2, WK, NJ, PRE, true, true>, 1},        \
  {6, 1, PRE, 1, WK, NJ, 0, gemm_rows_reg_kernel<1, WK, NJ, PRE, false, true>, 1},       \
  {6, 2, PRE, 1, WK, NJ, 0, gemm_rows_reg_kernel<2, WK, NJ, PRE, false, true>, 1},

#define FP8BS_STREAM_SWIGLU_ENTRY(WK, D)                                          \
  {4, 1, 1, 1, WK, D, 1, gemm_stream_kernel<1, WK, D, true, true>, 1},           \
  {4, 2, 1, 1, WK, D, 1, gemm_stream_kernel<2, WK, D, true, true>, 1},           \
  {4, 4, 1, 1, WK, D, 1, gemm_stream_kernel<4, WK, D, true, true>, 1},           \
  {4, 1, 1, 1, WK, D, 0, gemm_stream_kernel<1, WK, D, false, true>, 1},          \
  {4, 2, 1, 1, WK, D, 0, gemm_stream_kernel<2, WK, D, false, true>, 1},          \
  {4, 4, 1, 1, WK, D, 0, gemm_stream_kernel<4, WK, D, false, true>, 1},

// Streaming row-range kernel: (waves along K, tiles in flight); the entry's
// mt field holds the staging passes (1: m <= 8, 2: m <= 16, 4: m <= 32).
#define FP8BS_STREAM_ENTRY(WK, D)                                             \
  {4, 1, 1, 1, WK, D, 1, gemm_stream_kernel<1, WK, D, true>},                \
  {4, 2, 1, 1, WK, D, 1, gemm_stream_kernel<2, WK, D, true>},                \
  {4, 4, 1, 1, WK, D, 1, gemm_stream_kernel<4, WK, D, true>},                \
  {4, 1, 1, 1, WK, D, 0, gemm_stream_kernel<1, WK, D, false>},               \
  {4, 2, 1, 1, WK, D, 0, gemm_stream_kernel<2, WK, D, false>},               \
  {4, 4, 1, 1, WK, D, 0, gemm_stream_kernel<4, WK, D, false>},


#define FP8BS_STREAM_TILES_ENTRY(WK, D)                                                  \
  {4, 1, 1, 1, WK, D, 1, gemm_stream_kernel<1, WK, D, true, false, true>, 0, 1},        \
  {4, 2, 1, 1, WK, D, 1, gemm_stream_kernel<2, WK, D, true, false, true>, 0, 1},        \
  {4, 4, 1, 1, WK, D, 1, gemm_stream_kernel<4, WK, D, true, false, true>, 0, 1},        \
  {4, 1, 1, 1, WK, D, 0, gemm_stream_kernel<1, WK, D, false, false, true>, 0, 1},       \
  {4, 2, 1, 1, WK, D, 0, gemm_stream_kernel<2, WK, D, false, false, true>, 0, 1},       \
  {4, 4, 1, 1, WK, D, 0, gemm_stream_kernel<4, WK, D, false, false, true>, 0, 1},

#define FP8BS_ROWS_REG_TILES_ENTRY(WK, NJ, PRE)                                             \
  {6, 1, PRE, 1, WK, NJ, 1, gemm_rows_reg_kernel<1, WK, NJ, PRE, true, false, true>, 0, 1},  \
  {6, 2, PRE, 1, WK, NJ, 1, gemm_rows_reg_kernel<2, WK, NJ, PRE, true, false, true>, 0, 1},  \
  {6, 1, PRE, 1, WK, NJ, 0, gemm_rows_reg_kernel<1, WK, NJ, PRE, false, false, true>, 0, 1}, \
  {6, 2, PRE, 1, WK, NJ, 0, gemm_rows_reg_kernel<2, WK, NJ, PRE, false, false, true>, 0, 1},

// Stream-K kernel: (streaming waves, tiles in flight per wave, of which
// requested before the activation cast), both weight layouts.
#define FP8BS_STREAMK_ENTRY(WK, D, PRE)                                                   \
  {7, 1, PRE, 1, WK, D, 1, gemm_streamk_kernel<1, WK, D, PRE, true, false>, 0, 0},        \
  {7, 2, PRE, 1, WK, D, 1, gemm_streamk_kernel<2, WK, D, PRE, true, false>, 0, 0},        \
  {7, 1, PRE, 1, WK, D, 0, gemm_streamk_kernel<1, WK, D, PRE, false, false>, 0, 0},       \
  {7, 2, PRE, 1, WK, D, 0, gemm_streamk_kernel<2, WK, D, PRE, false, false>, 0, 0},       \
  {7, 1, PRE, 1, WK, D, 1, gemm_streamk_kernel<1, WK, D, PRE, true, true>, 0, 1},         \
  {7, 2, PRE, 1, WK, D, 1, gemm_streamk_kernel<2, WK, D, PRE, true, true>, 0, 1},         \
  {7, 1, PRE, 1, WK, D, 0, gemm_streamk_kernel<1, WK, D, PRE, false, true>, 0, 1},        \
  {7, 2, PRE, 1, WK, D, 0, gemm_streamk_kernel<2, WK, D, PRE, false, true>, 0, 1},
