// Table of the compiled GEMM kernel variants, shared by the translation
// units that instantiate them and the host code that picks one.
#pragma once

#include "fp8bs_gemm.h"

namespace fp8bs {

struct KernelEntry {
  int path;    // 1 = MFMA, 2 = DOT
  int mt;      // MFMA: 16-row activation tiles (1: m <= 16, 2: m <= 32); DOT: max m
  int tn;      // MFMA: 16-row weight tiles per wave; DOT: 8-row groups per wave
  int wn, wk, d;
  int fused, split;
  void (*fn)(GemmParams);
};

extern const KernelEntry g_mfma_entries[];
extern const int g_mfma_count;
extern const KernelEntry g_dot_entries[];
extern const int g_dot_count;

}  // namespace fp8bs

// (tiles_n, waves_n, waves_k, depth) shapes compiled for the MFMA path.
#define FP8BS_MFMA_SHAPES(X) \
  X(1, 1, 8, 5)              \
  X(1, 1, 4, 5)              \
  X(1, 2, 4, 5)              \
  X(1, 4, 1, 4)              \
  X(1, 4, 2, 4)              \
  X(2, 2, 2, 4)              \
  X(2, 4, 1, 4)              \
  X(2, 2, 1, 8)

// (groups_n, waves_n, waves_k, depth) shapes compiled for the DOT path.
#define FP8BS_DOT_SHAPES(X) \
  X(2, 1, 8, 5)             \
  X(2, 4, 1, 4)             \
  X(4, 2, 2, 4)
