// Instantiations of the MFMA GEMM kernel for every compiled shape, for one
// and two 16-row activation tiles, fused or pre-quantized activations, and
// direct or split output.
#include "fp8bs_registry.h"

namespace fp8bs {

#define FP8BS_MFMA_ENTRY(TN, WN, WK, D)                                                    \
  {1, 1, TN, WN, WK, D, 1, 0, gemm_mfma_kernel<1, TN, WN, WK, D, true, false>},            \
  {1, 1, TN, WN, WK, D, 1, 1, gemm_mfma_kernel<1, TN, WN, WK, D, true, true>},             \
  {1, 1, TN, WN, WK, D, 0, 0, gemm_mfma_kernel<1, TN, WN, WK, D, false, false>},           \
  {1, 1, TN, WN, WK, D, 0, 1, gemm_mfma_kernel<1, TN, WN, WK, D, false, true>},            \
  {1, 2, TN, WN, WK, D, 1, 0, gemm_mfma_kernel<2, TN, WN, WK, D, true, false>},            \
  {1, 2, TN, WN, WK, D, 1, 1, gemm_mfma_kernel<2, TN, WN, WK, D, true, true>},             \
  {1, 2, TN, WN, WK, D, 0, 0, gemm_mfma_kernel<2, TN, WN, WK, D, false, false>},           \
  {1, 2, TN, WN, WK, D, 0, 1, gemm_mfma_kernel<2, TN, WN, WK, D, false, true>},

const KernelEntry g_mfma_entries[] = {FP8BS_MFMA_SHAPES(FP8BS_MFMA_ENTRY)};
const int g_mfma_count = sizeof(g_mfma_entries) / sizeof(g_mfma_entries[0]);

}  // namespace fp8bs
