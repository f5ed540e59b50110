// Instantiations of the DOT GEMM kernel (m <= 1, 2, 4) for every compiled
// shape, fused or pre-quantized activations, and direct or split output.
#include "fp8bs_registry.h"

namespace fp8bs {

#define FP8BS_DOT_ENTRY_M(MD, RT, WN, WK, D)                                              \
  {2, MD, RT, WN, WK, D, 1, 0, gemm_dot_kernel<MD, RT, WN, WK, D, true, false>},          \
  {2, MD, RT, WN, WK, D, 1, 1, gemm_dot_kernel<MD, RT, WN, WK, D, true, true>},           \
  {2, MD, RT, WN, WK, D, 0, 0, gemm_dot_kernel<MD, RT, WN, WK, D, false, false>},         \
  {2, MD, RT, WN, WK, D, 0, 1, gemm_dot_kernel<MD, RT, WN, WK, D, false, true>},
#define FP8BS_DOT_ENTRY(RT, WN, WK, D) \
  FP8BS_DOT_ENTRY_M(1, RT, WN, WK, D) FP8BS_DOT_ENTRY_M(2, RT, WN, WK, D) FP8BS_DOT_ENTRY_M(4, RT, WN, WK, D)

const KernelEntry g_dot_entries[] = {FP8BS_DOT_SHAPES(FP8BS_DOT_ENTRY)};
const int g_dot_count = sizeof(g_dot_entries) / sizeof(g_dot_entries[0]);

}  // namespace fp8bs
