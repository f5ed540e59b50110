// Instantiations of GEMM kernel shapes (tiles, waves along N, waves along K,
// blocks in flight) registered in the kernel table.
#include "fp8bs_registry.h"

namespace fp8bs {
static KernelRegistrar reg_mfma_g({
    FP8BS_MFMA_ENTRY(1, 8, 1, 5)
    FP8BS_MFMA_ENTRY(1, 8, 2, 2)
    FP8BS_MFMA_ENTRY(2, 4, 1, 5)
});
}  // namespace fp8bs
