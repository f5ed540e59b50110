// Instantiations of GEMM kernel shapes (tiles, waves along N, waves along K,
// blocks in flight) registered in the kernel table.
#include "fp8bs_registry.h"

namespace fp8bs {
static KernelRegistrar reg_mfma_b({
    FP8BS_MFMA_ENTRY(1, 1, 4, 5)
    FP8BS_MFMA_ENTRY(1, 1, 4, 8)
    FP8BS_MFMA_ENTRY(1, 2, 4, 5)
});
}  // namespace fp8bs
