// Instantiations of GEMM kernel shapes (tiles, waves along N, waves along K,
// blocks in flight) registered in the kernel table.
#include "fp8bs_registry.h"

namespace fp8bs {
static KernelRegistrar reg_mfma_h({
    FP8BS_MFMA_ENTRY(2, 2, 2, 4)
    FP8BS_MFMA_ENTRY(2, 2, 4, 2)
    FP8BS_MFMA_ENTRY(1, 2, 8, 2)
});
}  // namespace fp8bs
