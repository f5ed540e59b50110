// Instantiations of GEMM kernel shapes (tiles, waves along N, waves along K,
// blocks in flight) registered in the kernel table.
#include "fp8bs_registry.h"

namespace fp8bs {
static KernelRegistrar reg_mfma_e({
    FP8BS_MFMA_ENTRY(1, 4, 1, 5)
    FP8BS_MFMA_ENTRY(1, 4, 2, 5)
    FP8BS_MFMA_ENTRY(1, 4, 4, 2)
});
}  // namespace fp8bs
