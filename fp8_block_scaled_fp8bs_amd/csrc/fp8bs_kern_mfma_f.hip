// Instantiations of GEMM kernel shapes (tiles, waves along N, waves along K,
// blocks in flight) registered in the kernel table.
#include "fp8bs_registry.h"

namespace fp8bs {
static KernelRegistrar reg_mfma_f({
    FP8BS_MFMA_ENTRY(1, 5, 1, 5)
    FP8BS_MFMA_ENTRY(1, 5, 2, 5)
    FP8BS_MFMA_ENTRY(1, 5, 2, 2)
});
}  // namespace fp8bs
