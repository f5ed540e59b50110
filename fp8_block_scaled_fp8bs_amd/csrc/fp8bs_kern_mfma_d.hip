// Instantiations of GEMM kernel shapes (tiles, waves along N, waves along K,
// blocks in flight) registered in the kernel table.
#include "fp8bs_registry.h"

namespace fp8bs {
static KernelRegistrar reg_mfma_d({
    FP8BS_MFMA_ENTRY(4, 1, 8, 1)
    FP8BS_MFMA_ENTRY(4, 1, 4, 2)
    FP8BS_MFMA_ENTRY(2, 1, 8, 4)
});
}  // namespace fp8bs
