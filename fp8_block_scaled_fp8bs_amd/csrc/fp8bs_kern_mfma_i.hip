// Instantiations of the MFMA GEMM kernel (tiles per wave, waves along N,
// waves along K, blocks in flight) registered in the kernel table: shapes
// that keep a wave's whole K range of a split in flight at once.
#include "fp8bs_registry.h"

namespace fp8bs {
static KernelRegistrar reg_mfma_i({
    FP8BS_MFMA_ENTRY(1, 5, 1, 10)
    FP8BS_MFMA_ENTRY(2, 5, 1, 5)
    FP8BS_MFMA_ENTRY(1, 4, 1, 10)
});
}  // namespace fp8bs
