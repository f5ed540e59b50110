// Instantiations of the row-range GEMM kernel (waves along K, tiles in
// flight per wave, tiles issued before the cast) registered in the kernel
// table.
#include "fp8bs_registry.h"

namespace fp8bs {
static KernelRegistrar reg_rows_b({
    FP8BS_ROWS_ENTRY(8, 6, 2)
    FP8BS_ROWS_ENTRY(16, 2, 1)
    FP8BS_ROWS_ENTRY(16, 3, 1)
    FP8BS_ROWS_ENTRY(4, 8, 2)
});
}  // namespace fp8bs
