// Instantiations of the row-range GEMM kernel (waves along K, tiles in
// flight per wave, tiles issued before the cast) registered in the kernel
// table.
#include "fp8bs_registry.h"

namespace fp8bs {
static KernelRegistrar reg_rows_a({
    FP8BS_ROWS_ENTRY(8, 4, 2)
    FP8BS_ROWS_ENTRY(8, 4, 4)
    FP8BS_ROWS_ENTRY(8, 2, 2)
    FP8BS_ROWS_ENTRY(8, 3, 1)
});
}  // namespace fp8bs
