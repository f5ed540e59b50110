// Instantiations of the row-range GEMM kernel with register-resident
// activations (waves along K, K blocks per wave, weight slots issued before
// the cast) registered in the kernel table, and the configuration the
// up/gate call selects with the SwiGLU epilogue inside the GEMM.
#include "fp8bs_registry.h"

namespace fp8bs {
static KernelRegistrar reg_rows_reg({
    FP8BS_ROWS_REG_ENTRY(8, 5, 1)
    FP8BS_ROWS_REG_ENTRY(8, 5, 2)
    FP8BS_ROWS_REG_ENTRY(8, 4, 2)
    FP8BS_ROWS_REG_SWIGLU_ENTRY(8, 5, 1)
});
}  // namespace fp8bs
