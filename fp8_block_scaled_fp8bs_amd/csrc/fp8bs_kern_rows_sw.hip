// Instantiations of the row-range GEMM kernels with the SwiGLU epilogue
// (the configurations the fused up/gate call selects) and with K split,
// registered in the kernel table.
#include "fp8bs_registry.h"

namespace fp8bs {
static KernelRegistrar reg_rows_sw({
    FP8BS_ROWS_SWIGLU_ENTRY(8, 4, 4)
    FP8BS_ROWS_SWIGLU_ENTRY(8, 3, 1)
    FP8BS_ROWS_SWIGLU_ENTRY(8, 6, 2)
    FP8BS_STREAM_SWIGLU_ENTRY(8, 6)
    FP8BS_STREAM_SWIGLU_ENTRY(8, 4)
    FP8BS_ROWS_SPLIT_ENTRY(8, 4, 4)
    FP8BS_ROWS_SPLIT_ENTRY(8, 3, 1)
    FP8BS_ROWS_SPLIT_ENTRY(8, 6, 2)
    FP8BS_ROWS_SPLIT_ENTRY(8, 4, 2)
});
}  // namespace fp8bs
