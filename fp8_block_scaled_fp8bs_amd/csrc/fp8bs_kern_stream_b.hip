// Instantiations of the streaming row-range GEMM kernel (waves along K,
// tiles in flight per wave) registered in the kernel table.
#include "fp8bs_registry.h"

namespace fp8bs {
static KernelRegistrar reg_stream_b({
    FP8BS_STREAM_ENTRY(16, 2)
    FP8BS_STREAM_ENTRY(16, 3)
    FP8BS_STREAM_ENTRY(4, 8)
    FP8BS_STREAM_ENTRY(16, 5)
    FP8BS_STREAM_ENTRY(8, 8)
});
}  // namespace fp8bs
