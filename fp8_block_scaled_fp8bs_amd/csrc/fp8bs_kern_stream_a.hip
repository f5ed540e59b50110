// Instantiations of the streaming row-range GEMM kernel (waves along K,
// tiles in flight per wave) registered in the kernel table.
#include "fp8bs_registry.h"

namespace fp8bs {
static KernelRegistrar reg_stream_a({
    FP8BS_STREAM_ENTRY(8, 4)
    FP8BS_STREAM_ENTRY(8, 2)
    FP8BS_STREAM_ENTRY(8, 6)
});
}  // namespace fp8bs
