// Instantiations of GEMM kernel shapes (tiles, waves along N, waves along K,
// blocks in flight) registered in the kernel table.
#include "fp8bs_registry.h"

namespace fp8bs {
static KernelRegistrar reg_dot_a({
    FP8BS_DOT_ENTRY(2, 1, 8, 5)
    FP8BS_DOT_ENTRY(2, 4, 1, 5)
    FP8BS_DOT_ENTRY(4, 2, 2, 4)
    FP8BS_DOT_ENTRY(1, 1, 8, 5)
});
}  // namespace fp8bs
