// Instantiations of GEMM kernel shapes (tiles, waves along N, waves along K,
// blocks in flight) registered in the kernel table.
#include "fp8bs_registry.h"

namespace fp8bs {
static KernelRegistrar reg_dot_b({
    FP8BS_DOT_ENTRY(2, 1, 8, 2)
    FP8BS_DOT_ENTRY(4, 1, 8, 2)
    FP8BS_DOT_ENTRY(2, 2, 4, 4)
});
}  // namespace fp8bs
