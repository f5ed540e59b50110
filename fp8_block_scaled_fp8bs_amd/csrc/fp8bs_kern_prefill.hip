// The prefill-size GEMM kernel registered in the kernel table.
#include "fp8bs_prefill.h"
#include "fp8bs_registry.h"

namespace fp8bs {
static KernelRegistrar reg_prefill({
    {5, 1, 1, 2, 1, 2, 0, gemm_prefill_kernel<0>, 0},
});
}  // namespace fp8bs
