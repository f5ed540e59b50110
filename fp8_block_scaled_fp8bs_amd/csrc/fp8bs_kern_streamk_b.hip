// Instantiations of the stream-K decode kernel: 6 streaming waves, 8
// tiles in flight per wave, 3 of them requested before the activation cast.
#include "fp8bs_registry.h"

namespace fp8bs {
static KernelRegistrar reg_streamk_b({
    FP8BS_STREAMK_ENTRY(6, 8, 3)
});
}  // namespace fp8bs
