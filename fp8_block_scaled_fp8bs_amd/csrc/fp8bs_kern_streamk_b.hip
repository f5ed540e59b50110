// Instantiations of the stream-K decode kernel: 8 streaming waves, 7
// tiles in flight per wave, 7 of them requested before the activation cast.
#include "fp8bs_registry.h"

namespace fp8bs {
static KernelRegistrar reg_streamk_b({
    FP8BS_STREAMK_ENTRY(8, 7, 7)
});
}  // namespace fp8bs
