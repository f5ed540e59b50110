// Instantiations of the stream-K decode kernel: 8 streaming waves, 7
// tiles in flight per wave, 2 of them requested before the activation cast.
#include "fp8bs_registry.h"

namespace fp8bs {
static KernelRegistrar reg_streamk_a({
    FP8BS_STREAMK_ENTRY(8, 7, 2)
});
}  // namespace fp8bs
