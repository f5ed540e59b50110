// Instantiations of the stream-K decode kernel: 4 streaming waves, 10
// tiles in flight per wave, 3 of them requested before the activation cast.
#include "fp8bs_registry.h"

namespace fp8bs {
static KernelRegistrar reg_streamk_e({
    FP8BS_STREAMK_ENTRY(4, 10, 3)
});
}  // namespace fp8bs
