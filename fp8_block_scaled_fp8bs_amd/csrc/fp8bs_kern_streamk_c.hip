// Instantiations of the stream-K decode kernel: 8 streaming waves, 6
// tiles in flight per wave, 3 of them requested before the activation cast.
#include "fp8bs_registry.h"

namespace fp8bs {
static KernelRegistrar reg_streamk_c({
    FP8BS_STREAMK_ENTRY(8, 6, 3)
});
}  // namespace fp8bs
