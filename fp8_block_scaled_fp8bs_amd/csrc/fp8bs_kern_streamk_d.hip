// Instantiations of the stream-K decode kernel: 8 streaming waves, 8
// tiles in flight per wave, 4 of them requested before the activation cast.
#include "fp8bs_registry.h"

namespace fp8bs {
static KernelRegistrar reg_streamk_d({
    FP8BS_STREAMK_ENTRY(8, 8, 4)
});
}  // namespace fp8bs
