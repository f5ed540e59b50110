// Instantiations of the row-range kernel with the weight stream through LDS
// (tile-layout weights): rings of 3 and 6 stages of 16 KB. On the
// vocabulary layer 3 stages (two steps in flight) are fastest: at m = 12
// 194.6 us against 203.3 with 4 stages and 283 with 2.
#include "fp8bs_registry.h"

namespace fp8bs {
static KernelRegistrar reg_rows_dma({
    FP8BS_ROWS_DMA_ENTRY(3)
    FP8BS_ROWS_DMA_ENTRY(6)
});
}  // namespace fp8bs
