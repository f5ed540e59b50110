// Instantiations of the MFMA grid kernel reading weights in the tile layout
// (tiles per wave, waves along N, waves along K, blocks in flight): the
// shapes the configuration table selects for that layout.
#include "fp8bs_registry.h"

namespace fp8bs {
static KernelRegistrar reg_tiles_b({
    FP8BS_MFMA_TILES_ENTRY(2, 5, 1, 5)
    FP8BS_MFMA_TILES_ENTRY(1, 1, 4, 5)
    FP8BS_MFMA_TILES_ENTRY(1, 1, 8, 5)
    FP8BS_MFMA_TILES_ENTRY(4, 1, 4, 2)
    FP8BS_MFMA_TILES_ENTRY(1, 2, 4, 2)
});
}  // namespace fp8bs
