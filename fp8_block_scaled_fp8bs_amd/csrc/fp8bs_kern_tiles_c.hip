// Instantiations of the row-range kernels reading weights in the tile
// layout: row range (waves along K, tiles in flight, of which issued before
// the activation cast), streaming row range (waves along K, tiles in
// flight) and register-activation row range (waves along K, K blocks per
// wave, weight slots requested before the cast).
#include "fp8bs_registry.h"

namespace fp8bs {
static KernelRegistrar reg_tiles_c({
    FP8BS_ROWS_TILES_ENTRY(8, 4, 4)
    FP8BS_ROWS_TILES_ENTRY(8, 3, 1)
    FP8BS_ROWS_TILES_ENTRY(8, 6, 2)
    FP8BS_STREAM_TILES_ENTRY(8, 6)
    FP8BS_ROWS_REG_TILES_ENTRY(8, 5, 1)
});
}  // namespace fp8bs
