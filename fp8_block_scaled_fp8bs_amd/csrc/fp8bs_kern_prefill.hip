// The prefill-size GEMM kernels registered in the kernel table: 4 waves on
// 128 x 128 output tiles and 8 waves on 256 x 128 tiles, with a one-block
// register pipeline (depth 1) or a ring of `depth` LDS stages filled by
// direct global-to-LDS loads, refilled when the next block starts
// (tiles_n 1) or as soon as a block's operands are in registers (tiles_n 2);
// the direct-load kernel also on tile-layout weights (4 and 8 waves, 2 stages).
#include "fp8bs_prefill.h"
#include "fp8bs_registry.h"

namespace fp8bs {
static KernelRegistrar reg_prefill({
    {5, 1, 1, 2, 2, 1, 0, gemm_prefill_kernel<2>, 0},
    {5, 1, 1, 4, 2, 1, 0, gemm_prefill_kernel<4>, 0},
    {5, 1, 1, 2, 2, 2, 0, gemm_prefill_dma_kernel<2, 2>, 0},
    {5, 1, 1, 2, 2, 4, 0, gemm_prefill_dma_kernel<2, 4>, 0},
    {5, 1, 1, 4, 2, 2, 0, gemm_prefill_dma_kernel<4, 2>, 0},
    {5, 1, 1, 4, 2, 3, 0, gemm_prefill_dma_kernel<4, 3>, 0},
    {5, 1, 2, 2, 2, 2, 0, gemm_prefill_dma_kernel<2, 2, true>, 0},
    {5, 1, 2, 4, 2, 2, 0, gemm_prefill_dma_kernel<4, 2, true>, 0},
    {5, 1, 2, 4, 2, 3, 0, gemm_prefill_dma_kernel<4, 3, true>, 0},
    // the same direct-load kernel reading tile-layout weights
    {5, 1, 1, 2, 2, 2, 0, gemm_prefill_dma_kernel<2, 2, false, true>, 0, 1},
    {5, 1, 1, 4, 2, 2, 0, gemm_prefill_dma_kernel<4, 2, false, true>, 0, 1},
});
}  // namespace fp8bs
