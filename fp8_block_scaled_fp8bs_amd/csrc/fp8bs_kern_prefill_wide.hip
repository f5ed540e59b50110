// Prefill-size GEMM kernels with wide wave tiles (8 waves, 16 JM x 128
// outputs per wave): 256 x 256 (JM = 4) and 192 x 256 (JM = 3) output tiles
// with two LDS stages, on row-major and tile-layout weights. A configuration
// selects them with waves_n 2, waves_k = JM, depth 2, and tiles_n 3 (grid
// schedule, K split over grid z) or 4 (1-D schedule: whole tiles in
// complete rounds, the rest as half tiles); tiles_n 5 runs (64 JM) x 160
// tiles (5 weight subtiles per wave) on the 1-D schedule, for n a
// multiple of 160.
#include "fp8bs_prefill.h"
#include "fp8bs_registry.h"

namespace fp8bs {
static KernelRegistrar reg_prefill_wide({
    {5, 1, PF_WIDE, 2, 4, 2, 0, gemm_prefill_wide_kernel<4, 2>, 0},
    {5, 1, PF_WIDE, 2, 4, 2, 0, gemm_prefill_wide_kernel<4, 2, true>, 0, 1},
    {5, 1, PF_WIDE_1D, 2, 4, 2, 0, gemm_prefill_wide_kernel<4, 2>, 0},
    {5, 1, PF_WIDE_1D, 2, 4, 2, 0, gemm_prefill_wide_kernel<4, 2, true>, 0, 1},
    {5, 1, PF_WIDE, 2, 3, 2, 0, gemm_prefill_wide_kernel<3, 2>, 0},
    {5, 1, PF_WIDE, 2, 3, 2, 0, gemm_prefill_wide_kernel<3, 2, true>, 0, 1},
    {5, 1, PF_WIDE_1D, 2, 3, 2, 0, gemm_prefill_wide_kernel<3, 2>, 0},
    {5, 1, PF_WIDE_1D, 2, 3, 2, 0, gemm_prefill_wide_kernel<3, 2, true>, 0, 1},
    {5, 1, PF_WIDE_160, 2, 4, 2, 0, gemm_prefill_wide_kernel<4, 2, false, PFW_NARROW_N>, 0},
    {5, 1, PF_WIDE_160, 2, 4, 2, 0, gemm_prefill_wide_kernel<4, 2, true, PFW_NARROW_N>, 0, 1},
    {5, 1, PF_WIDE_160, 2, 3, 2, 0, gemm_prefill_wide_kernel<3, 2, false, PFW_NARROW_N>, 0},
    {5, 1, PF_WIDE_160, 2, 3, 2, 0, gemm_prefill_wide_kernel<3, 2, true, PFW_NARROW_N>, 0, 1},
});
}  // namespace fp8bs
