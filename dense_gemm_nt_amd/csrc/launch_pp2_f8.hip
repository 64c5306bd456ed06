// Launch table of the 256x256 ping-pong kernel for one pair of FP8 operand
// formats (GNT_F8_IN = IN_F8 + 2 * (A is E5M2) + (B is E5M2)), indexed
// [scale mode][out dtype]: per-tensor scales, then blockwise; and the table of
// its grouped launches.  Compiled only through launch_pp2_f8_<formats>.hip,
// which sets GNT_F8_IN, GNT_F8_TABLE and GNT_F8_GROUPED_TABLE.
#ifndef GNT_F8_IN
#error "include through launch_pp2_f8_<formats>.hip"
#endif
#include "gemm_nt_launch.hpp"
#include "gemm_nt_pp2.hpp"

namespace gnt {

template <int SC, int OUT>
static hipError_t launch_pp2_f8(const KernelArgs &a, unsigned grid, hipStream_t s)
{
    hipLaunchKernelGGL((gemm_nt_pp2<GNT_F8_IN, OUT, false, false, SC>), dim3(grid), dim3(512), 0,
                       s, a);
    return hipGetLastError();
}

LaunchTable GNT_F8_TABLE = {
    {launch_pp2_f8<0, 0>, launch_pp2_f8<0, 1>, launch_pp2_f8<0, 2>},
    {launch_pp2_f8<1, 0>, launch_pp2_f8<1, 1>, launch_pp2_f8<1, 2>},
};

// the same formats in grouped launches (one problem per group)
template <int SC, int OUT>
static hipError_t launch_pp2_f8_grouped(const KernelArgs &a, unsigned grid, hipStream_t s)
{
    hipLaunchKernelGGL((gemm_nt_pp2<GNT_F8_IN, OUT, false, false, SC, true>), dim3(grid),
                       dim3(512), 0, s, a);
    return hipGetLastError();
}

LaunchTable GNT_F8_GROUPED_TABLE = {
    {launch_pp2_f8_grouped<0, 0>, launch_pp2_f8_grouped<0, 1>, launch_pp2_f8_grouped<0, 2>},
    {launch_pp2_f8_grouped<1, 0>, launch_pp2_f8_grouped<1, 1>, launch_pp2_f8_grouped<1, 2>},
};

}  // namespace gnt
