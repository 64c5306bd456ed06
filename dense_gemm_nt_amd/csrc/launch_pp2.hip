// Launch table of the 256x256 ping-pong kernel over the 16 KB-unit LDS ring
// (gemm_nt_pp2.hpp) for one operand layout, chosen by GNT_PP2_AM / GNT_PP2_BNM
// (1 = that operand MN-major) and named by GNT_PP2_TABLE.
#include "gemm_nt_launch.hpp"
#include "gemm_nt_pp2.hpp"

#ifndef GNT_PP2_TABLE
#define GNT_PP2_AM 0
#define GNT_PP2_BNM 0
#define GNT_PP2_TABLE kPP2_kk
#endif

namespace gnt {

template <int IN, int OUT>
static hipError_t launch_pp2(const KernelArgs &a, unsigned grid, hipStream_t s)
{
    hipLaunchKernelGGL((gemm_nt_pp2<IN, OUT, GNT_PP2_AM != 0, GNT_PP2_BNM != 0>), dim3(grid),
                       dim3(512), 0, s, a);
    return hipGetLastError();
}

LaunchTable GNT_PP2_TABLE = {
    {launch_pp2<0, 0>, launch_pp2<0, 1>, launch_pp2<0, 2>},
    {launch_pp2<1, 0>, launch_pp2<1, 1>, launch_pp2<1, 2>},
};

}  // namespace gnt
