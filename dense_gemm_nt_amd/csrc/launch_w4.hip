// Launch table of the four-wave 256 x 128 decode tile (gemm_nt_w4.hpp).
#include "gemm_nt_launch.hpp"
#include "gemm_nt_w4.hpp"

namespace gnt {

template <int IN, int OUT, int BN>
static hipError_t launch_w4(const KernelArgs &a, unsigned grid, hipStream_t s)
{
    hipLaunchKernelGGL((gemm_nt_w4<IN, OUT, BN>), dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

#define GNT_W4_TABLE(BN)                                                                        \
    {                                                                                           \
        {launch_w4<0, 0, BN>, launch_w4<0, 1, BN>, launch_w4<0, 2, BN>},                        \
        {launch_w4<1, 0, BN>, launch_w4<1, 1, BN>, launch_w4<1, 2, BN>},                        \
    }

LaunchTable kW4_128 = GNT_W4_TABLE(128);

}  // namespace gnt
