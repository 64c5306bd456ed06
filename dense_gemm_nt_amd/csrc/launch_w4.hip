// Launch table of the four-wave 256x256 tile (gemm_nt_w4.hpp).
#include "gemm_nt_launch.hpp"
#include "gemm_nt_w4.hpp"

namespace gnt {

template <int IN, int OUT>
static hipError_t launch_w4(const KernelArgs &a, unsigned grid, hipStream_t s)
{
    hipLaunchKernelGGL((gemm_nt_w4<IN, OUT>), dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

LaunchTable kW4 = {
    {launch_w4<0, 0>, launch_w4<0, 1>, launch_w4<0, 2>},
    {launch_w4<1, 0>, launch_w4<1, 1>, launch_w4<1, 2>},
};

}  // namespace gnt
