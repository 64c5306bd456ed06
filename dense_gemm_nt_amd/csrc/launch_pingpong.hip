// Launch table of the first 256x256 ping-pong kernel (gemm_nt_pingpong.hpp).
#include "gemm_nt_launch.hpp"
#include "gemm_nt_pingpong.hpp"

namespace gnt {

template <int IN, int OUT>
static hipError_t launch_pingpong(const KernelArgs &a, unsigned grid, hipStream_t s)
{
    hipLaunchKernelGGL((gemm_nt_pingpong<IN, OUT, 64, 2, 0>), dim3(grid), dim3(512), 0, s, a);
    return hipGetLastError();
}

LaunchTable kPingpong256 = {
    {launch_pingpong<0, 0>, launch_pingpong<0, 1>, launch_pingpong<0, 2>},
    {launch_pingpong<1, 0>, launch_pingpong<1, 1>, launch_pingpong<1, 2>},
};

}  // namespace gnt
