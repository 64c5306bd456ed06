// Launch table of the 256x256 ping-pong kernel for grouped launches (one
// problem per group, the problem looked up per block), [in dtype][out dtype].
#include "gemm_nt_launch.hpp"
#include "gemm_nt_pp2.hpp"

namespace gnt {

template <int IN, int OUT>
static hipError_t launch_pp2_grouped(const KernelArgs &a, unsigned grid, hipStream_t s)
{
    hipLaunchKernelGGL((gemm_nt_pp2<IN, OUT, false, false, 0, true>), dim3(grid), dim3(512), 0, s,
                       a);
    return hipGetLastError();
}

LaunchTable kPP2_grouped = {
    {launch_pp2_grouped<0, 0>, launch_pp2_grouped<0, 1>, launch_pp2_grouped<0, 2>},
    {launch_pp2_grouped<1, 0>, launch_pp2_grouped<1, 1>, launch_pp2_grouped<1, 2>},
};

}  // namespace gnt
