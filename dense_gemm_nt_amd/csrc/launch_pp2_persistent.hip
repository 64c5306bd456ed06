// Launch table of the 256x256 ping-pong kernel with persistent blocks (each
// block loops over work units of its XCD's run), [in dtype][out dtype].
#include "gemm_nt_launch.hpp"
#include "gemm_nt_pp2.hpp"

namespace gnt {

template <int IN, int OUT>
static hipError_t launch_pp2_persistent(const KernelArgs &a, unsigned grid, hipStream_t s)
{
    hipLaunchKernelGGL((gemm_nt_pp2<IN, OUT, false, false, 0, false, true>), dim3(grid),
                       dim3(512), 0, s, a);
    return hipGetLastError();
}

LaunchTable kPP2_persistent = {
    {launch_pp2_persistent<0, 0>, launch_pp2_persistent<0, 1>, launch_pp2_persistent<0, 2>},
    {launch_pp2_persistent<1, 0>, launch_pp2_persistent<1, 1>, launch_pp2_persistent<1, 2>},
};

}  // namespace gnt
