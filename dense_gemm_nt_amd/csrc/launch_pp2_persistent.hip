// Launch tables of the 256x256 ping-pong kernel with persistent blocks (each
// block loops over work units of its XCD's run) and of its stream-K form
// (each block runs a contiguous range of (tile, k-slab) units and stores FP32
// partial slots; the output type only matters to the reduction that follows,
// so one instantiation per input type serves every output type),
// [in dtype][out dtype].
#include "gemm_nt_launch.hpp"
#include "gemm_nt_pp2.hpp"

namespace gnt {

template <int IN, int OUT, int PS>
static hipError_t launch_pp2_ps(const KernelArgs &a, unsigned grid, hipStream_t s)
{
    hipLaunchKernelGGL((gemm_nt_pp2<IN, OUT, false, false, 0, false, PS>), dim3(grid), dim3(512),
                       0, s, a);
    return hipGetLastError();
}

LaunchTable kPP2_persistent = {
    {launch_pp2_ps<0, 0, 1>, launch_pp2_ps<0, 1, 1>, launch_pp2_ps<0, 2, 1>},
    {launch_pp2_ps<1, 0, 1>, launch_pp2_ps<1, 1, 1>, launch_pp2_ps<1, 2, 1>},
};

LaunchTable kPP2_streamk = {
    {launch_pp2_ps<0, OUT_FP32, 2>, launch_pp2_ps<0, OUT_FP32, 2>, launch_pp2_ps<0, OUT_FP32, 2>},
    {launch_pp2_ps<1, OUT_FP32, 2>, launch_pp2_ps<1, OUT_FP32, 2>, launch_pp2_ps<1, OUT_FP32, 2>},
};

}  // namespace gnt
