// Launch tables of the kernel-template tiles (gemm_nt_kernel.hpp), part one.
#include "gemm_nt_kernel.hpp"
#include "gemm_nt_launch.hpp"

namespace gnt {

template <int BM, int BN, int BK, int WM, int WN, int ST, int IN, int OUT, bool KMASK, bool ROT>
static hipError_t launch_tile(const KernelArgs &a, unsigned grid, hipStream_t s)
{
    hipLaunchKernelGGL((gemm_nt_kernel<BM, BN, BK, WM, WN, ST, IN, OUT, KMASK, ROT>), dim3(grid),
                       dim3(WM * WN * 64), 0, s, a);
    return hipGetLastError();
}

#define GNT_TILE_TABLE(BM, BN, BK, WM, WN, ST, KM, R)                                            \
    {                                                                                            \
        {launch_tile<BM, BN, BK, WM, WN, ST, 0, 0, KM, R>, launch_tile<BM, BN, BK, WM, WN, ST, 0, 1, KM, R>, \
         launch_tile<BM, BN, BK, WM, WN, ST, 0, 2, KM, R>},                                      \
        {launch_tile<BM, BN, BK, WM, WN, ST, 1, 0, KM, R>, launch_tile<BM, BN, BK, WM, WN, ST, 1, 1, KM, R>, \
         launch_tile<BM, BN, BK, WM, WN, ST, 1, 2, KM, R>},                                      \
    }

#ifndef GNT_TILES_PART_B
LaunchTable kTile128x128_w8_s4 = GNT_TILE_TABLE(128, 128, 64, 2, 4, 4, false, false);
LaunchTable kTile128x128_w8_s4_rot = GNT_TILE_TABLE(128, 128, 64, 2, 4, 4, false, true);
LaunchTable kTile128x128_w8_s4_kmask_rot = GNT_TILE_TABLE(128, 128, 64, 2, 4, 4, true, true);
#else
LaunchTable kTile128x128_w8_s4_kmask = GNT_TILE_TABLE(128, 128, 64, 2, 4, 4, true, false);
LaunchTable kTile128x128_w8_s2 = GNT_TILE_TABLE(128, 128, 64, 2, 4, 2, false, false);
LaunchTable kTile128x128_w8_s2_rot = GNT_TILE_TABLE(128, 128, 64, 2, 4, 2, false, true);
LaunchTable kTile32x128_w4_s6 = GNT_TILE_TABLE(32, 128, 64, 1, 4, 6, false, false);
LaunchTable kTile32x128_w4_s6_rot = GNT_TILE_TABLE(32, 128, 64, 1, 4, 6, false, true);
#endif

}  // namespace gnt
