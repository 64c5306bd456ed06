// Launch tables of the kernel-template tiles (gemm_nt_kernel.hpp), part two.
#define GNT_TILES_PART_B
#include "launch_tiles_a.hip"
