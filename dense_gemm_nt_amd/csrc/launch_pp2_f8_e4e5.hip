// Launch table of the 256x256 ping-pong kernel with A in E4M3 and B in E5M2.
#define GNT_F8_IN 3
#define GNT_F8_TABLE kPP2_f8_e4e5
#define GNT_F8_GROUPED_TABLE kPP2_f8_e4e5_grouped
#include "launch_pp2_f8.hip"
