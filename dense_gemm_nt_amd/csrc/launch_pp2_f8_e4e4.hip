// Launch table of the 256x256 ping-pong kernel with A in E4M3 and B in E4M3.
#define GNT_F8_IN 2
#define GNT_F8_TABLE kPP2_f8_e4e4
#define GNT_F8_GROUPED_TABLE kPP2_f8_e4e4_grouped
#include "launch_pp2_f8.hip"
