// Launch table of the 256x256 ping-pong kernel with A MN-major and B MN-major.
#define GNT_PP2_AM 1
#define GNT_PP2_BNM 1
#define GNT_PP2_TABLE kPP2_mm
#include "launch_pp2.hip"
