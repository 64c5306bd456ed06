// Launch table of the 256x256 ping-pong kernel with A MN-major and B K-major.
#define GNT_PP2_AM 1
#define GNT_PP2_BNM 0
#define GNT_PP2_TABLE kPP2_mk
#include "launch_pp2.hip"
