// Launch table of the 256x256 ping-pong kernel with A K-major and B MN-major.
#define GNT_PP2_AM 0
#define GNT_PP2_BNM 1
#define GNT_PP2_TABLE kPP2_km
#include "launch_pp2.hip"
