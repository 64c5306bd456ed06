// gemm_nt_launch.hpp -- launch tables of the kernel family.  Each table lives in
// a translation unit of its own (launch_*.hip) so the instantiations compile in
// parallel; the host side (gemm_nt.hip) picks one entry per call.
#pragma once

#include <hip/hip_runtime.h>

#include "gemm_nt_common.hpp"

namespace gnt {

typedef hipError_t (*launch_fn)(const KernelArgs &, unsigned grid, hipStream_t);
// [in dtype][out dtype]; not const, so that device compilation, which gives
// const namespace-scope tables a device copy, leaves these host-only
typedef launch_fn LaunchTable[2][3];

// kernel-template tiles (gemm_nt_kernel.hpp), in the order of their names,
// walking K in order and (_rot) in the rotated slab order
extern LaunchTable kTile128x128_w8_s4, kTile128x128_w8_s4_kmask, kTile128x128_w8_s2,
    kTile32x128_w4_s6;
extern LaunchTable kTile128x128_w8_s4_rot, kTile128x128_w8_s4_kmask_rot, kTile128x128_w8_s2_rot,
    kTile32x128_w4_s6_rot;
// the 256x256 ping-pong kernel (gemm_nt_pp2.hpp), by operand layout: K-major A and B (NT), MN-major B, MN-major A,
// both MN-major
extern LaunchTable kPP2_kk, kPP2_km, kPP2_mk, kPP2_mm;
// FP8 inputs on the same kernel, one table per (A format, B format) with E4M3
// = e4 and E5M2 = e5, indexed [scale mode (per tensor, blockwise)][out dtype]
extern LaunchTable kPP2_f8_e4e4, kPP2_f8_e4e5, kPP2_f8_e5e4, kPP2_f8_e5e5;
// and in grouped launches, [scale mode][out dtype]
extern LaunchTable kPP2_f8_e4e4_grouped, kPP2_f8_e4e5_grouped, kPP2_f8_e5e4_grouped,
    kPP2_f8_e5e5_grouped;
// grouped launches (16-bit inputs, K-major operands), [in dtype][out dtype]
extern LaunchTable kPP2_grouped;
// persistent blocks over the tiles of one problem, and its stream-K form
// (16-bit, K-major)
extern LaunchTable kPP2_persistent, kPP2_streamk;
// the four-wave 256x128 tile (gemm_nt_w4.hpp), 16-bit, K-major
extern LaunchTable kW4_128;

}  // namespace gnt
