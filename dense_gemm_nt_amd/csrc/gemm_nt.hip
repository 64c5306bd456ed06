// gemm_nt.hip -- host side of the NT GEMM library: the C ABI declared in
// include/gemm_nt.h, argument checks, the per-shape plan and the launches.
//
// Planning follows "A Blackwell GEMM by Hand in CuTe DSL", section 1 (M decides
// the regime; the number of tiles against the number of compute units decides
// decode performance) and section 9 (smaller N tiles and split-K for decode;
// libraries ship a family of kernels and pick per shape).  Here the family is a
// handful of tile shapes of one kernel template; a shape picks its tile by M
// and then splits K until the grid covers the 256 compute units.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <new>
#include <vector>

#include "gemm_nt.h"
#include "gemm_nt_launch.hpp"

// Per-tile arrival counters of the in-kernel two-split reduction, at the end of
// every workspace (handle or scratch): zero between calls (each call's second
// arrival resets its tile's counter).
#define GEMM_COUNTER_BYTES ((int64_t)64 << 10)

// Scratch of gemm_run_noalloc: the split-K / stream-K partials of calls that may
// not allocate.  Each device the library runs on holds its own copy from the
// first call on it until the process ends.  In host code the name stands for
// the host-side shadow, never a device address: the device address comes from
// hipGetSymbolAddress (per device, see noalloc_scratch) and only that address is
// passed to kernels.
static __device__ __align__(256) uint8_t scratch[GEMM_NOALLOC_SCRATCH_BYTES + GEMM_COUNTER_BYTES];

namespace {

using gnt::KernelArgs;
using gnt::launch_fn;

constexpr int kNumCUs = 256;
constexpr int64_t kMaxLeadingDim = (int64_t)1 << 22;   // keeps tile byte offsets below 2^31
constexpr int64_t kDefaultWorkspaceMB = 128;

// The 256x256 ping-pong tile for the other operand layouts, indexed by
// 2 * (A MN-major) + (B MN-major) - 1.
typedef launch_fn (*LaunchTableRef)[3];   // a [2][3] launch table
const LaunchTableRef kLayoutFns[3] = {gnt::kPP2_km, gnt::kPP2_mk, gnt::kPP2_mm};

hipError_t launch_splitk_sum(const KernelArgs &a, int out_dtype, hipStream_t s)
{
    const int64_t threads = (int64_t)a.M * ((a.N + 3) / 4);
    const unsigned grid = (unsigned)((threads + 255) / 256);
    if (out_dtype == GEMM_BF16)
        hipLaunchKernelGGL(gnt::splitk_sum<gnt::OUT_BF16>, dim3(grid), dim3(256), 0, s, a);
    else if (out_dtype == GEMM_FP16)
        hipLaunchKernelGGL(gnt::splitk_sum<gnt::OUT_FP16>, dim3(grid), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(gnt::splitk_sum<gnt::OUT_FP32>, dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_streamk_sum(const KernelArgs &a, int G, int out_dtype, hipStream_t s)
{
    const int64_t threads = (int64_t)a.M * ((a.N + 3) / 4);
    const unsigned grid = (unsigned)((threads + 255) / 256);
    if (out_dtype == GEMM_BF16)
        hipLaunchKernelGGL(gnt::streamk_sum<gnt::OUT_BF16>, dim3(grid), dim3(256), 0, s, a, G);
    else if (out_dtype == GEMM_FP16)
        hipLaunchKernelGGL(gnt::streamk_sum<gnt::OUT_FP16>, dim3(grid), dim3(256), 0, s, a, G);
    else
        hipLaunchKernelGGL(gnt::streamk_sum<gnt::OUT_FP32>, dim3(grid), dim3(256), 0, s, a, G);
    return hipGetLastError();
}

struct Config {
    const char *name;
    int bm, bn, bk, waves, stages;
    int lds;        // LDS bytes per workgroup
    int kmask;      // zeroes operand columns past K in registers (any K)
    int splitk;     // supports splits > 1
    launch_fn (*fn)[3];   // [in dtype][out dtype]
    launch_fn (*fn_rot)[3];   // the same tiles in the rotated k-slab order (or null)
};

// The kernel family.  The kernel-template tiles use stages * (BM + BN) * BK * 2
// bytes of LDS (at most 160 KB) and give each wave a (BM/WM) x (BN/WN) block of
// 32x32 MFMA tiles.  Configurations with kmask = 1 zero the operand columns past
// K in registers and are the only ones planned when K is not a multiple of 8.
const Config kConfigs[] = {
    {"128x128x64_w8_s4", 128, 128, 64, 8, 4, 131072, 0, 1, gnt::kTile128x128_w8_s4, gnt::kTile128x128_w8_s4_rot},
    {"128x128x64_w8_s4_kmask", 128, 128, 64, 8, 4, 131072, 1, 1, gnt::kTile128x128_w8_s4_kmask,
     gnt::kTile128x128_w8_s4_kmask_rot},
    {"256x256x64_w8_pp2", 256, 256, 64, 8, 9, 147456, 0, 1, gnt::kPP2_kk, nullptr},
    {"128x128x64_w8_s2", 128, 128, 64, 8, 2, 65536, 0, 1, gnt::kTile128x128_w8_s2, gnt::kTile128x128_w8_s2_rot},
    {"32x128x64_w4_s6", 32, 128, 64, 4, 6, 122880, 0, 1, gnt::kTile32x128_w4_s6, gnt::kTile32x128_w4_s6_rot},
    {"256x128x64_w4_u8", 256, 128, 64, 4, 8, 163840, 0, 1, gnt::kW4_128, nullptr},
};
constexpr int kNumConfigs = sizeof(kConfigs) / sizeof(kConfigs[0]);
enum {
    CFG_T128x128 = 0,
    CFG_T128x128_KMASK = 1,
    CFG_PP2_256x256 = 2,
    CFG_T128x128_S2 = 3,
    CFG_T32x128 = 4,
    CFG_W4_256x128 = 5,
};

struct Plan {
    int cfg;
    int stream;            // stream-K: the persistent ping-pong kernel + streamk_sum
    int sk_maxseg;         // stream-K partial slots per block
    int64_t sk_units;      // stream-K units, tiles * k_tiles
    int tiles_m, tiles_n;
    int k_tiles;
    int splits;
    int kt_per_split;
    int group_m;
    int64_t grid;
    int64_t ws_bytes;
    int inreduce;          // two K splits reduced inside the kernel (no second pass)
};

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Whether the tile kernels (32x128, 128x128) walk their k-slabs in the
// rotated order (SlabOrder; `mode` as GEMM_ROTATE).  Rotation spreads the
// blocks' row offsets over the memory channels, which pays where B streams
// from HBM and A is small (M <= 128: 1 x 4096 x 16384 38.0 -> 28.3 us,
// 127 x 28672 x 8192 102.6 -> 95.4, 1 x 8192 x 8192 30.0 -> 28.2).  With 256
// rows of A that every tile reads, tiles at different slabs no longer share
// A's slabs in L2 as they go (256 x 8192 x 8192 on the four-wave tile: 57.3
// -> 62.3 us), and on the large shapes it measured level or slower, so the
// 256-row tiles always walk K in order.
bool rotate_slabs(int mode, int64_t M) { return mode == 2 || (mode == 1 && M <= 128); }

// The launch function of configuration `cfg`, in the rotated slab order when
// `rot` and the configuration has one.
launch_fn config_fn(int cfg, bool rot, int in_dtype, int out_dtype)
{
    const Config &c = kConfigs[cfg];
    return (rot && c.fn_rot ? c.fn_rot : c.fn)[in_dtype][out_dtype];
}

int find_config(const char *name)
{
    for (int i = 0; i < kNumConfigs; ++i)
        if (strcmp(kConfigs[i].name, name) == 0)
            return i;
    return -1;
}

// Pick the tile shape and the K split for a problem.  `ws_bytes` bounds the
// split-K partial storage; `force_cfg` / `force_splits` (>= 0 / > 0) override.
Plan make_plan(int64_t M, int64_t N, int64_t K, int64_t ws_bytes, int force_cfg, int force_splits,
               int streamk = 0, int inreduce = 1)
{
    Plan p{};
    int cfg;
    // A tile family's blocks with the K splits the split rule below would give
    // it (at least min_slabs 64-deep slabs each), and the fraction of their
    // passes of the machine they fill.
    const int64_t kt64 = cdiv(K, 64);
    auto blocks = [&](int64_t tiles, int64_t min_slabs) {
        int64_t s = 1;
        if (tiles < kNumCUs && kt64 >= 16)
            s = std::max<int64_t>(1, std::min<int64_t>(kNumCUs / tiles, kt64 / min_slabs));
        return tiles * s;
    };
    auto fill = [](int64_t b) { return (double)b / (double)(cdiv(b, kNumCUs) * kNumCUs); };
    if (force_cfg >= 0) {
        cfg = force_cfg;
    } else if (K % 8) {
        cfg = CFG_T128x128_KMASK;
    } else if (M <= 64) {
        // The 32x128 tile, while its tiles fit one pass of the machine: two
        // 32-row tiles per column still beat one 128-row tile at 64 x 4096 x
        // 4096 (15.3 against 20.8 us) and are level with it at 40 x 8192 x 8192
        // (32.3 against 32.5).  Past one pass (M > 32 over N > 16384) the
        // second, mostly empty pass costs more than the 128-row tile's idle
        // rows: 40 x 28672 x 8192 73.9 against 103.2 us, 64 x 28672 x 8192 77.0
        // against 110.9.  From M = 96 the 128x128 tile is faster by half.
        cfg = M <= 32 || cdiv(M, 32) * cdiv(N, 128) <= kNumCUs ? CFG_T32x128 : CFG_T128x128;
    } else if (M <= 128) {
        cfg = CFG_T128x128;
    } else if (M <= 256) {
        // Decode batches: the whole of M in one 256-row tile of the ping-pong
        // kernel (A stays in L2, every compute unit streams its own 256-row
        // panel of B), and split-K below to bring the grid up to the machine.
        // When that tile would need more than four K splits (few N tiles:
        // 256 x 10240 x 8192, 256 x 8192 x 8192, 256 x 8192 x 28672), the
        // four-wave 256 x 128 tile fills the machine with half as many splits,
        // i.e. half the FP32 partial traffic (interleaved medians: 59.5 -> 56.6,
        // 53.0 -> 50.0, 126.2 -> 123.0 us; with two splits, at 256 x 28672 x
        // 8192, the ping-pong tile stays faster: 122.6 against 126.1 us).
        //
        // Either 256-row tile only while its blocks fill the machine as well
        // as the 128x128 tile's would (the fraction of the passes they fill,
        // with the K splits the split rule below gives each): with short K or
        // few N tiles the 256-row tiles' splits (at least 20 slabs each) leave
        // most compute units idle.  Interleaved medians: 192 x 4096 x 4096
        // 22.4 us on the 128x128 tile against 42.8 on the ping-pong tile,
        // 200 x 6144 x 3072 24.3 against 55.1, 256 x 8192 x 2048 21.7 against
        // 41.6, 256 x 2048 x 8192 26.5 against 33.9 on the four-wave tile; and
        // the four-wave tile over the ping-pong one when it fills more
        // (256 x 16384 x 4096: 45.3 against 53.0 us), or as much while the
        // ping-pong tile's splits would hold fewer than 64 slabs each
        // (256 x 28672 x 4096: 62.7 against 67.1 us; at K = 8192, 64 slabs
        // per split, the ping-pong tile: 121.8 against 124.3).
        cfg = CFG_PP2_256x256;
        const int64_t t256 = cdiv(N, 256);
        const int64_t s256 = std::min<int64_t>(kNumCUs / std::max<int64_t>(1, t256), kt64 / 20);
        const int64_t b_w4 = blocks(cdiv(N, 128), 20), b_128 = blocks(cdiv(M, 128) * cdiv(N, 128), 8);
        const int64_t b_pp2 = blocks(t256, 20);
        double f = fill(b_pp2);
        const bool short_splits = kt64 * t256 / b_pp2 < 64;
        if (t256 < kNumCUs && (s256 > 4 || fill(b_w4) > f || (fill(b_w4) == f && short_splits))) {
            cfg = CFG_W4_256x128;
            f = fill(b_w4);
        }
        if (fill(b_128) > f)
            cfg = CFG_T128x128;
    } else {
        // The 256x256 ping-pong tile when its blocks fill at least half the
        // machine, with the K splits the split rule below would give it (at
        // least 20 k-slabs each); smaller tiles otherwise.
        const int64_t big = std::max<int64_t>(1, cdiv(M, 256) * cdiv(N, 256));
        const int64_t ksplit = std::min<int64_t>(kNumCUs / big, cdiv(K, 64) / 20);
        cfg = big * std::max<int64_t>(1, ksplit) >= kNumCUs / 2 ? CFG_PP2_256x256 : CFG_T128x128;
        // ... and the 128x128 tile even then, when its tiles fit one pass and
        // fill it at least as well (640 x 2048 x 8192: 37.9 against 50.6 us;
        // 768 x 4096 x 4096 40.9 against 44.5; 384 x 8192 x 4096 41.9 against
        // 45.6).  Its plans past one pass (the two-stage ring) measured mixed
        // against the ping-pong tile and keep the rule above.
        const int64_t t128 = cdiv(M, 128) * cdiv(N, 128);
        if (cfg == CFG_PP2_256x256 && t128 < kNumCUs && fill(blocks(t128, 8)) >= fill(blocks(big, 20)))
            cfg = CFG_T128x128;
    }
    // The 32x128 tile wherever the 128x128 tile was chosen above M = 64 but
    // the 32-row tiles, in one pass with their own K splits, fill the machine
    // strictly better: small squares and small problems with short K.  On
    // the small ragged shapes it takes, the two tiles, each with its own K
    // splits, measured level (178 x 640 x 2240: 11.0 us both; 74 x 1408 x
    // 512 8.8; 618 x 704 x 3968 16.4 against 16.3), where the plans that
    // earlier rules made for them took 16.6, 11.2 and 19.8 us.  On a tie
    // the 128x128 tile, whose blocks do more work per byte staged.
    if (cfg == CFG_T128x128 && M > 64) {
        const int64_t t32 = cdiv(M, 32) * cdiv(N, 128), t128 = cdiv(M, 128) * cdiv(N, 128);
        if (t32 <= kNumCUs && fill(blocks(t32, 8)) > fill(blocks(t128, 8)))
            cfg = CFG_T32x128;
    }
    // 128x128 tiles that overflow one pass of the machine but fit two: the
    // two-stage ring (64 KB of LDS) lets two blocks share a compute unit, so
    // they all run at once instead of leaving a second, nearly empty wave.
    if (cfg == CFG_T128x128 && force_cfg < 0) {
        const int64_t t128 = cdiv(M, 128) * cdiv(N, 128);
        if (t128 > kNumCUs && t128 <= 2 * kNumCUs)
            cfg = CFG_T128x128_S2;
    }
    if ((K % 8) && !kConfigs[cfg].kmask)
        cfg = CFG_T128x128_KMASK;
    const Config &c = kConfigs[cfg];
    p.cfg = cfg;
    p.tiles_m = (int)cdiv(M, c.bm);
    p.tiles_n = (int)cdiv(N, c.bn);
    p.k_tiles = (int)cdiv(K, c.bk);
    const int64_t tiles = (int64_t)p.tiles_m * p.tiles_n;

    int splits = 1;
    if (!c.splitk) {
        splits = 1;
    } else if (force_splits > 0) {
        splits = force_splits;
    } else if (tiles < kNumCUs && (int64_t)p.k_tiles * c.bk >= 16 * 64) {
        // Fill the compute units, keeping at least 512 of K per split (1280
        // for the 256x256 tiles, whose 256 KB FP32 partial per split costs as
        // much as streaming about 256 of K of B).
        // For M <= 32 the 32-row tile's blocks each stream their own rows of
        // B, once: with a block on every compute unit those streams measured
        // up to 60% slower than with about three quarters of them (more
        // concurrent DRAM streams, not more bytes), so the split count aims
        // there, rounded to the nearest.
        const int min_slabs = (c.bm == 256 ? 20 : 8) * 64 / c.bk;
        if (cfg == CFG_T32x128 && M <= 32)
            splits = (int)((3 * kNumCUs / 4 + tiles / 2) / tiles);
        else
            splits = (int)(kNumCUs / tiles);
        if (splits > p.k_tiles / min_slabs)
            splits = p.k_tiles / min_slabs;
        if (splits < 1)
            splits = 1;
    }
    // For M <= 32 the 32-row tile streams B rows whose K splits start
    // kt_per_split * 128 bytes apart.  Starts a multiple of 4 KB apart measured
    // up to 20% slower (the blocks of one B row then hit the same DRAM channels
    // together), so the nearest split count with another stride is taken.
    // Only when the fill rule split K: with one split no two blocks start in
    // the same B row.
    if (cfg == CFG_T32x128 && M <= 32 && force_splits <= 0 && p.k_tiles >= 16 && splits > 1) {
        auto aliased = [&](int sp) { return (cdiv(p.k_tiles, sp) * c.bk * 2) % 4096 == 0; };
        auto ok = [&](int sp) { return sp >= 1 && sp <= 8 && p.k_tiles / sp >= 8 && !aliased(sp); };
        if (aliased(splits)) {
            for (int d = 1; d < 8; ++d) {
                if (ok(splits - d)) {
                    splits -= d;
                    break;
                }
                if (ok(splits + d)) {
                    splits += d;
                    break;
                }
            }
        }
    }
    while (splits > 1 && (int64_t)splits * M * N * 4 > ws_bytes)
        --splits;
    if (p.k_tiles == 0)
        splits = 1;
    if (splits > p.k_tiles && p.k_tiles > 0)
        splits = p.k_tiles;
    p.kt_per_split = splits > 1 ? (int)cdiv(p.k_tiles, splits) : p.k_tiles;
    if (splits > 1)
        splits = (int)cdiv(p.k_tiles, p.kt_per_split);   // no empty split
    p.splits = splits;
    p.group_m = p.tiles_m >= 4 ? 4 : p.tiles_m;
    if (p.group_m < 1)
        p.group_m = 1;
    p.grid = tiles * splits;
    p.ws_bytes = splits > 1 ? (int64_t)splits * M * N * 4 : 0;
    // Two K splits on the 256-row tiles, any number on the tile kernels with a
    // ring deeper than two stages: the last split of a tile to finish adds the
    // others' partials (one BM x BN FP32 slot per split and tile) and stores
    // the tile, instead of a second pass over [splits][M][N] partials.
    const bool many = cfg != CFG_PP2_256x256 && cfg != CFG_W4_256x128 && c.stages > 2;
    const bool two = cfg == CFG_PP2_256x256 || cfg == CFG_W4_256x128;
    if (inreduce && ((splits == 2 && two) || (splits >= 2 && many)) &&
        tiles * 4 <= GEMM_COUNTER_BYTES) {
        const int64_t need = tiles * splits * (int64_t)c.bm * c.bn * 4;
        if (need <= ws_bytes) {
            p.inreduce = 1;
            p.ws_bytes = need;
        }
    }

    // Stream-K (the CuTe page's section 9 names it beside split-K): when the
    // ping-pong tiles with their K splits leave at least 3/8 of the compute
    // units idle, every unit takes an equal run of the tiles * k_tiles
    // (tile, k-slab) units instead, each tile it touches giving one partial
    // (a 256 KB slot).  Only for runs of at least 32 k-slabs: each segment
    // refills the pipeline and writes a whole partial tile, which shorter runs
    // do not pay back.  `streamk`: 0 never, 1 by this rule (the default), 2
    // whenever the tile is the ping-pong one.  Interleaved medians on operands
    // read cold: 3000 x 3000 x 5000 (144 tiles) 126 us against 141 without;
    // 2304 x 2304 x 8192 (three splits fill the machine) 130 against 88;
    // 3000 x 3000 x 1536 (runs of 13 slabs) 70 against 50.  With operands
    // resident in the memory-side cache the first one reverses (125 against
    // 118): stream-K pays where the idle compute units would add HBM streams.
    if (streamk > 0 && cfg == CFG_PP2_256x256 && force_splits <= 0 && tiles > 0 && p.k_tiles > 0) {
        const int64_t T = tiles * p.k_tiles;
        const int64_t G = std::min<int64_t>(kNumCUs, T);
        const int64_t L = (T + G - 1) / G;                 // longest run
        const int maxseg = (int)((L - 1) / p.k_tiles + 2);
        const int64_t ws = G * maxseg * (int64_t)256 * 256 * 4;
        const bool idle = p.grid * 8 <= (int64_t)kNumCUs * 5;
        if (ws <= ws_bytes && T < INT32_MAX && (streamk == 2 || (idle && L >= 32))) {
            p.stream = 1;
            p.sk_units = T;
            p.sk_maxseg = maxseg;
            p.splits = 1;
            p.kt_per_split = p.k_tiles;
            p.grid = G;
            p.ws_bytes = ws;
        }
    }
    return p;
}

}  // namespace

// Plans of a handle's recent shapes: the planner's result depends only on the
// problem and on the handle's fixed settings, so a repeated shape skips it.
struct PlanCacheEntry {
    int64_t M, N, K;
    int cfg, streamk, inreduce;   // make_plan's per-call arguments
    int valid;
    Plan plan;
};
constexpr int kPlanCacheSize = 16;

struct gemm_handle_s {
    int device;
    float *partials;
    int64_t ws_bytes;
    int force_cfg;
    int force_splits;
    int persistent;    // GEMM_PERSIST=1: ping-pong tiles run by 256 persistent blocks
    int inreduce;      // GEMM_INREDUCE: 1 (default) two K splits reduced in the kernel, 0 never
    int streamk;       // GEMM_STREAMK: 0 off, 1 by the plan rule (default), 2 whenever
                       // the ping-pong tile is planned
    int rotate;        // GEMM_ROTATE: the tile kernels' rotated k-slab order (SlabOrder): 0 never,
                       // 1 by the rule of rotate_slabs (default), 2 always
    int log;
    // grouped launches: pinned staging of the problem list and an event that
    // marks when the last copy out of it has run
    uint8_t *staging;
    int64_t staging_bytes;
    hipEvent_t staged;
    int staged_pending;
    PlanCacheEntry plans[kPlanCacheSize];
    int plan_next;
};

namespace {

// make_plan with the handle's workspace and split settings, through its cache
// (the handle is used by one caller at a time, so the cache takes no lock).
Plan handle_plan(gemm_handle_s *h, int64_t M, int64_t N, int64_t K, int cfg, int streamk,
                 int inreduce)
{
    for (const PlanCacheEntry &e : h->plans)
        if (e.valid && e.M == M && e.N == N && e.K == K && e.cfg == cfg && e.streamk == streamk &&
            e.inreduce == inreduce)
            return e.plan;
    PlanCacheEntry &e = h->plans[h->plan_next];
    h->plan_next = (h->plan_next + 1) % kPlanCacheSize;
    e = PlanCacheEntry{M, N, K, cfg, streamk, inreduce, 1,
                       make_plan(M, N, K, h->ws_bytes, cfg, h->force_splits, streamk, inreduce)};
    return e.plan;
}

}  // namespace

extern "C" {

const char *gemm_status_string(int s)
{
    switch (s) {
    case GEMM_OK: return "GEMM_OK";
    case GEMM_ERR_INVALID_ARG: return "GEMM_ERR_INVALID_ARG";
    case GEMM_ERR_UNSUPPORTED: return "GEMM_ERR_UNSUPPORTED";
    case GEMM_ERR_MISALIGNED: return "GEMM_ERR_MISALIGNED";
    case GEMM_ERR_ALLOC: return "GEMM_ERR_ALLOC";
    case GEMM_ERR_HIP: return "GEMM_ERR_HIP";
    default: return "GEMM_ERR_UNKNOWN";
    }
}

// The argument checks of every run; a_row / b_row are the extents a row of A /
// B holds (K for a K-major operand, M or N for an MN-major one).
static gemm_status_t validate(const void *A, const void *B, void *C, int64_t M, int64_t N,
                              int64_t K, int64_t lda, int64_t ldb, int64_t ldc, int64_t a_row,
                              int64_t b_row, int in_dtype, int out_dtype)
{
    if (in_dtype != GEMM_BF16 && in_dtype != GEMM_FP16)
        return GEMM_ERR_UNSUPPORTED;
    if (out_dtype != GEMM_BF16 && out_dtype != GEMM_FP16 && out_dtype != GEMM_FP32)
        return GEMM_ERR_UNSUPPORTED;
    if (M < 0 || N < 0 || K < 0)
        return GEMM_ERR_INVALID_ARG;
    if (lda < a_row || ldb < b_row || ldc < N || lda < 0 || ldb < 0)
        return GEMM_ERR_INVALID_ARG;
    if (M >= INT32_MAX || N >= INT32_MAX || K >= INT32_MAX || ldc >= INT32_MAX)
        return GEMM_ERR_UNSUPPORTED;
    if (lda >= kMaxLeadingDim || ldb >= kMaxLeadingDim)
        return GEMM_ERR_UNSUPPORTED;
    if (M == 0 || N == 0)
        return GEMM_OK;
    if (!C)
        return GEMM_ERR_INVALID_ARG;
    const uintptr_t out_size = out_dtype == GEMM_FP32 ? 4 : 2;
    if ((uintptr_t)C % out_size)
        return GEMM_ERR_MISALIGNED;
    if (K == 0)
        return GEMM_OK;
    if (!A || !B)
        return GEMM_ERR_INVALID_ARG;
    if ((uintptr_t)A % 16 || (uintptr_t)B % 16 || lda % 8 || ldb % 8)
        return GEMM_ERR_MISALIGNED;
    return GEMM_OK;
}

gemm_status_t gemm_validate(const void *A, const void *B, void *C, int64_t M, int64_t N, int64_t K,
                            int64_t lda, int64_t ldb, int64_t ldc, int in_dtype, int out_dtype)
{
    return validate(A, B, C, M, N, K, lda, ldb, ldc, K, K, in_dtype, out_dtype);
}

gemm_status_t gemm_plan(int64_t M, int64_t N, int64_t K, int in_dtype, int out_dtype, gemm_plan_t *out)
{
    if (!out)
        return GEMM_ERR_INVALID_ARG;
    memset(out, 0, sizeof(*out));
    if (in_dtype != GEMM_BF16 && in_dtype != GEMM_FP16)
        return GEMM_ERR_UNSUPPORTED;
    if (out_dtype != GEMM_BF16 && out_dtype != GEMM_FP16 && out_dtype != GEMM_FP32)
        return GEMM_ERR_UNSUPPORTED;
    if (M < 0 || N < 0 || K < 0)
        return GEMM_ERR_INVALID_ARG;
    if (M >= INT32_MAX || N >= INT32_MAX || K >= INT32_MAX)
        return GEMM_ERR_UNSUPPORTED;
    const Plan p = make_plan(M, N, K, kDefaultWorkspaceMB << 20, -1, -1, 1);
    const Config &c = kConfigs[p.cfg];
    out->block_m = c.bm;
    out->block_n = c.bn;
    out->block_k = c.bk;
    out->waves = c.waves;
    out->stages = c.stages;
    out->lds_bytes = c.lds;
    out->splits = p.splits;
    out->tiles = (int64_t)p.tiles_m * p.tiles_n;
    out->workgroups = (M == 0 || N == 0) ? 0 : p.grid;
    out->workspace_bytes = p.ws_bytes;
    out->streamk = p.stream;
    out->inreduce = p.inreduce;
    snprintf(out->name, sizeof(out->name), "%s", c.name);
    return GEMM_OK;
}

gemm_status_t gemm_create(gemm_handle_t *out)
{
    if (!out)
        return GEMM_ERR_INVALID_ARG;
    *out = nullptr;
    gemm_handle_s *h = new (std::nothrow) gemm_handle_s{};
    if (!h)
        return GEMM_ERR_ALLOC;
    h->force_cfg = -1;
    h->force_splits = -1;
    h->persistent = 0;
    int64_t mb = kDefaultWorkspaceMB;
    if (const char *e = getenv("GEMM_WORKSPACE_MB"))
        mb = atoll(e) > 0 ? atoll(e) : mb;
    if (const char *e = getenv("GEMM_CONFIG")) {
        h->force_cfg = find_config(e);
        if (h->force_cfg < 0) {   // a named kernel that does not exist is an error, not a fallback
            delete h;
            return GEMM_ERR_INVALID_ARG;
        }
    }
    if (const char *e = getenv("GEMM_SPLITS"))
        h->force_splits = atoi(e);
    if (const char *e = getenv("GEMM_PERSIST"))
        h->persistent = atoi(e) != 0;
    h->streamk = 1;
    if (const char *e = getenv("GEMM_STREAMK"))
        h->streamk = atoi(e);
    if (const char *e = getenv("GEMM_LOG"))
        h->log = atoi(e);
    h->rotate = 1;
    if (const char *e = getenv("GEMM_ROTATE"))
        h->rotate = atoi(e);
    h->ws_bytes = mb << 20;
    h->inreduce = 1;
    if (const char *e = getenv("GEMM_INREDUCE"))
        h->inreduce = atoi(e) != 0;
    if (hipGetDevice(&h->device) != hipSuccess) {
        delete h;
        return GEMM_ERR_HIP;
    }
    if (const char *e = getenv("GEMM_TEST_FAIL_ALLOC")) {
        if (atoi(e)) {
            delete h;
            return GEMM_ERR_ALLOC;
        }
    }
    if (hipMalloc(&h->partials, (size_t)(h->ws_bytes + GEMM_COUNTER_BYTES)) != hipSuccess) {
        (void)hipGetLastError();
        delete h;
        return GEMM_ERR_ALLOC;
    }
    // the arrival counters start at zero (every call leaves them at zero)
    if (hipMemset(reinterpret_cast<uint8_t *>(h->partials) + h->ws_bytes, 0, (size_t)GEMM_COUNTER_BYTES) !=
            hipSuccess ||
        hipDeviceSynchronize() != hipSuccess) {
        (void)hipGetLastError();
        (void)hipFree(h->partials);
        delete h;
        return GEMM_ERR_HIP;
    }
    *out = h;
    return GEMM_OK;
}

gemm_status_t gemm_destroy(gemm_handle_t h)
{
    if (!h)
        return GEMM_OK;
    gemm_status_t st = GEMM_OK;
    if (hipFree(h->partials) != hipSuccess)
        st = GEMM_ERR_HIP;
    if (h->staging && hipHostFree(h->staging) != hipSuccess)
        st = GEMM_ERR_HIP;
    if (h->staged && hipEventDestroy(h->staged) != hipSuccess)
        st = GEMM_ERR_HIP;
    delete h;
    return st;
}

gemm_status_t gemm_run(gemm_handle_t h, const void *A, const void *B, void *C, int64_t M, int64_t N,
                       int64_t K, int64_t lda, int64_t ldb, int64_t ldc, int in_dtype, int out_dtype,
                       hipStream_t stream)
{
    return gemm_run_ex(h, A, B, C, M, N, K, lda, ldb, ldc, in_dtype, out_dtype, nullptr, stream);
}

gemm_status_t gemm_run_ex(gemm_handle_t h, const void *A, const void *B, void *C, int64_t M,
                          int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc, int in_dtype,
                          int out_dtype, const gemm_epilogue_t *epi, hipStream_t stream)
{
    return gemm_run_layout(h, GEMM_K_MAJOR, GEMM_K_MAJOR, A, B, C, M, N, K, lda, ldb, ldc, in_dtype,
                           out_dtype, epi, stream);
}

}  // extern "C"

namespace {

// `own_bias`: the bias pointer comes with the descriptor (false for grouped
// launches, whose biases come with each problem).
gemm_status_t check_epilogue(const gemm_epilogue_t *epi, bool own_bias = true)
{
    if (!epi)
        return GEMM_OK;
    if (epi->bias_along < GEMM_BIAS_NONE || epi->bias_along > GEMM_BIAS_M)
        return GEMM_ERR_INVALID_ARG;
    if (epi->activation < GEMM_ACT_NONE || epi->activation > GEMM_ACT_GELU)
        return GEMM_ERR_INVALID_ARG;
    if (own_bias && epi->bias_along != GEMM_BIAS_NONE && (!epi->bias || (uintptr_t)epi->bias % 4))
        return GEMM_ERR_INVALID_ARG;
    if (!std::isfinite(epi->alpha) || !std::isfinite(epi->beta))
        return GEMM_ERR_UNSUPPORTED;
    return GEMM_OK;
}

gemm_status_t check_device(gemm_handle_t h)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess)
        return GEMM_ERR_HIP;
    return dev == h->device ? GEMM_OK : GEMM_ERR_INVALID_ARG;
}

// Device memory for split-K and stream-K partials: the handle's workspace, or
// the static scratch of gemm_run_noalloc.
struct Workspace {
    float *partials;
    int64_t bytes;         // for partials and grouped problem lists
    unsigned *counters;    // GEMM_COUNTER_BYTES of arrival counters
    int log;
};

Workspace workspace_of(gemm_handle_t h)
{
    return Workspace{h->partials, h->ws_bytes,
                     reinterpret_cast<unsigned *>(reinterpret_cast<uint8_t *>(h->partials) + h->ws_bytes), h->log};
}

// Fill the plan-, output- and epilogue-dependent fields of `a` (whose operand
// fields the caller has set), then enqueue the kernel and, with split-K, the
// ordered sum of the partials.
gemm_status_t enqueue(const Workspace &ws, const Plan &p, KernelArgs &a, launch_fn fn, void *C,
                      int64_t M, int64_t N, int64_t K, int64_t ldc, int out_dtype,
                      const gemm_epilogue_t *epi, hipStream_t stream)
{
    if ((p.splits > 1 || p.stream) && p.ws_bytes > ws.bytes)
        return GEMM_ERR_UNSUPPORTED;
    if (p.grid <= 0 || p.grid >= INT32_MAX)
        return GEMM_ERR_UNSUPPORTED;
    a.C = C;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.ldc = (int)ldc;
    a.tiles_m = p.tiles_m;
    a.tiles_n = p.tiles_n;
    a.k_tiles = p.k_tiles;
    a.splits = p.splits;
    a.kt_per_split = p.kt_per_split;
    a.group_m = p.group_m;
    const uintptr_t vec_bytes = out_dtype == GEMM_FP32 ? 16 : 8;
    a.vec_store = (ldc % 4 == 0) && ((uintptr_t)C % vec_bytes == 0);
    const int64_t out_size = out_dtype == GEMM_FP32 ? 4 : 2;
    a.rows16 = ((ldc * out_size) % 16 == 0) && ((uintptr_t)C % 16 == 0);
    // B, when at most two tile rows of blocks read it, is streamed
    a.nt_b = p.tiles_m <= 2;
    a.partials = ws.partials;
    a.sk_units = p.stream ? (int)p.sk_units : 0;
    a.sk_maxseg = p.sk_maxseg;
    a.inreduce = p.inreduce;
    a.counters = ws.counters;
    a.alpha = 1.0f;
    if (epi) {
        a.alpha = epi->alpha;
        a.beta = epi->beta;
        a.bias = epi->bias_along != GEMM_BIAS_NONE ? epi->bias : nullptr;
        a.bias_along = epi->bias_along;
        a.act = epi->activation;
        a.bias_vec = ((uintptr_t)a.bias % 16) == 0;
        a.epi = !(a.alpha == 1.0f && a.beta == 0.0f && a.bias_along == GEMM_BIAS_NONE &&
                  a.act == GEMM_ACT_NONE);
    }
    if (ws.log)
        fprintf(stderr, "gemm_nt: M=%lld N=%lld K=%lld cfg=%s tiles=%dx%d splits=%d kt/split=%d grid=%lld%s\n",
                (long long)M, (long long)N, (long long)K, kConfigs[p.cfg].name, p.tiles_m,
                p.tiles_n, p.splits, p.kt_per_split, (long long)p.grid,
                p.stream ? " stream-K" : p.inreduce ? " reduced in-kernel" : "");
    hipError_t e = fn(a, (unsigned)p.grid, stream);
    if (e == hipSuccess && p.splits > 1 && !p.inreduce)
        e = launch_splitk_sum(a, out_dtype, stream);
    if (e == hipSuccess && p.stream)
        e = launch_streamk_sum(a, (int)p.grid, out_dtype, stream);
    return e == hipSuccess ? GEMM_OK : GEMM_ERR_HIP;
}

}  // namespace

extern "C" {

gemm_status_t gemm_run_layout(gemm_handle_t h, int layout_a, int layout_b, const void *A,
                              const void *B, void *C, int64_t M, int64_t N, int64_t K,
                              int64_t lda, int64_t ldb, int64_t ldc, int in_dtype, int out_dtype,
                              const gemm_epilogue_t *epi, hipStream_t stream)
{
    if (!h)
        return GEMM_ERR_INVALID_ARG;
    if ((layout_a != GEMM_K_MAJOR && layout_a != GEMM_MN_MAJOR) ||
        (layout_b != GEMM_K_MAJOR && layout_b != GEMM_MN_MAJOR))
        return GEMM_ERR_INVALID_ARG;
    const bool am = layout_a == GEMM_MN_MAJOR, bnm = layout_b == GEMM_MN_MAJOR;
    gemm_status_t st = validate(A, B, C, M, N, K, lda, ldb, ldc, am ? M : K, bnm ? N : K,
                                in_dtype, out_dtype);
    if (st != GEMM_OK)
        return st;
    if ((am || bnm) && K % 8 && M && N)
        return GEMM_ERR_UNSUPPORTED;
    if ((st = check_epilogue(epi)) != GEMM_OK)
        return st;
    if (M == 0 || N == 0)
        return GEMM_OK;
    if ((st = check_device(h)) != GEMM_OK)
        return st;

    const bool nt = !am && !bnm;
    if (!nt && h->force_cfg >= 0 && h->force_cfg != CFG_PP2_256x256)
        return GEMM_ERR_UNSUPPORTED;
    const Plan p = handle_plan(h, M, N, K, nt ? h->force_cfg : CFG_PP2_256x256,
                               nt ? h->streamk : 0, h->inreduce && !h->persistent);
    KernelArgs a{};
    a.A = static_cast<const uint16_t *>(A);
    a.B = static_cast<const uint16_t *>(B);
    a.lda = (int)lda;
    a.ldb = (int)ldb;
    launch_fn fn = nt ? config_fn(p.cfg, rotate_slabs(h->rotate, M), in_dtype, out_dtype)
                      : kLayoutFns[2 * am + bnm - 1][in_dtype][out_dtype];
    Plan q = p;
    if (p.stream) {
        fn = gnt::kPP2_streamk[in_dtype][out_dtype];
    } else if (nt && h->persistent && p.cfg == CFG_PP2_256x256 && p.grid > kNumCUs) {
        fn = gnt::kPP2_persistent[in_dtype][out_dtype];
        q.grid = kNumCUs;
    }
    return enqueue(workspace_of(h), q, a, fn, C, M, N, K, ldc, out_dtype, epi, stream);
}

}  // extern "C"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];

// The device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.  Concurrent first calls look it up
// twice and store the same address.
gemm_status_t noalloc_scratch(void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess)
        return GEMM_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices)
        return GEMM_ERR_UNSUPPORTED;
    void *ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!ptr) {
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return GEMM_ERR_HIP;
        }
        g_scratch_ptr[dev].store(ptr, std::memory_order_release);
    }
    *out = ptr;
    return GEMM_OK;
}

}  // namespace

extern "C" {

gemm_status_t gemm_run_noalloc(const void *A, const void *B, void *C, int64_t M, int64_t N,
                               int64_t K, int64_t lda, int64_t ldb, int64_t ldc, int in_dtype,
                               int out_dtype, hipStream_t stream)
{
    gemm_status_t st = validate(A, B, C, M, N, K, lda, ldb, ldc, K, K, in_dtype, out_dtype);
    if (st != GEMM_OK)
        return st;
    if (M == 0 || N == 0)
        return GEMM_OK;
    void *ptr = nullptr;
    if ((st = noalloc_scratch(&ptr)) != GEMM_OK)
        return st;
    // gemm_run's plan with its partials bounded by the scratch: a stream-K plan
    // that would need more takes the split plan (K split partials never need
    // more than 64 MiB: at most 256 tiles x splits of 256 x 256 FP32 values)
    const Plan p = make_plan(M, N, K, GEMM_NOALLOC_SCRATCH_BYTES, -1, -1, 1);
    if ((p.splits > 1 || p.stream) && p.ws_bytes > GEMM_NOALLOC_SCRATCH_BYTES)
        return GEMM_ERR_UNSUPPORTED;
    KernelArgs a{};
    a.A = static_cast<const uint16_t *>(A);
    a.B = static_cast<const uint16_t *>(B);
    a.lda = (int)lda;
    a.ldb = (int)ldb;
    launch_fn fn = p.stream ? gnt::kPP2_streamk[in_dtype][out_dtype]
                            : config_fn(p.cfg, rotate_slabs(1, M), in_dtype, out_dtype);
    const Workspace ws{static_cast<float *>(ptr), GEMM_NOALLOC_SCRATCH_BYTES,
                       reinterpret_cast<unsigned *>(static_cast<uint8_t *>(ptr) + GEMM_NOALLOC_SCRATCH_BYTES), 0};
    return enqueue(ws, p, a, fn, C, M, N, K, ldc, out_dtype, nullptr, stream);
}

}  // extern "C"

namespace {

// Copy a grouped launch's problem list and tile table into the workspace
// (through the pinned staging buffer) and launch `fn` over `tiles` blocks.
gemm_status_t stage_and_launch(gemm_handle_t h, const std::vector<gnt::GroupDesc> &descs,
                               int64_t tiles, KernelArgs &a, launch_fn fn, hipStream_t stream)
{
    const int num_groups = (int)descs.size();
    const int64_t desc_bytes = (int64_t)num_groups * (int64_t)sizeof(gnt::GroupDesc);
    const int64_t bytes = desc_bytes + tiles * 4;
    if (bytes > h->ws_bytes)
        return GEMM_ERR_UNSUPPORTED;
    gemm_status_t st = check_device(h);
    if (st != GEMM_OK)
        return st;
    // Stage in pinned memory (so the copy is a true stream-ordered DMA and the
    // call does not wait for the stream), after the previous copy out of the
    // staging buffer has run.
    if (h->staged_pending) {
        if (hipEventSynchronize(h->staged) != hipSuccess)
            return GEMM_ERR_HIP;
        h->staged_pending = 0;
    }
    if (!h->staged && hipEventCreateWithFlags(&h->staged, hipEventDisableTiming) != hipSuccess) {
        h->staged = nullptr;
        return GEMM_ERR_HIP;
    }
    if (bytes > h->staging_bytes) {
        if (h->staging && hipHostFree(h->staging) != hipSuccess)
            return GEMM_ERR_HIP;
        h->staging = nullptr;
        h->staging_bytes = 0;
        const int64_t want = bytes < (1 << 16) ? (1 << 16) : bytes;
        if (hipHostMalloc((void **)&h->staging, (size_t)want, hipHostMallocDefault) != hipSuccess) {
            h->staging = nullptr;
            return GEMM_ERR_ALLOC;
        }
        h->staging_bytes = want;
    }
    memcpy(h->staging, descs.data(), (size_t)desc_bytes);
    int *table = reinterpret_cast<int *>(h->staging + desc_bytes);
    for (int g = 0; g < num_groups; ++g) {
        const int64_t n = (int64_t)descs[g].tiles_m * descs[g].tiles_n;
        for (int64_t t = 0; t < n; ++t)
            table[descs[g].tile_start + t] = g;
    }
    uint8_t *dev = reinterpret_cast<uint8_t *>(h->partials);
    if (hipMemcpyAsync(dev, h->staging, (size_t)bytes, hipMemcpyHostToDevice, stream) != hipSuccess)
        return GEMM_ERR_HIP;
    if (hipEventRecord(h->staged, stream) != hipSuccess)
        return GEMM_ERR_HIP;
    h->staged_pending = 1;

    a.groups = reinterpret_cast<const gnt::GroupDesc *>(dev);
    a.tile_group = reinterpret_cast<const int *>(dev + desc_bytes);
    a.group_m = 4;
    a.splits = 1;
    hipError_t e = fn(a, (unsigned)tiles, stream);
    return e == hipSuccess ? GEMM_OK : GEMM_ERR_HIP;
}

void fill_group_epilogue(KernelArgs &a, const gemm_epilogue_t *epi)
{
    a.alpha = 1.0f;
    if (epi) {
        a.alpha = epi->alpha;
        a.beta = epi->beta;
        a.bias_along = epi->bias_along;
        a.act = epi->activation;
        a.epi = !(a.alpha == 1.0f && a.beta == 0.0f && a.bias_along == GEMM_BIAS_NONE &&
                  a.act == GEMM_ACT_NONE);
    }
}

gemm_status_t run_grouped(gemm_handle_t h, const gemm_group_problem_t *problems, int num_groups,
                          int in_dtype, int out_dtype, const gemm_epilogue_t *epi,
                          hipStream_t stream)
{
    if (!h || num_groups < 0 || (num_groups > 0 && !problems))
        return GEMM_ERR_INVALID_ARG;
    gemm_status_t st = check_epilogue(epi, false);
    if (st != GEMM_OK)
        return st;
    if (epi && epi->bias)
        return GEMM_ERR_INVALID_ARG;   // the bias of group g is problems[g].bias
    const bool with_bias = epi && epi->bias_along != GEMM_BIAS_NONE;
    std::vector<gnt::GroupDesc> descs;
    descs.reserve(num_groups);
    int64_t tiles = 0;
    for (int g = 0; g < num_groups; ++g) {
        const gemm_group_problem_t &q = problems[g];
        st = validate(q.A, q.B, q.C, q.M, q.N, q.K, q.lda, q.ldb, q.ldc, q.K, q.K, in_dtype,
                      out_dtype);
        if (st != GEMM_OK)
            return st;
        if (q.K % 8)
            return GEMM_ERR_UNSUPPORTED;
        if (with_bias && q.M && q.N && (!q.bias || (uintptr_t)q.bias % 4))
            return GEMM_ERR_INVALID_ARG;
        gnt::GroupDesc d{};
        d.A = static_cast<const uint16_t *>(q.A);
        d.B = static_cast<const uint16_t *>(q.B);
        d.C = q.C;
        d.bias = with_bias ? q.bias : nullptr;
        d.M = (int)q.M, d.N = (int)q.N, d.K = (int)q.K;
        d.lda = (int)q.lda, d.ldb = (int)q.ldb, d.ldc = (int)q.ldc;
        d.tiles_m = (int)cdiv(q.M, 256);
        d.tiles_n = (int)cdiv(q.N, 256);
        d.k_tiles = (int)cdiv(q.K, 64);
        d.tile_start = (int)tiles;
        const int64_t out_size = out_dtype == GEMM_FP32 ? 4 : 2;
        const uintptr_t vec_bytes = out_dtype == GEMM_FP32 ? 16 : 8;
        d.flags = ((q.ldc % 4 == 0) && ((uintptr_t)q.C % vec_bytes == 0) ? gnt::GD_VEC_STORE : 0) |
                  (((q.ldc * out_size) % 16 == 0) && ((uintptr_t)q.C % 16 == 0) ? gnt::GD_ROWS16 : 0) |
                  (d.bias && (uintptr_t)d.bias % 16 == 0 ? gnt::GD_BIAS_VEC : 0) |
                  (d.tiles_m <= 2 ? gnt::GD_NT_B : 0);
        descs.push_back(d);
        tiles += (int64_t)d.tiles_m * d.tiles_n;
        if (tiles >= INT32_MAX)
            return GEMM_ERR_UNSUPPORTED;
    }
    if (tiles == 0)
        return GEMM_OK;
    KernelArgs a{};
    fill_group_epilogue(a, epi);
    if (h->log)
        fprintf(stderr, "gemm_nt: grouped, %d groups, %lld tiles\n", num_groups, (long long)tiles);
    return stage_and_launch(h, descs, tiles, a, gnt::kPP2_grouped[in_dtype][out_dtype], stream);
}

gemm_status_t run_grouped_fp8(gemm_handle_t h, int a_dtype, int b_dtype,
                              const gemm_group_problem_fp8_t *problems, int num_groups,
                              int out_dtype, int scale_mode, int block_m,
                              const gemm_epilogue_t *epi, hipStream_t stream)
{
    if (!h || num_groups < 0 || (num_groups > 0 && !problems))
        return GEMM_ERR_INVALID_ARG;
    const bool fa8 = a_dtype == GEMM_FP8_E4M3 || a_dtype == GEMM_FP8_E5M2;
    const bool fb8 = b_dtype == GEMM_FP8_E4M3 || b_dtype == GEMM_FP8_E5M2;
    if (!fa8 || !fb8)
        return GEMM_ERR_UNSUPPORTED;
    if (scale_mode != GEMM_SCALE_TENSOR && scale_mode != GEMM_SCALE_BLOCK)
        return GEMM_ERR_INVALID_ARG;
    const bool blockwise = scale_mode == GEMM_SCALE_BLOCK;
    if (blockwise && block_m != 1 && block_m != 128)
        return GEMM_ERR_INVALID_ARG;
    gemm_status_t st = check_epilogue(epi, false);
    if (st != GEMM_OK)
        return st;
    if (epi && epi->bias)
        return GEMM_ERR_INVALID_ARG;
    const bool with_bias = epi && epi->bias_along != GEMM_BIAS_NONE;
    std::vector<gnt::GroupDesc> descs;
    descs.reserve(num_groups);
    int64_t tiles = 0;
    for (int g = 0; g < num_groups; ++g) {
        const gemm_group_problem_fp8_t &q = problems[g];
        st = validate(q.A, q.B, q.C, q.M, q.N, q.K, q.lda, q.ldb, q.ldc, q.K, q.K, GEMM_BF16,
                      out_dtype);
        if (st != GEMM_OK)
            return st;
        const bool empty = q.M == 0 || q.N == 0;
        if (!empty && (!q.scale_a || !q.scale_b || (uintptr_t)q.scale_a % 4 ||
                       (uintptr_t)q.scale_b % 4))
            return GEMM_ERR_INVALID_ARG;
        if (with_bias && !empty && (!q.bias || (uintptr_t)q.bias % 4))
            return GEMM_ERR_INVALID_ARG;
        if (!empty && q.K % 16)
            return GEMM_ERR_UNSUPPORTED;
        if (!empty && (q.lda % 16 || q.ldb % 16))
            return GEMM_ERR_MISALIGNED;
        const int64_t nkb = (q.K + 127) / 128;
        const int64_t sfa = blockwise ? (q.M + block_m - 1) / block_m * nkb * 4 : 4;
        const int64_t sfb = blockwise ? (q.N + 127) / 128 * nkb * 4 : 4;
        if (sfa >= INT32_MAX || sfb >= INT32_MAX)
            return GEMM_ERR_UNSUPPORTED;
        gnt::GroupDesc d{};
        d.A = static_cast<const uint16_t *>(q.A);
        d.B = static_cast<const uint16_t *>(q.B);
        d.C = q.C;
        d.bias = with_bias ? q.bias : nullptr;
        d.M = (int)q.M, d.N = (int)q.N, d.K = (int)q.K;
        d.lda = (int)q.lda, d.ldb = (int)q.ldb, d.ldc = (int)q.ldc;
        d.tiles_m = (int)cdiv(q.M, 256);
        d.tiles_n = (int)cdiv(q.N, 256);
        d.k_tiles = (int)nkb;            // a slab is 128 FP8 values
        d.tile_start = (int)tiles;
        d.sf_ld = (int)nkb;
        d.scale_a = q.scale_a;
        d.scale_b = q.scale_b;
        d.sfa_bytes = (uint32_t)sfa;
        d.sfb_bytes = (uint32_t)sfb;
        const int64_t out_size = out_dtype == GEMM_FP32 ? 4 : 2;
        const uintptr_t vec_bytes = out_dtype == GEMM_FP32 ? 16 : 8;
        d.flags = ((q.ldc % 4 == 0) && ((uintptr_t)q.C % vec_bytes == 0) ? gnt::GD_VEC_STORE : 0) |
                  (((q.ldc * out_size) % 16 == 0) && ((uintptr_t)q.C % 16 == 0) ? gnt::GD_ROWS16 : 0) |
                  (d.bias && (uintptr_t)d.bias % 16 == 0 ? gnt::GD_BIAS_VEC : 0) |
                  (d.tiles_m <= 2 ? gnt::GD_NT_B : 0);
        descs.push_back(d);
        tiles += (int64_t)d.tiles_m * d.tiles_n;
        if (tiles >= INT32_MAX)
            return GEMM_ERR_UNSUPPORTED;
    }
    if (tiles == 0)
        return GEMM_OK;
    KernelArgs a{};
    fill_group_epilogue(a, epi);
    a.sfa_shift = block_m == 128 ? 7 : 0;
    static LaunchTableRef const kF8G[2][2] = {{gnt::kPP2_f8_e4e4_grouped, gnt::kPP2_f8_e4e5_grouped},
                                              {gnt::kPP2_f8_e5e4_grouped, gnt::kPP2_f8_e5e5_grouped}};
    const launch_fn fn =
        kF8G[a_dtype == GEMM_FP8_E5M2][b_dtype == GEMM_FP8_E5M2][scale_mode][out_dtype];
    if (h->log)
        fprintf(stderr, "gemm_nt: grouped FP8, %d groups, %lld tiles\n", num_groups,
                (long long)tiles);
    return stage_and_launch(h, descs, tiles, a, fn, stream);
}

}  // namespace

extern "C" {

gemm_status_t gemm_run_grouped_fp8(gemm_handle_t h, int a_dtype, int b_dtype,
                                   const gemm_group_problem_fp8_t *problems, int num_groups,
                                   int out_dtype, int scale_mode, int block_m,
                                   const gemm_epilogue_t *epi, hipStream_t stream)
{
    try {
        return run_grouped_fp8(h, a_dtype, b_dtype, problems, num_groups, out_dtype, scale_mode,
                               block_m, epi, stream);
    } catch (...) {
        return GEMM_ERR_ALLOC;
    }
}

gemm_status_t gemm_run_grouped(gemm_handle_t h, const gemm_group_problem_t *problems,
                               int num_groups, int in_dtype, int out_dtype,
                               const gemm_epilogue_t *epi, hipStream_t stream)
{
    // the host-side problem list is built in std::vectors: no exception may
    // cross the C boundary
    try {
        return run_grouped(h, problems, num_groups, in_dtype, out_dtype, epi, stream);
    } catch (...) {
        return GEMM_ERR_ALLOC;
    }
}

gemm_status_t gemm_run_fp8(gemm_handle_t h, int a_dtype, int b_dtype, const void *A,
                           const void *B, void *C, int64_t M, int64_t N, int64_t K, int64_t lda,
                           int64_t ldb, int64_t ldc, int out_dtype,
                           const gemm_fp8_scales_t *scales, const gemm_epilogue_t *epi,
                           hipStream_t stream)
{
    if (!h || !scales)
        return GEMM_ERR_INVALID_ARG;
    const bool fa8 = a_dtype == GEMM_FP8_E4M3 || a_dtype == GEMM_FP8_E5M2;
    const bool fb8 = b_dtype == GEMM_FP8_E4M3 || b_dtype == GEMM_FP8_E5M2;
    if (!fa8 || !fb8)
        return GEMM_ERR_UNSUPPORTED;
    // the 16-bit checks (sizes, leading dimensions, output, alignment of the
    // bases), then the FP8 row granularity: 16 elements = 16 bytes
    gemm_status_t st = validate(A, B, C, M, N, K, lda, ldb, ldc, K, K, GEMM_BF16, out_dtype);
    if (st != GEMM_OK)
        return st;
    if (scales->mode != GEMM_SCALE_TENSOR && scales->mode != GEMM_SCALE_BLOCK)
        return GEMM_ERR_INVALID_ARG;
    if (scales->mode == GEMM_SCALE_BLOCK && scales->block_m != 1 && scales->block_m != 128)
        return GEMM_ERR_INVALID_ARG;
    if (!scales->a || !scales->b || (uintptr_t)scales->a % 4 || (uintptr_t)scales->b % 4)
        return GEMM_ERR_INVALID_ARG;
    if ((st = check_epilogue(epi)) != GEMM_OK)
        return st;
    if (M == 0 || N == 0)
        return GEMM_OK;
    if (K % 16)
        return GEMM_ERR_UNSUPPORTED;
    if (lda % 16 || ldb % 16)
        return GEMM_ERR_MISALIGNED;
    const int64_t nkb = (K + 127) / 128;
    const int64_t sfa_rows = scales->mode == GEMM_SCALE_BLOCK ? (M + scales->block_m - 1) / scales->block_m : 1;
    const int64_t sfb_rows = scales->mode == GEMM_SCALE_BLOCK ? (N + 127) / 128 : 1;
    const int64_t sfa_bytes = sfa_rows * (scales->mode == GEMM_SCALE_BLOCK ? nkb : 1) * 4;
    const int64_t sfb_bytes = sfb_rows * (scales->mode == GEMM_SCALE_BLOCK ? nkb : 1) * 4;
    if (sfa_bytes >= INT32_MAX || sfb_bytes >= INT32_MAX)
        return GEMM_ERR_UNSUPPORTED;
    if ((st = check_device(h)) != GEMM_OK)
        return st;
    if (h->force_cfg >= 0 && h->force_cfg != CFG_PP2_256x256)
        return GEMM_ERR_UNSUPPORTED;
    // A slab is 128 bytes of each row: 128 FP8 values, planned as 64 16-bit ones
    const Plan p = handle_plan(h, M, N, K / 2, CFG_PP2_256x256, 0, h->inreduce);
    KernelArgs a{};
    a.A = static_cast<const uint16_t *>(A);
    a.B = static_cast<const uint16_t *>(B);
    a.lda = (int)lda;
    a.ldb = (int)ldb;
    a.scale_a = scales->a;
    a.scale_b = scales->b;
    a.sf_ld = (int)nkb;
    a.sfa_shift = scales->block_m == 128 ? 7 : 0;
    a.sfa_bytes = (uint32_t)sfa_bytes;
    a.sfb_bytes = (uint32_t)sfb_bytes;
    static LaunchTableRef const kF8[2][2] = {{gnt::kPP2_f8_e4e4, gnt::kPP2_f8_e4e5},
                                             {gnt::kPP2_f8_e5e4, gnt::kPP2_f8_e5e5}};
    const launch_fn fn = kF8[a_dtype == GEMM_FP8_E5M2][b_dtype == GEMM_FP8_E5M2][scales->mode][out_dtype];
    return enqueue(workspace_of(h), p, a, fn, C, M, N, K, ldc, out_dtype, epi, stream);
}

}  // extern "C"
