// gemm_nt_common.hpp -- pieces shared by the gfx950 NT GEMM kernels: vector
// types, the kernel argument block, buffer-resource and direct-to-LDS load
// helpers, hand-placed waits and barriers, the MFMA wrapper, the LDS row
// swizzle, the XCD-aware tile order and the epilogue store.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gnt {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// Input formats: the 16-bit ones, and the FP8 pairs IN_F8 + 2 * (A is E5M2) +
// (B is E5M2), each operand E4M3 or E5M2 (OCP 8-bit floating point).
enum : int { IN_BF16 = 0, IN_FP16 = 1, IN_F8 = 2 };
enum : int { OUT_BF16 = 0, OUT_FP16 = 1, OUT_FP32 = 2 };

// One problem of a grouped launch ("CUTLASS Deep Dive", "Grouped GEMM -- MoE's
// workhorse": each tile looks up its problem, then runs the usual mainloop).
// Written by the host into device memory, one per group.
struct GroupDesc {
    const uint16_t *A;
    const uint16_t *B;
    void *C;
    const float *bias;     // FP32 bias of this group (when the epilogue has one)
    int M, N, K;
    int lda, ldb, ldc;     // elements
    int tile_start;        // the group's first position in the launch's tile list
    int tiles_m, tiles_n, k_tiles;
    int flags;             // GD_VEC_STORE | GD_ROWS16 | GD_BIAS_VEC | GD_NT_B
    int sf_ld;             // FP8: k-blocks per scale row
    const float *scale_a;  // FP8: this group's scales (per tensor or blockwise)
    const float *scale_b;
    uint32_t sfa_bytes, sfb_bytes;
};
enum : int { GD_VEC_STORE = 1, GD_ROWS16 = 2, GD_BIAS_VEC = 4, GD_NT_B = 8 };

struct KernelArgs {
    const uint16_t *A;
    const uint16_t *B;
    void *C;
    int M, N, K;
    int lda, ldb, ldc;     // elements
    int tiles_m, tiles_n;
    int k_tiles;           // ceil(K / BK)
    int splits;            // K splits per tile (1 = none)
    int kt_per_split;      // k-slabs per split
    int group_m;           // tile rows per group of the tile order
    int vec_store;         // 1 when 4 consecutive C elements may be stored as one vector
    int rows16;            // 1 when every row of C starts 16-byte aligned
    int nt_b;              // 1: B is loaded with the non-temporal policy (at most two
                           // tile rows, so each B element is read by at most two blocks)
    float *partials;       // split-K partials, dense [splits][M][N] FP32; stream-K
                           // partials, [block][segment][256][256] FP32
    int sk_units;          // stream-K: tiles * k_tiles (0: off); block b of the grid G
                           // takes units [b T / G, (b + 1) T / G) in tile-major order
    int sk_maxseg;         // stream-K: partial slots per block
    int inreduce;          // two K splits reduced in the kernel: partial of tile t,
                           // split s in slot 2 t + s of `partials` (in register
                           // order), arrivals counted in counters[t]
    unsigned *counters;    // per-tile arrival counters, zero between calls
    // fused epilogue D = act(alpha * acc + beta * C_old + bias), applied when epi != 0
    float alpha, beta;
    const float *bias;     // FP32, N values (bias_along == 1) or M values (2)
    int bias_along;        // 0 none, 1 along n (one per column), 2 along m (one per row)
    int act;               // 0 none, 1 ReLU, 2 GELU (x * Phi(x), erf form)
    int bias_vec;          // 1 when the bias pointer is 16-byte aligned
    int epi;               // 1 when the epilogue is not the identity
    // FP8 scales: one FP32 value each (per tensor), or blockwise: A's
    // [ceil(M / 2^sfa_shift)][sf_ld] and B's [ceil(N / 128)][sf_ld] row-major,
    // sf_ld = ceil(K / 128) blocks along K
    const float *scale_a;
    const float *scale_b;
    int sf_ld;
    int sfa_shift;         // log2 of the rows per A scale (0 or 7)
    uint32_t sfa_bytes, sfb_bytes;
    // grouped launch: the problems, and each launch position's problem index
    const GroupDesc *groups;
    const int *tile_group;
};

// The order in which a tile visits the k-slabs of its range [kt0, kt0 + nk).
// With ROT, local slab i is slab kt0 + (i + rot) mod nf for i < nf.  Here nf
// counts the range's whole slabs, and rot = (n0 / 256) mod nf for a tile
// whose first column is n0.  A partial last slab of K keeps its place at the
// end, where the kernels' K-tail handling expects it.  So tiles of
// neighbouring 256-column blocks start at different slabs.  When every block
// walks K in step, all the rows a launch reads at one moment sit at one
// offset within their row.  With a power-of-two row pitch those addresses
// share their low bits, and the requests load a few memory channels only.  A
// streaming probe of a decode-shaped B operand (28672 rows of 16 KB, 224
// blocks reading 128 bytes of 256 rows per step) reached 4.7 TB/s in step and
// 6.1 TB/s with the starts rotated when consecutive blocks took consecutive
// tiles, and 5.6-5.8 against 6.0 in the kernels' XCD-aware block order; in the
// small-M tile kernels rotation measured 5-25% faster (the host's rule,
// rotate_slabs, also says why the 256-row tiles never rotate).  The slab sum
// is the same sum in another order, fixed by an output's 256-column block and
// its split's range: every launch of a shape gives the same bits.  Without
// ROT, slab kt0 + i: the order is a template parameter because its few scalar
// instructions per slab measured about 1% on the large shapes.
template <bool ROT>
struct SlabOrder {
    int kt0, nf, rot;
    __device__ __forceinline__ int operator()(int i) const
    {
        if constexpr (!ROT)
            return kt0 + i;
        const int j = i + rot;
        const int r = j - (j >= nf ? nf : 0);
        return kt0 + (i < nf ? r : i);
    }
};

// `partial_last`: K is not a multiple of the slab depth.
template <bool ROT>
__device__ __forceinline__ SlabOrder<ROT> slab_order(int kt0, int nk, int k_tiles, bool partial_last, int n0)
{
    if constexpr (!ROT)
        return SlabOrder<ROT>{kt0, nk, 0};
    const int nf = nk - ((partial_last && kt0 + nk == k_tiles) ? 1 : 0);
    return SlabOrder<ROT>{kt0, nf, nf > 1 ? (n0 >> 8) % nf : 0};
}

// Keep a scalar computed where it stands: the empty asm reads and writes it,
// so the arithmetic behind it cannot sink past the barriers to its first use.
__device__ __forceinline__ void pin_scalar(int &x) { asm volatile("" : "+s"(x)); }

// Byte offset added to a load that must return zeros: beyond every buffer's
// num_records, so the buffer unit returns 0 without touching memory.
constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    // word 3: the gfx9 raw-buffer format (32-bit data, no swizzle, no stride).
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

// One wave-wide 16-byte-per-lane load written straight into LDS at
// lds_addr + 16 * lane.  Issued through asm so the compiler does not treat every
// later LDS read as dependent on it; completion is tracked with vmcnt by hand.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff,
                                           uint32_t lds_addr)
{
    asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds"
                 :
                 : "v"(voff), "s"(rs), "s"(soff), "{m0}"(lds_addr));
}

// load_lds16 with the non-temporal cache policy when NT: for an operand whose
// bytes the launch reads once or twice, so that its lines do not take the place
// of lines many blocks will read again.  A template flag, so the policy is an
// immediate of the instruction and the load path has no branch.
template <bool NT>
__device__ __forceinline__ void load_lds16_policy(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff,
                                                  uint32_t lds_addr)
{
    if constexpr (NT)
        asm volatile("buffer_load_dwordx4 %0, %1, %2 offen nt lds"
                     :
                     : "v"(voff), "s"(rs), "s"(soff), "{m0}"(lds_addr));
    else
        load_lds16(rs, voff, soff, lds_addr);
}

// One wave-wide 4-byte-per-lane load into LDS at lds_addr + 4 * lane (lanes
// whose offset is out of range write zeros), completion tracked with vmcnt by
// hand like load_lds16.  Also used to pull cache lines into L2 ahead of their
// real load, with the LDS bytes dropped (touch_lds4).
__device__ __forceinline__ void load_lds4(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff,
                                          uint32_t lds_addr)
{
    asm volatile("buffer_load_dword %0, %1, %2 offen lds"
                 :
                 : "v"(voff), "s"(rs), "s"(soff), "{m0}"(lds_addr));
}

__device__ __forceinline__ void touch_lds4(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff,
                                           uint32_t lds_addr)
{
    asm volatile("buffer_load_dword %0, %1, %2 offen lds"
                 :
                 : "v"(voff), "s"(rs), "s"(soff), "{m0}"(lds_addr));
}

template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void wait_lgkmcnt0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }

template <int IN>
__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c)
{
    if constexpr (IN == IN_BF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// One v_mfma_f32_32x32x64_f8f6f4: the 32 k-values of a lane's row come from
// two 16-byte fragments (k 0..15 and 16..31 of its half of the 64-deep step).
// The B tile is the first operand, so its format goes in the first format field.
template <int IN>
__device__ __forceinline__ f32x16 mfma32x32x64_f8(u32x4 b0, u32x4 b1, u32x4 a0, u32x4 a1, f32x16 c)
{
    constexpr int fa = (IN - IN_F8) >> 1, fb = (IN - IN_F8) & 1;
    const i32x8 x = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3],
                     (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
    const i32x8 y = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                     (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
    // zero scale operands select the unscaled instruction
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, y, c, fb, fa, 0, 0, 0, 0);
}

// Swizzle key of LDS row r for a row of CH 16-byte chunks.  Depends only on
// r mod 16, so every 16-row group a load fills and every 32-row MFMA operand
// block sees the same pattern.  Sixteen consecutive rows reading one logical
// chunk land in sixteen different groups of four banks (of 64): for 128-byte
// rows through the low three row bits and the row's half of the bank array,
// for 64-byte rows through r mod 4 (which quarter of the banks the row starts
// in) and (r / 4) mod 4.
template <int CH>
__device__ __forceinline__ int row_key(int r)
{
    if constexpr (CH == 8)
        return (r & 7) ^ ((r >> 3) & 1);
    else
        return (r >> 2) & 3;
}

// Launch-order position of block `bid` among G blocks: the hardware deals
// consecutive block ids round-robin over the 8 XCDs, so renumbering gives each
// XCD one contiguous run of positions (tiles that share operand panels in its
// private L2).
__device__ __forceinline__ int xcd_order(int bid, int G)
{
    const int x = bid & 7, slot = bid >> 3;
    const int q = G >> 3, r = G & 7;
    return x * q + (x < r ? x : r) + slot;
}

// Tile t of a tiles_m x tiles_n grid in grouped order: groups of group_m tile
// rows, column by column within a group.
__device__ __forceinline__ void tile_order(int t, int tiles_m, int tiles_n, int group_m, int &tm,
                                           int &tn)
{
    const int per_group = group_m * tiles_n;
    const int g = t / per_group;
    const int first_m = g * group_m;
    const int gsz = (tiles_m - first_m) < group_m ? (tiles_m - first_m) : group_m;
    const int w = t - g * per_group;
    tm = first_m + w % gsz;
    tn = w / gsz;
}

// Block id -> (tile row, tile column, K split).  See the header comment.
__device__ __forceinline__ void map_block(int bid, int G, int tiles_m, int tiles_n, int group_m,
                                          int &tm, int &tn, int &split)
{
    const int v = xcd_order(bid, G);
    const int tiles = tiles_m * tiles_n;
    split = v / tiles;
    tile_order(v - split * tiles, tiles_m, tiles_n, group_m, tm, tn);
}

// Block id -> (tile row, tile column, K split) with the K splits of one tile
// adjacent in launch order: they then fall in one XCD's contiguous run of
// positions (xcd_order), next to each other in its L2, which is where the
// in-kernel split-K reduction exchanges their partials.
__device__ __forceinline__ void map_block_split_minor(int bid, int G, int tiles_m, int tiles_n, int group_m,
                                                      int splits, int &tm, int &tn, int &split)
{
    const int v = xcd_order(bid, G);
    const int t = v / splits;
    split = v - t * splits;
    tile_order(t, tiles_m, tiles_n, group_m, tm, tn);
}

// Two K splits reduced inside the GEMM kernel ("A Blackwell GEMM by Hand in
// CuTe DSL", section 9: split-K for decode, here with the partials combined by
// the two CTAs themselves instead of a second pass).  Each split of tile t
// stores its FP32 partial in register order (lane l's register group g of wave
// w at byte (w * G + g) * 1024 + 16 l of its slot: each store instruction
// writes 1 KB contiguously) with device-coherent stores, waits for them, and
// counts its arrival on counters[t].  The split that arrives second adds the
// other's partial to its registers as 0 + (own + other): IEEE addition is
// commutative, so the bits are the same whichever split came second, and they
// equal those of the ordered second pass, (0 + p0) + p1.  It resets the
// counter for the next call and returns true; the first returns false and is
// done.  No block waits for another, so there is no spin and no dependence on
// which blocks are resident.  `flag` is a word of LDS no wave is using; every
// wave of the block calls this with its own accumulators (NW waves, G register
// groups of four per lane).
template <int NW, int FN, int FM>
__device__ __forceinline__ bool splitk2_arrive(const KernelArgs &p, f32x16 (&acc)[FN][FM], int tile, int split,
                                               int wave, int lane, uint32_t *flag)
{
    constexpr int G = FN * FM * 4;                        // register groups per lane
    constexpr uint32_t SLOT = (uint32_t)NW * G * 1024u;   // bytes per split partial
    constexpr int SC1 = 16;                               // device-coherent access
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(reinterpret_cast<const uint8_t *>(p.partials) + (int64_t)tile * 2 * SLOT, 2u * SLOT);
    const uint32_t vo = (uint32_t)(wave * G) * 1024u + (uint32_t)lane * 16u;
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int g = (fn * FM + fm) * 4 + q;
                const f32x4 v = {acc[fn][fm][4 * q], acc[fn][fm][4 * q + 1], acc[fn][fm][4 * q + 2],
                                 acc[fn][fm][4 * q + 3]};
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, vo + g * 1024u,
                                                       (uint32_t)split * SLOT, SC1);
                // a few stores at a time, so the accumulators are not all copied out first
                if ((g & 3) == 3)
                    __builtin_amdgcn_sched_barrier(0);
            }
    wait_vmcnt<0>();
    wg_barrier();
    if (wave == 0 && lane == 0)
        *flag = __hip_atomic_fetch_add(p.counters + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    wg_barrier();
    const uint32_t arrived = __builtin_amdgcn_readfirstlane(*flag);
    wg_barrier();                                         // every wave has read the flag
    if (arrived == 0)
        return false;
    const uint32_t other = (uint32_t)(split ^ 1) * SLOT;
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int g = (fn * FM + fm) * 4 + q;
                const f32x4 o = __builtin_bit_cast(
                    f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, vo + g * 1024u, other, SC1));
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc[fn][fm][4 * q + e] = 0.0f + (acc[fn][fm][4 * q + e] + o[e]);
                // eight loads in flight at a time: enough to cover the latency,
                // few enough registers to keep every accumulator in place
                if ((g & 7) == 7)
                    __builtin_amdgcn_sched_barrier(0);
            }
    if (wave == 0 && lane == 0)
        __hip_atomic_store(p.counters + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
}

// Any number S = p.splits >= 2 of K splits reduced inside the kernel, by the
// last of a tile's splits to finish (the tile kernels; the same exchange as
// splitk2_arrive).  Each split stores its FP32 partial in register order into
// slot `split` of the tile's S slots with device-coherent stores, waits for
// them and counts its arrival on counters[tile].  The split that counts last
// adds the partials in split order, ((0 + p_0) + p_1) + ..., its own from its
// registers and the others' with device-coherent loads, the loads of RS splits
// in flight at a time.  That is the order, hence the bits, of the second pass
// (splitk_sum), whichever split came last.  It resets the counter for the
// next call and returns true; the others return false and are done.  No block
// waits for another.  `flag` is a word of LDS no wave is using.
template <int NW, int FN, int FM>
__device__ __forceinline__ bool splitk_arrive(const KernelArgs &p, f32x16 (&acc)[FN][FM], int tile, int split,
                                              int wave, int lane, uint32_t *flag)
{
    constexpr int G = FN * FM * 4;                        // register groups per lane
    constexpr uint32_t SLOT = (uint32_t)NW * G * 1024u;   // bytes per split partial
    constexpr int SC1 = 16;                               // device-coherent access
    constexpr int RS = G >= 16 ? 1 : 16 / G;              // splits read per round
    const int S = p.splits;
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(reinterpret_cast<const uint8_t *>(p.partials) + (int64_t)tile * S * SLOT, (uint32_t)S * SLOT);
    const uint32_t vo = (uint32_t)(wave * G) * 1024u + (uint32_t)lane * 16u;
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int g = (fn * FM + fm) * 4 + q;
                const f32x4 v = {acc[fn][fm][4 * q], acc[fn][fm][4 * q + 1], acc[fn][fm][4 * q + 2],
                                 acc[fn][fm][4 * q + 3]};
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, vo + g * 1024u,
                                                       (uint32_t)split * SLOT, SC1);
            }
    wait_vmcnt<0>();
    wg_barrier();
    if (wave == 0 && lane == 0)
        *flag = __hip_atomic_fetch_add(p.counters + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    wg_barrier();
    const uint32_t arrived = __builtin_amdgcn_readfirstlane(*flag);
    wg_barrier();                                         // every wave has read the flag
    if (arrived != (uint32_t)(S - 1))
        return false;
    f32x4 tot[G];
#pragma unroll
    for (int g = 0; g < G; ++g)
        tot[g] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
    for (int s0 = 0; s0 < S; s0 += RS) {
        f32x4 buf[RS][G];
#pragma unroll
        for (int c = 0; c < RS; ++c) {
            const int s = s0 + c;
            if (s < S && s != split) {
#pragma unroll
                for (int g = 0; g < G; ++g)
                    buf[c][g] = __builtin_bit_cast(
                        f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, vo + g * 1024u, (uint32_t)s * SLOT, SC1));
            }
        }
#pragma unroll
        for (int c = 0; c < RS; ++c) {
            const int s = s0 + c;
            if (s >= S)
                continue;
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int g = (fn * FM + fm) * 4 + q;
                        const f32x4 own = {acc[fn][fm][4 * q], acc[fn][fm][4 * q + 1], acc[fn][fm][4 * q + 2],
                                           acc[fn][fm][4 * q + 3]};
                        tot[g] += s == split ? own : buf[c][g];
                    }
        }
    }
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc[fn][fm][4 * q + e] = tot[(fn * FM + fm) * 4 + q][e];
    if (wave == 0 && lane == 0)
        __hip_atomic_store(p.counters + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
}

template <int OUT>
__device__ __forceinline__ void store4(void *C, int64_t idx, f32x4 v, bool vec, int valid)
{
    if constexpr (OUT == OUT_FP32) {
        float *c = static_cast<float *>(C) + idx;
        if (vec && valid >= 4) {
            *reinterpret_cast<f32x4 *>(c) = v;
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (i < valid)
                    c[i] = v[i];
        }
    } else {
        uint16_t h[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (OUT == OUT_BF16)
                h[i] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v[i]));
            else
                h[i] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(v[i]));
        }
        uint16_t *c = static_cast<uint16_t *>(C) + idx;
        if (vec && valid >= 4) {
            u32x2 w;
            w[0] = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
            w[1] = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
            *reinterpret_cast<u32x2 *>(c) = w;
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (i < valid)
                    c[i] = h[i];
        }
    }
}

// Zero the elements of an 8-value operand chunk from index `nvalid` on.
__device__ __forceinline__ u32x4 mask_chunk(u32x4 x, int nvalid)
{
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        uint32_t m = (2 * d < nvalid ? 0x0000FFFFu : 0u) | (2 * d + 1 < nvalid ? 0xFFFF0000u : 0u);
        x[d] &= m;
    }
    return x;
}

// The prior contents of C[m][n .. n+3] (the first `valid` of them) as FP32.
template <int OUT>
__device__ __forceinline__ f32x4 load4(const void *C, int64_t idx, bool vec, int valid)
{
    f32x4 r = {0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (OUT == OUT_FP32) {
        const float *c = static_cast<const float *>(C) + idx;
        if (vec && valid >= 4) {
            r = *reinterpret_cast<const f32x4 *>(c);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (i < valid)
                    r[i] = c[i];
        }
    } else {
        const uint16_t *c = static_cast<const uint16_t *>(C) + idx;
        uint16_t h[4] = {0, 0, 0, 0};
        if (vec && valid >= 4) {
            const u32x2 w = *reinterpret_cast<const u32x2 *>(c);
            h[0] = (uint16_t)w[0];
            h[1] = (uint16_t)(w[0] >> 16);
            h[2] = (uint16_t)w[1];
            h[3] = (uint16_t)(w[1] >> 16);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (i < valid)
                    h[i] = c[i];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (OUT == OUT_BF16)
                r[i] = static_cast<float>(__builtin_bit_cast(__bf16, h[i]));
            else
                r[i] = static_cast<float>(__builtin_bit_cast(_Float16, h[i]));
        }
    }
    return r;
}

// GELU in its exact form x * Phi(x) = x / 2 * (1 + erf(x / sqrt 2)), with erf
// from Abramowitz and Stegun, Handbook of Mathematical Functions, formula
// 7.1.26: erf(z) = 1 - t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-z^2),
// t = 1 / (1 + p z) for z >= 0, odd in z, |error| <= 1.5e-7.  About a dozen
// VALU operations against several dozen for the library erf; the formula's
// error, below 2^-22 of |x| in the result, is inside the epilogue's bound.
__device__ __forceinline__ float gelu_erf(float x)
{
    const float z = fabsf(x) * 0.70710678118654752440f;
    const float t = __builtin_amdgcn_rcpf(1.0f + 0.3275911f * z);
    float poly = 1.061405429f;
    poly = poly * t - 1.453152027f;
    poly = poly * t + 1.421413741f;
    poly = poly * t - 0.284496736f;
    poly = poly * t + 0.254829592f;
    const float e = 1.0f - poly * t * __expf(-z * z);   // erf(|x| / sqrt 2)
    return 0.5f * x * (1.0f + copysignf(e, x));
}

// Fused epilogue ("CUTLASS Deep Dive", the Tutorial 01/05 epilogues and the
// EVT / "Bias + ReLU" passages: alpha times the accumulator plus beta times
// the existing C, plus a bias, through an activation, in one pass as the tile
// is written back) on the FP32 sums of C[m][n .. n+3], the first `valid` of
// which are inside the output.  Every value is read and then written by the
// same lane, so reading C_old here is race-free.
template <int OUT>
__device__ __forceinline__ f32x4 epilogue4(const KernelArgs &p, int m, int n, f32x4 x, int valid)
{
    const int64_t idx = (int64_t)m * p.ldc + n;
    f32x4 old = {0.0f, 0.0f, 0.0f, 0.0f};
    if (p.beta != 0.0f)
        old = load4<OUT>(p.C, idx, p.vec_store != 0, valid);
    // n is a multiple of 4 at every call, so bias + n is 16-byte aligned with bias
    f32x4 b = {0.0f, 0.0f, 0.0f, 0.0f};
    if (p.bias_along == 1) {
        if (p.bias_vec && valid >= 4) {
            b = *reinterpret_cast<const f32x4 *>(p.bias + n);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (i < valid)
                    b[i] = p.bias[n + i];
        }
    } else if (p.bias_along == 2) {
        const float bm = p.bias[m];
        b = (f32x4){bm, bm, bm, bm};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float v = p.alpha * x[i];
        if (p.beta != 0.0f)
            v += p.beta * old[i];
        v += b[i];
        if (p.act == 1)
            v = fmaxf(v, 0.0f);
        else if (p.act == 2)
            v = gelu_erf(v);
        x[i] = v;
    }
    return x;
}

// Epilogue of one lane's 4-element group C[m][n .. n+3] (n < N).  Without a
// K split the FP32 sum is converted and stored into C; with one, the split's
// FP32 partial goes to its slice of the workspace (dense [split][M][N]) and the
// reduction kernel below finishes the job.
template <int OUT>
__device__ __forceinline__ void store_result(const KernelArgs &p, int split, int m, int n, f32x4 x)
{
    const int valid = p.N - n;
    if (p.splits > 1) {
        float *ws = p.partials + (int64_t)split * p.M * p.N;
        store4<OUT_FP32>(ws, (int64_t)m * p.N + n, x, (p.N & 3) == 0, valid);
    } else {
        if (p.epi)
            x = epilogue4<OUT>(p, m, n, x, valid);
        store4<OUT>(p.C, (int64_t)m * p.ldc + n, x, p.vec_store != 0, valid);
    }
}

// One wave's block of C (or of a split-K partial) written through LDS with
// lane-contiguous stores, for any row alignment of the output.  The block is
// (32 FM) x (32 FN) accumulators in the MFMA layout: lane l holds rows
// 32 fm + l % 32, columns 32 fn + 8 q + 4 (l / 32) .. +4.  It is staged as FP32
// rows of 32 FN values, the 16-byte chunk c of row r at chunk c ^ (r & KEYM), so
// the column-wise staging writes spread over the banks.  The read-back gives
// lane l consecutive columns of one row, so every store instruction (4 or 2
// bytes per lane) writes whole row segments, where the direct stores of the
// MFMA layout touch 32 rows per instruction.  Elements at or past (rows, cols)
// are not stored.  Only the calling wave touches `stage`
// (4096 FM FN bytes).
template <int OUT, int FN, int FM>
__device__ __forceinline__ void store_block_rows(const f32x16 (&acc)[FN][FM], uint8_t *stage, void *C,
                                                 int64_t ld, int rows, int cols, int lane)
{
    constexpr int DPR = 32 * FN;                      // values per staged row
    constexpr int ROWB = 4 * DPR;
    constexpr int KEYM = (DPR / 4 < 16 ? DPR / 4 : 16) - 1;
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = fm * 32 + (lane & 31);
                const int c = fn * 8 + 2 * q + (lane >> 5);
                const f32x4 v = {acc[fn][fm][4 * q], acc[fn][fm][4 * q + 1], acc[fn][fm][4 * q + 2],
                                 acc[fn][fm][4 * q + 3]};
                *reinterpret_cast<f32x4 *>(stage + r * ROWB + ((c ^ (r & KEYM)) * 16)) = v;
            }
    wait_lgkmcnt0();
#pragma unroll 4
    for (int i = 0; i < FM * FN * 16; ++i) {
        const int idx = i * 64 + lane;
        const int r = idx / DPR, c = idx % DPR;
        const float x = *reinterpret_cast<const float *>(stage + r * ROWB + (((c >> 2) ^ (r & KEYM)) * 16) +
                                                         (c & 3) * 4);
        if (r < rows && c < cols) {
            const int64_t off = (int64_t)r * ld + c;
            if constexpr (OUT == OUT_FP32)
                static_cast<float *>(C)[off] = x;
            else if constexpr (OUT == OUT_BF16)
                static_cast<uint16_t *>(C)[off] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
            else
                static_cast<uint16_t *>(C)[off] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
        }
    }
}

// Epilogue through LDS for one wave's 64 x 128 block of C (full tile only).
// Staging C through shared memory and storing it with wide row-contiguous
// writes is what "Optimizing GEMMs using tcgen05 - Part 1" measures as its last
// phase (scattered stores replaced by one bulk store per block).  Here the
// accumulator layout gives each lane four consecutive columns of one row, so
// direct stores put only 16 bytes of a row per pair of lanes in each
// instruction; staged through the wave's own 16 KB of LDS, every store
// instruction writes whole 256- or 512-byte row segments.  The 16-byte chunk c
// of staged row r sits at chunk c ^ (r mod 16) to keep the column-wise writes
// off a single bank group.  Only the calling wave touches `stage`.
// acc is [FN = 4][FM = 2] blocks of 32 x 32; the block's first element is
// C[m0][n0] with m0, n0 relative to `dst`, which holds rows of `ld` elements.
// NT stores with the non-temporal policy: for C, which the launch does not
// read again (split-K partials, read next by the reduction, keep the default).
template <typename T, bool NT = false>
__device__ __forceinline__ void store_block_staged(const f32x16 (&acc)[4][2], uint8_t *stage, T *dst,
                                                   int64_t ld, int lane)
{
    constexpr int ES = sizeof(T);
    constexpr int ROWB = 128 * ES;           // staged row bytes (256 or 512)
    constexpr int CPR = ROWB / 16;           // 16-byte chunks per row
    constexpr int ROWS = 16384 / ROWB;       // rows per pass (64 or 32)
    constexpr int PASSES = 64 / ROWS;
    const int h = lane >> 5, r0 = lane & 31;
#pragma unroll
    for (int pass = 0; pass < PASSES; ++pass) {
        // write this pass's rows: fm blocks [pass * ROWS / 32, +ROWS / 32)
#pragma unroll
        for (int fmp = 0; fmp < ROWS / 32; ++fmp) {
            const int fm = pass * (ROWS / 32) + fmp;
            const int r = fmp * 32 + r0;   // row within this pass
#pragma unroll
            for (int fn = 0; fn < 4; ++fn)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int col = fn * 32 + 8 * q + 4 * h;
                    const int byte = col * ES;
                    const int c = (byte >> 4) ^ (r & 15);
                    uint8_t *a = stage + r * ROWB + c * 16 + (byte & 15);
                    if constexpr (ES == 4) {
                        f32x4 v = {acc[fn][fm][4 * q], acc[fn][fm][4 * q + 1], acc[fn][fm][4 * q + 2],
                                   acc[fn][fm][4 * q + 3]};
                        *reinterpret_cast<f32x4 *>(a) = v;
                    } else {
                        uint16_t e[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            if constexpr (__is_same(T, __bf16))
                                e[i] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(acc[fn][fm][4 * q + i]));
                            else
                                e[i] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(acc[fn][fm][4 * q + i]));
                        }
                        u32x2 w = {(uint32_t)e[0] | ((uint32_t)e[1] << 16), (uint32_t)e[2] | ((uint32_t)e[3] << 16)};
                        *reinterpret_cast<u32x2 *>(a) = w;
                    }
                }
        }
        wait_lgkmcnt0();
        // read back row-contiguous 16-byte chunks and store them
        constexpr int LPR = CPR;             // lanes per row in one read
        constexpr int RPR = 64 / LPR;        // rows per read instruction
#pragma unroll
        for (int j = 0; j < ROWS / RPR; ++j) {
            const int r = j * RPR + lane / LPR;
            const int c = lane % LPR;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(stage + r * ROWB + ((c ^ (r & 15)) * 16));
            T *g = dst + (int64_t)(pass * ROWS + r) * ld + c * (16 / ES);
            if constexpr (NT)
                __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(g));
            else
                *reinterpret_cast<u32x4 *>(g) = v;
        }
        wait_lgkmcnt0();
    }
}

// Raw prior-C values of four consecutive outputs (aligned vector load) and
// their FP32 values.
template <int OUT>
struct OldC {
    typedef u32x2 raw;
};
template <>
struct OldC<OUT_FP32> {
    typedef f32x4 raw;
};
template <int OUT>
__device__ __forceinline__ typename OldC<OUT>::raw load_old4(const void *C, int64_t idx)
{
    if constexpr (OUT == OUT_FP32)
        return *reinterpret_cast<const f32x4 *>(static_cast<const float *>(C) + idx);
    else
        return *reinterpret_cast<const u32x2 *>(static_cast<const uint16_t *>(C) + idx);
}
template <int OUT>
__device__ __forceinline__ f32x4 old4_value(typename OldC<OUT>::raw w)
{
    if constexpr (OUT == OUT_FP32) {
        return w;
    } else {
        f32x4 r;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint16_t h = (uint16_t)(w[i >> 1] >> (16 * (i & 1)));
            if constexpr (OUT == OUT_BF16)
                r[i] = static_cast<float>(__builtin_bit_cast(__bf16, h));
            else
                r[i] = static_cast<float>(__builtin_bit_cast(_Float16, h));
        }
        return r;
    }
}

// The staged whole-tile store with the fused epilogue: a wave's 64 x 128 block
// goes through its 16 KB of LDS as FP32, 32 rows per pass, and the epilogue is
// applied on the way out, where each lane holds four consecutive columns of
// one row: the bias and prior-C loads are then row-contiguous vectors, and
// the accumulators need no extra registers.  The lane's bias vector is the
// same for every row; the prior C values of each step of rows are loaded one
// step ahead (the first before the staging writes), so their round trips
// overlap the LDS traffic and the arithmetic.  The first element of the
// block is C[m0][n0].
template <int OUT>
__device__ __forceinline__ void store_block_staged_epi(const KernelArgs &p, const f32x16 (&acc)[4][2],
                                                       uint8_t *stage, int m0, int n0, int lane)
{
    constexpr int ROWB = 512;                // 128 FP32 per staged row
    typedef typename OldC<OUT>::raw raw_t;
    const int h = lane >> 5, r0 = lane & 31;
    const int c = lane & 31, n = n0 + 4 * c;  // read-back chunk of this lane
    const bool has_old = p.beta != 0.0f;
    f32x4 bn = {0.0f, 0.0f, 0.0f, 0.0f};
    if (p.bias_along == 1)
        bn = p.bias_vec ? *reinterpret_cast<const f32x4 *>(p.bias + n)
                        : (f32x4){p.bias[n], p.bias[n + 1], p.bias[n + 2], p.bias[n + 3]};
    // step s = SP fm + t covers rows fm * 32 + 2 (J t + j) + lane / 32, j < J: 8-row
    // steps for 16-bit outputs, 4-row steps for FP32 (whose prior values take
    // twice the registers)
    constexpr int J = OUT == OUT_FP32 ? 4 : 8, SP = 16 / J;
    auto row_of = [&](int st, int j) { return (st / SP) * 32 + 2 * (J * (st % SP) + j) + (lane >> 5); };
    raw_t cur[J], nxt[J];
    if (has_old)
#pragma unroll
        for (int j = 0; j < J; ++j)
            cur[j] = load_old4<OUT>(p.C, (int64_t)(m0 + row_of(0, j)) * p.ldc + n);
#pragma unroll
    for (int fm = 0; fm < 2; ++fm) {
        // write rows fm*32 .. +32 (chunk c of row r at c ^ (r mod 16))
#pragma unroll
        for (int fn = 0; fn < 4; ++fn)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int col = fn * 32 + 8 * q + 4 * h;
                const int cc = (col >> 2) ^ (r0 & 15);
                f32x4 v = {acc[fn][fm][4 * q], acc[fn][fm][4 * q + 1], acc[fn][fm][4 * q + 2],
                           acc[fn][fm][4 * q + 3]};
                *reinterpret_cast<f32x4 *>(stage + r0 * ROWB + cc * 16) = v;
            }
        wait_lgkmcnt0();
#pragma unroll
        for (int t = 0; t < SP; ++t) {
            const int st = SP * fm + t;
            if (has_old && st + 1 < 2 * SP)
#pragma unroll
                for (int j = 0; j < J; ++j)
                    nxt[j] = load_old4<OUT>(p.C, (int64_t)(m0 + row_of(st + 1, j)) * p.ldc + n);
            f32x4 x[J];
#pragma unroll
            for (int j = 0; j < J; ++j) {
                const int r = row_of(st, j) - fm * 32;
                x[j] = *reinterpret_cast<const f32x4 *>(stage + r * ROWB + ((c ^ (r & 15)) * 16));
            }
#pragma unroll
            for (int j = 0; j < J; ++j) {
                const int m = m0 + row_of(st, j);
                const float bm = p.bias_along == 2 ? p.bias[m] : 0.0f;
                const f32x4 old = has_old ? old4_value<OUT>(cur[j]) : (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
                f32x4 y;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float v = p.alpha * x[j][e] + p.beta * old[e] + bn[e] + bm;
                    if (p.act == 1)
                        v = fmaxf(v, 0.0f);
                    else if (p.act == 2)
                        v = gelu_erf(v);
                    y[e] = v;
                }
                store4<OUT>(p.C, (int64_t)m * p.ldc + n, y, true, 4);
            }
#pragma unroll
            for (int j = 0; j < J; ++j)
                cur[j] = nxt[j];
        }
        wait_lgkmcnt0();
    }
}

// Split-K reduction ("A Blackwell GEMM by Hand in CuTe DSL", section 9: each
// CTA reduces a K slice, a second pass combines them).  One thread per group of
// four consecutive outputs of a row adds the partials in split order 0, 1, ...
// (a fixed order, so results are reproducible), converts, and stores.
template <int OUT>
__global__ __launch_bounds__(256) void splitk_sum(KernelArgs p)
{
    const int nvec = (p.N + 3) >> 2;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= (int64_t)p.M * nvec)
        return;
    const int m = (int)(t / nvec);
    const int n = (int)(t - (int64_t)m * nvec) * 4;
    const int valid = p.N - n;
    const int64_t plane = (int64_t)p.M * p.N;
    const float *src = p.partials + (int64_t)m * p.N + n;
    f32x4 sum = {0.0f, 0.0f, 0.0f, 0.0f};
    if ((p.N & 3) == 0) {
        for (int s = 0; s < p.splits; ++s)
            sum += *reinterpret_cast<const f32x4 *>(src + s * plane);
    } else {
        for (int s = 0; s < p.splits; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (i < valid)
                    sum[i] += src[s * plane + i];
    }
    if (p.epi)
        sum = epilogue4<OUT>(p, m, n, sum, valid);
    store4<OUT>(p.C, (int64_t)m * p.ldc + n, sum, p.vec_store != 0, valid);
}

// Stream-K reduction: the outputs of tile t are the sum of the partials of
// the blocks whose unit ranges meet [t k_tiles, (t + 1) k_tiles), added in block
// order (a fixed order, so results are reproducible), then the epilogue and the
// store.  Block b's range starts at floor(b T / G); the block holding unit u is
// ceil((u + 1) G / T) - 1, and tile t is segment t - floor(start(b) / k_tiles)
// of block b.  One thread per group of four consecutive outputs of a row.
template <int OUT>
__global__ __launch_bounds__(256) void streamk_sum(KernelArgs p, int G)
{
    const int nvec = (p.N + 3) >> 2;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= (int64_t)p.M * nvec)
        return;
    const int m = (int)(t / nvec);
    const int n = (int)(t - (int64_t)m * nvec) * 4;
    const int valid = p.N - n;
    const int tile = (m >> 8) * p.tiles_n + (n >> 8);
    const int64_t T = p.sk_units;
    const int64_t u0 = (int64_t)tile * p.k_tiles, u1 = u0 + p.k_tiles - 1;
    const int b0 = (int)(((u0 + 1) * G + T - 1) / T - 1);
    const int b1 = (int)(((u1 + 1) * G + T - 1) / T - 1);
    const int in_tile = (m & 255) * 256 + (n & 255);
    f32x4 sum = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int b = b0; b <= b1; ++b) {
        const int seg = tile - (int)(((int64_t)b * T / G) / p.k_tiles);
        const float *src = p.partials + ((int64_t)b * p.sk_maxseg + seg) * 65536 + in_tile;
        sum += *reinterpret_cast<const f32x4 *>(src);
    }
    if (p.epi)
        sum = epilogue4<OUT>(p, m, n, sum, valid);
    store4<OUT>(p.C, (int64_t)m * p.ldc + n, sum, p.vec_store != 0, valid);
}

}  // namespace gnt
