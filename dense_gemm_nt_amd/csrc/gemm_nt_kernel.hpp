// gemm_nt_kernel.hpp -- the gfx950 (CDNA4) NT GEMM kernel.
//
// C[M,N] = A[M,K] . B[N,K]^T, 16-bit inputs, FP32 accumulation, 16- or 32-bit
// output.  The tiled form is the one of "Matmul on sm_120", The tiled view: each
// workgroup owns one BM x BN tile of C and streams BK-deep slabs of A and B
// along K.  What follows restates, for CDNA4, the pieces the pages build on
// Blackwell:
//
//  * Operand staging ("A Blackwell GEMM by Hand in CuTe DSL", sections 3 and 7:
//    a ring of shared-memory stages filled ahead of the MMAs).  Here the ring
//    lives in LDS and is filled by buffer loads that write LDS directly (no VGPR
//    round trip).  A wave-wide load writes 1 KB of LDS lane-contiguously, so the
//    XOR swizzle is applied on the global side: the lane whose LDS slot is
//    physical chunk p of row r fetches logical chunk p ^ key(r).
//  * Swizzle (same page, section 6: a 128-byte XOR swizzle spreads one logical
//    column of 8 rows over 8 bank groups).  key(r) also differs between rows r
//    and r+8, so a 16-lane group of 16 consecutive rows is spread as well.
//  * Stage hand-off (same page, sections 2-3: full/empty barriers with phases).
//    Each wave counts its own outstanding LDS-bound loads with vmcnt; one
//    workgroup barrier per k-slab both publishes the slab just landed and frees
//    the slab everybody has finished reading, which the next loads overwrite.
//  * Matrix instruction (the pages' tcgen05 / mma.sync).  v_mfma_f32_32x32x16
//    (bf16 or f16) takes both operands from VGPRs: lane l supplies row l % 32
//    and 8 consecutive k of one operand.  The B tile is the first operand and
//    the A tile the second, so accumulator register 4q + i of lane l holds
//    C[m = l % 32][n = 8q + 4 (l / 32) + i]: four consecutive columns of one row
//    per group, which the epilogue writes as one vector.
//  * Tile order ("Matmul on sm_120", kernel 1: block swizzle; "A Blackwell GEMM
//    by Hand", section 8: grouped order).  Workgroups are dispatched to the 8
//    XCDs round robin; the block id is first remapped so each XCD receives a
//    contiguous run of virtual ids, then virtual ids walk tiles in groups of
//    GROUP_M tile rows, so an XCD's resident tiles share A rows and B rows in
//    its own L2.
//  * Split-K (same page, section 9; "CUTLASS Deep Dive", the stream-K
//    scheduler).  With splits > 1 each workgroup reduces a contiguous range of
//    k-slabs; every split writes its FP32 partial tile, and the last one to
//    arrive at the tile's counter adds all partials in split order (so the
//    result does not depend on arrival order), writes C and re-arms the
//    counter.  No floating-point atomics.
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

enum : int { IN_BF16 = 0, IN_FP16 = 1 };
enum : int { OUT_BF16 = 0, OUT_FP16 = 1, OUT_FP32 = 2 };

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
    float *partials;       // split-K partial tiles
    unsigned *counters;    // split-K arrival counters, one per tile, zero between calls
};

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

// Swizzle key of LDS row r for a row of CH 16-byte chunks.  Depends only on
// r mod 16, so every 32-row MFMA operand block sees the same pattern.
template <int CH>
__device__ __forceinline__ int row_key(int r)
{
    if constexpr (CH == 8)
        return (r & 7) ^ ((r >> 3) & 1);
    else
        return ((r >> 1) ^ (r >> 3)) & 3;
}

// Block id -> (tile row, tile column, K split).  See the header comment.
__device__ __forceinline__ void map_block(int bid, int G, int tiles_m, int tiles_n, int group_m,
                                          int &tm, int &tn, int &split)
{
    const int x = bid & 7, slot = bid >> 3;
    const int q = G >> 3, r = G & 7;
    const int v = x * q + (x < r ? x : r) + slot;
    const int tiles = tiles_m * tiles_n;
    split = v / tiles;
    const int t = v - split * tiles;
    const int per_group = group_m * tiles_n;
    const int g = t / per_group;
    const int first_m = g * group_m;
    const int gsz = (tiles_m - first_m) < group_m ? (tiles_m - first_m) : group_m;
    const int w = t - g * per_group;
    tm = first_m + w % gsz;
    tn = w / gsz;
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

template <int BM, int BN, int BK, int WM, int WN, int STAGES, int IN, int OUT, bool KMASK>
__global__ __launch_bounds__(WM *WN * 64, 1) void gemm_nt_kernel(KernelArgs p)
{
    constexpr int NWAVES = WM * WN;
    constexpr int NT = NWAVES * 64;
    constexpr int PITCH = BK * 2;          // bytes per LDS row (K-major)
    constexpr int CH = BK / 8;             // 16-byte chunks per row
    constexpr int RPI = 64 / CH;           // rows written by one wave-wide load (1 KB)
    constexpr int A_BYTES = BM * PITCH;    // one stage of A
    constexpr int B_BYTES = BN * PITCH;
    constexpr int A_LOADS = BM / RPI / NWAVES;
    constexpr int B_LOADS = BN / RPI / NWAVES;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int KSTEPS = BK / 16;
    static_assert(CH == 8 || CH == 4, "BK must be 32 or 64");
    static_assert(A_LOADS * RPI * NWAVES == BM && B_LOADS * RPI * NWAVES == BN, "tile/load mismatch");
    static_assert(FM >= 1 && FN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "wave tile");

    __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES * (A_BYTES + B_BYTES)];
    __shared__ int s_last;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wave_m = wave / WN, wave_n = wave % WN;

    int tm, tn, split;
    map_block(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn, split);
    const int tile = tm * p.tiles_n + tn;
    const int m0 = tm * BM, n0 = tn * BN;
    const int kt_begin = split * p.kt_per_split;
    const int kt_end = min(p.k_tiles, kt_begin + p.kt_per_split);

    const int rows_a = min(BM, p.M - m0);
    const int rows_b = min(BN, p.N - n0);
    const __amdgpu_buffer_rsrc_t rsA =
        make_rsrc(p.A + (int64_t)m0 * p.lda, (uint32_t)rows_a * (uint32_t)p.lda * 2u);
    const __amdgpu_buffer_rsrc_t rsB =
        make_rsrc(p.B + (int64_t)n0 * p.ldb, (uint32_t)rows_b * (uint32_t)p.ldb * 2u);

    // Global byte offsets (within the tile's rows) of the chunks this lane loads.
    uint32_t voffA[A_LOADS], voffB[B_LOADS];
    int kcA[A_LOADS], kcB[B_LOADS];
#pragma unroll
    for (int j = 0; j < A_LOADS; ++j) {
        const int row = (j * NWAVES + wave) * RPI + lane / CH;
        const int c = (lane % CH) ^ row_key<CH>(row);
        const int rr = min(row, rows_a - 1);
        voffA[j] = (uint32_t)rr * (uint32_t)p.lda * 2u + (uint32_t)c * 16u;
        kcA[j] = c * 8;
    }
#pragma unroll
    for (int j = 0; j < B_LOADS; ++j) {
        const int row = (j * NWAVES + wave) * RPI + lane / CH;
        const int c = (lane % CH) ^ row_key<CH>(row);
        const int rr = min(row, rows_b - 1);
        voffB[j] = (uint32_t)rr * (uint32_t)p.ldb * 2u + (uint32_t)c * 16u;
        kcB[j] = c * 8;
    }

    const uint32_t lds_base = (uint32_t)(uintptr_t)smem;
    const uint32_t ldsA = lds_base;
    const uint32_t ldsB = lds_base + STAGES * A_BYTES;

    auto issue = [&](int kt, int s) {
        const uint32_t soff = (uint32_t)kt * (uint32_t)(BK * 2);
        const bool full = (kt + 1) * BK <= p.K;
        const int krem = p.K - kt * BK;
#pragma unroll
        for (int j = 0; j < A_LOADS; ++j) {
            const uint32_t v = (full || kcA[j] < krem) ? voffA[j] : kOutOfRange;
            load_lds16(rsA, v, soff, ldsA + s * A_BYTES + (j * NWAVES + wave) * 1024);
        }
#pragma unroll
        for (int j = 0; j < B_LOADS; ++j) {
            const uint32_t v = (full || kcB[j] < krem) ? voffB[j] : kOutOfRange;
            load_lds16(rsB, v, soff, ldsB + s * B_BYTES + (j * NWAVES + wave) * 1024);
        }
    };

    // Per-lane LDS read offsets of the MFMA operand chunk for each k16 step.
    int roff[KSTEPS];
    {
        const int r = lane & 31, h = lane >> 5;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks)
            roff[ks] = r * PITCH + (((2 * ks + h) ^ row_key<CH>(r)) * 16);
    }

    f32x16 acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[i][j][e] = 0.0f;

    // One BK slab from LDS: KSTEPS k16 steps of FN x FM MFMAs.  The operand
    // chunks of step ks+1 are read while the MFMAs of step ks run.
    auto compute_slab = [&](const uint8_t *sa, const uint8_t *sb, int kvalid) {
        u32x4 af[2][FM], bf[2][FN];
        auto fetch = [&](int ks, int slot) {
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
                af[slot][fm] = *reinterpret_cast<const u32x4 *>(sa + fm * 32 * PITCH + roff[ks]);
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                bf[slot][fn] = *reinterpret_cast<const u32x4 *>(sb + fn * 32 * PITCH + roff[ks]);
        };
        fetch(0, 0);
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            const int cur = ks & 1;
            if (ks + 1 < KSTEPS)
                fetch(ks + 1, cur ^ 1);
            if constexpr (KMASK) {
                const int nvalid = kvalid - (2 * ks + (lane >> 5)) * 8;
#pragma unroll
                for (int fm = 0; fm < FM; ++fm)
                    af[cur][fm] = mask_chunk(af[cur][fm], nvalid);
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
                    bf[cur][fn] = mask_chunk(bf[cur][fn], nvalid);
            }
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int fm = 0; fm < FM; ++fm)
                    acc[fn][fm] = mfma32x32x16<IN>(bf[cur][fn], af[cur][fm], acc[fn][fm]);
        }
    };

    const int nkt = kt_end - kt_begin;
    if (nkt > 0) {
        // Prologue: fill STAGES-1 slabs.
#pragma unroll
        for (int s = 0; s < STAGES - 1; ++s)
            if (s < nkt)
                issue(kt_begin + s, s);

        for (int i = 0; i < nkt; ++i) {
            const int s = i % STAGES;
            // Slab i landed for this wave once at most (STAGES-2) newer slabs are in flight.
            if (i + STAGES - 2 < nkt) {
                if constexpr (STAGES == 2)
                    wait_vmcnt<0>();
                else if constexpr (STAGES == 3)
                    wait_vmcnt<(A_LOADS + B_LOADS)>();
                else
                    wait_vmcnt<2 * (A_LOADS + B_LOADS)>();
            } else {
                wait_vmcnt<0>();
            }
            wait_lgkmcnt0();
            wg_barrier();
            if (i + STAGES - 1 < nkt)
                issue(kt_begin + i + STAGES - 1, (i + STAGES - 1) % STAGES);

            const uint8_t *sa = smem + s * A_BYTES + wave_m * WTM * PITCH;
            const uint8_t *sb = smem + STAGES * A_BYTES + s * B_BYTES + wave_n * WTN * PITCH;
            const int kt = kt_begin + i;
            // When K is not a multiple of 8 the slab holding column K-1 also holds
            // columns past K in its last chunk (the row's padding); KMASK builds
            // zero those in registers.  Without it K % 8 == 0 is required.
            compute_slab(sa, sb, p.K - kt * BK);
        }
    }

    if (p.splits > 1) {
        // Publish this split's partial tile, then let the last arrival reduce.
        constexpr int NV = FN * FM * 4;
        float *const base = p.partials + (int64_t)tile * p.splits * (BM * BN);
        float *const mine = base + (int64_t)split * (BM * BN);
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int v = (fn * FM + fm) * 4 + q;
                    f32x4 x = {acc[fn][fm][4 * q], acc[fn][fm][4 * q + 1], acc[fn][fm][4 * q + 2],
                               acc[fn][fm][4 * q + 3]};
                    *reinterpret_cast<f32x4 *>(mine + ((int64_t)v * NT + tid) * 4) = x;
                }
        __threadfence();
        __syncthreads();
        if (tid == 0) {
            const unsigned old = atomicAdd(p.counters + tile, 1u);
            s_last = (old == (unsigned)(p.splits - 1));
        }
        __syncthreads();
        if (!s_last)
            return;
        __threadfence();
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int v = (fn * FM + fm) * 4 + q;
                    f32x4 own = {acc[fn][fm][4 * q], acc[fn][fm][4 * q + 1], acc[fn][fm][4 * q + 2],
                                 acc[fn][fm][4 * q + 3]};
                    f32x4 sum = {0.0f, 0.0f, 0.0f, 0.0f};
                    for (int s2 = 0; s2 < p.splits; ++s2) {
                        f32x4 x = own;
                        if (s2 != split)
                            x = *reinterpret_cast<const f32x4 *>(base + (int64_t)s2 * (BM * BN) +
                                                                 ((int64_t)v * NT + tid) * 4);
                        sum += x;
                    }
                    acc[fn][fm][4 * q] = sum[0];
                    acc[fn][fm][4 * q + 1] = sum[1];
                    acc[fn][fm][4 * q + 2] = sum[2];
                    acc[fn][fm][4 * q + 3] = sum[3];
                }
        if (tid == 0)
            p.counters[tile] = 0u;
    }

    // Epilogue: convert and store.  Lane holds C[m][n .. n+3] per 4-register group.
    const bool vec = p.vec_store != 0;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
        const int m = m0 + wave_m * WTM + fm * 32 + (lane & 31);
        if (m >= p.M)
            continue;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = n0 + wave_n * WTN + fn * 32 + 8 * q + 4 * (lane >> 5);
                const int valid = p.N - n;
                if (valid <= 0)
                    continue;
                f32x4 x = {acc[fn][fm][4 * q], acc[fn][fm][4 * q + 1], acc[fn][fm][4 * q + 2],
                           acc[fn][fm][4 * q + 3]};
                store4<OUT>(p.C, (int64_t)m * p.ldc + n, x, vec, valid);
            }
        }
    }
}

}  // namespace gnt
