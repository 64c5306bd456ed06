// gemm_nt_pingpong.hpp -- 256x256 NT GEMM tile with eight wavefronts that take
// turns on the matrix cores (gfx950).
//
// The pages keep the tensor core busy by giving the loads and the MMAs to
// different warps ("A Blackwell GEMM by Hand in CuTe DSL", section 3: a producer
// warp and an MMA warp handing stages over through full/empty barriers; "Matmul
// on sm_120", kernel 2: a producer warp feeding consumer warps).  On CDNA4 the
// MFMA reads its operands from the issuing wave's own registers, so every wave
// must load its own fragments.  The role split therefore becomes a split in
// time: two wavefronts share each SIMD (8 per workgroup, 4 per group) and the
// two groups alternate between a memory phase (LDS -> register fragment reads,
// and for group 0 the direct-to-LDS loads of the next k-slab) and a compute
// phase (the 32 MFMAs of one k-slab).  While one group's wave on a SIMD reads
// LDS or waits, the other group's wave on the same SIMD keeps the matrix core
// busy.  A workgroup barrier ends every phase.
//
// Phases, for BK-deep k-slab i held in LDS stage i % S (S stages):
//   phase 2i   : group 0 reads slab i and issues the loads of slab i+S-1 into
//                stage (i+S-1) % S; group 1 computes slab i-1
//   phase 2i+1 : group 0 computes slab i, then waits until its loads of slab
//                i+1 have landed; group 1 reads slab i
// Stage (i+S-1) % S last held slab i-1, which group 1 finished reading in phase
// 2i-1, so it is free when group 0 starts the loads in phase 2i.  A slab's
// loads are issued 2(S-1) phases before it is first read: the ring depth is
// what hides the load latency ("A Blackwell GEMM by Hand", section 7: enough
// stages to cover latency / time per k-step), and with 160 KB of LDS the
// 32-deep slab lets five stages fit (four slabs in flight, 128 KB) where the
// 64-deep slab allows two (one slab, 64 KB).
//
// Output: wave w owns rows [128 (q / 2) + 64 (w / 4), +64) and columns
// [128 (q % 2), +128) of the tile, q = w % 4: 2 x 4 blocks of 32 x 32 with
// FP32 accumulators (128 registers).  Requires K % 8 == 0.
#pragma once

#include "gemm_nt_common.hpp"

namespace gnt {

// Wait until at most nslabs * step + extra of this wave's loads are in flight
// (nslabs between 0 and 3, wave-uniform).
template <int step, int extra>
__device__ __forceinline__ void wait_slabs(int nslabs)
{
    if (nslabs >= 3)
        wait_vmcnt<3 * step + extra>();
    else if (nslabs == 2)
        wait_vmcnt<2 * step + extra>();
    else if (nslabs == 1)
        wait_vmcnt<step + extra>();
    else
        wait_vmcnt<extra>();
}

template <int IN, int OUT, int BK, int S, int PF>
__global__ __launch_bounds__(512, 1) void gemm_nt_pingpong(KernelArgs p)
{
    constexpr int BM = 256, BN = 256;
    constexpr int PITCH = BK * 2;           // bytes per LDS row
    constexpr int CH = BK / 8;              // 16-byte chunks per row
    constexpr int RPI = 64 / CH;            // rows written by one 1 KB wave-wide load
    constexpr int A_BYTES = BM * PITCH;     // one stage of A
    constexpr int B_BYTES = BN * PITCH;
    constexpr int LOADS = BM / RPI / 4;     // per operand per loading wave and slab
    constexpr int PER_SLAB = 2 * LOADS;     // loads per loading wave and slab
    constexpr int FM = 2, FN = 4, KSTEPS = BK / 16;
    static_assert(S >= 2 && S <= 4 + 1 && (S - 2) <= 3, "ring depth");
    static_assert(S * (A_BYTES + B_BYTES) + (PF ? 2048 : 0) <= 160 * 1024, "LDS budget");
    static_assert(PF == 0 || BK == 64, "prefetch touches one 128-byte line per row");

    __shared__ __attribute__((aligned(1024))) uint8_t smem[S * (A_BYTES + B_BYTES) + (PF ? 2048 : 0)];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int group = wave >> 2;            // 0: loads + reads first, 1: computes first
    const int q = wave & 3;
    const int wm0 = (q >> 1) * 128 + group * 64;   // wave's first row within the tile
    const int wn0 = (q & 1) * 128;                 // wave's first column within the tile

    int tm, tn, split;
    map_block(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn, split);
    const int m0 = tm * BM, n0 = tn * BN;
    const int kt0 = split * p.kt_per_split;                     // this split's first k-slab
    const int nk = min(p.k_tiles, kt0 + p.kt_per_split) - kt0;  // and its slab count

    const int rows_a = min(BM, p.M - m0);
    const int rows_b = min(BN, p.N - n0);
    const __amdgpu_buffer_rsrc_t rsA =
        make_rsrc(p.A + (int64_t)m0 * p.lda, (uint32_t)rows_a * (uint32_t)p.lda * 2u);
    const __amdgpu_buffer_rsrc_t rsB =
        make_rsrc(p.B + (int64_t)n0 * p.ldb, (uint32_t)rows_b * (uint32_t)p.ldb * 2u);

    // Load slots of the group-0 waves: load j covers LDS rows RPI (4 j + q) .. +RPI.
    // The swizzle key of a row depends on the row mod 16 only, so this lane's
    // logical chunk lc and its byte offset within the first row group are the
    // same for every j; the row step 32 j goes into the scalar offset.  Rows past
    // the tile's last valid row, and chunks at or past K, read as zeros.
    const int lrow0 = q * RPI + lane / CH;
    const int lc = (lane % CH) ^ row_key<CH>(lrow0);
    const uint32_t lda2 = (uint32_t)p.lda * 2u, ldb2 = (uint32_t)p.ldb * 2u;
    const uint32_t voffA = (uint32_t)lrow0 * lda2 + (uint32_t)lc * 16u;
    const uint32_t voffB = (uint32_t)lrow0 * ldb2 + (uint32_t)lc * 16u;
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

    auto issue = [&](int i) {              // local slab i -> stage i % S
        const int s = i % S;
        const int kt = kt0 + i;
        const uint32_t koff = (uint32_t)kt * (uint32_t)(BK * 2);
        const bool kin = lc * 8 < p.K - kt * BK;
#pragma unroll
        for (int j = 0; j < LOADS; ++j) {
            const int rstep = 4 * RPI * j;
            const uint32_t dst = (uint32_t)((j * 4 + q) * 1024);
            const uint32_t va = (kin && lrow0 + rstep < rows_a) ? voffA : kOutOfRange;
            const uint32_t vb = (kin && lrow0 + rstep < rows_b) ? voffB : kOutOfRange;
            load_lds16(rsA, va, koff + (uint32_t)rstep * lda2, lds0 + s * A_BYTES + dst);
            load_lds16(rsB, vb, koff + (uint32_t)rstep * ldb2, lds0 + S * A_BYTES + s * B_BYTES + dst);
        }
    };

    // L2 prefetch of slab kt: lane l of group-1 wave q touches the 128-byte row
    // segment of A row 64 q + l and of B row 64 q + l (one line each), so the
    // four waves cover all 256 + 256 lines of the slab.  The 4-byte results land
    // in a scratch corner of LDS that nothing reads.
    const int prow = q * 64 + lane;
    const uint32_t pvA = prow < rows_a ? (uint32_t)prow * lda2 : kOutOfRange;
    const uint32_t pvB = prow < rows_b ? (uint32_t)prow * ldb2 : kOutOfRange;
    auto prefetch = [&](int i) {
        if constexpr (PF > 0) {
            const int kt = kt0 + i;
            const uint32_t koff = (uint32_t)kt * (uint32_t)(BK * 2);
            const bool kin = kt * BK < p.K && i < nk;
            const uint32_t junk = lds0 + S * (A_BYTES + B_BYTES) + q * 512;
            touch_lds4(rsA, kin ? pvA : kOutOfRange, koff, junk);
            touch_lds4(rsB, kin ? pvB : kOutOfRange, koff, junk + 256);
        }
    };
    // Lane offsets of the MFMA operand chunk of each k16 step within a 32-row block.
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

    u32x4 af[KSTEPS][FM], bf[KSTEPS][FN];

    auto read_slab = [&](int kt) {
        const uint8_t *sa = smem + (kt % S) * A_BYTES + wm0 * PITCH;
        const uint8_t *sb = smem + S * A_BYTES + (kt % S) * B_BYTES + wn0 * PITCH;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
                af[ks][fm] = *reinterpret_cast<const u32x4 *>(sa + fm * 32 * PITCH + roff[ks]);
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                bf[ks][fn] = *reinterpret_cast<const u32x4 *>(sb + fn * 32 * PITCH + roff[ks]);
        }
    };

    auto compute_slab = [&]() {
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int fm = 0; fm < FM; ++fm)
                    acc[fn][fm] = mfma32x32x16<IN>(bf[ks][fn], af[ks][fm], acc[fn][fm]);
    };

    // Phase boundary: nothing moves across it.
    auto phase_end = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        wg_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };

    // Group-0 waves issue, in order, slabs 0 .. S-2 and then, in phase 2i, slab
    // i+S-1.  Loads complete in issue order, so "slab j landed" means "at most
    // the loads issued after slab j are still in flight".  The L2 prefetches
    // (PF slabs ahead of the slab being loaded) are issued by group 1, which
    // never waits on its loads inside the loop, so their latency stays off the
    // critical path.
    if (nk > 0) {
        if (group == 0) {
            for (int i = 0; i < S - 1; ++i)
                if (i < nk)
                    issue(i);
            wait_slabs<PER_SLAB, 0>(min(nk, S - 1) - 1);
        } else {
            for (int d = 0; d < PF; ++d)
                prefetch(S - 1 + d);
        }
        phase_end();                       // slab 0 is in LDS
        if (group == 0) {
            for (int i = 0; i < nk; ++i) {
                if (i + S - 1 < nk)
                    issue(i + S - 1);
                read_slab(i);
                wait_lgkmcnt0();
                phase_end();               // end of phase 2i
                compute_slab();
                __builtin_amdgcn_sched_barrier(0);   // keep the wait behind the MFMAs
                // slab i+1 landed; slabs i+2 .. min(i+S-1, nk-1) may still fly
                wait_slabs<PER_SLAB, 0>(min(i + S - 1, nk - 1) - (i + 1));
                phase_end();               // end of phase 2i+1
            }
        } else {
            for (int i = 0; i < nk; ++i) {
                if (i > 0)
                    compute_slab();        // slab i-1
                phase_end();               // end of phase 2i
                prefetch(i + S - 1 + PF);
                read_slab(i);
                wait_lgkmcnt0();
                phase_end();               // end of phase 2i+1
            }
            compute_slab();                // slab nk-1
            wait_vmcnt<0>();
        }
    }

    // Epilogue.  Whole tiles go through LDS (the ring is free: the last LDS read
    // of the main loop happened before its last barrier) and leave as
    // row-contiguous 16-byte stores; edge tiles store straight from registers.
    const bool full = m0 + BM <= p.M && n0 + BN <= p.N;
    uint8_t *stage = smem + wave * 16384;
    if (full && p.splits > 1 && (p.N & 3) == 0) {
        float *ws = p.partials + (int64_t)split * p.M * p.N;
        store_block_staged<float>(acc, stage, ws + (int64_t)(m0 + wm0) * p.N + (n0 + wn0), p.N, lane);
        return;
    }
    if (full && p.splits == 1 && p.rows16 && p.epi) {
        store_block_staged_epi<OUT>(p, acc, stage, m0 + wm0, n0 + wn0, lane);
        return;
    }
    if (full && p.splits == 1 && p.rows16) {
        if constexpr (OUT == OUT_BF16)
            store_block_staged<__bf16>(acc, stage, static_cast<__bf16 *>(p.C) + (int64_t)(m0 + wm0) * p.ldc + (n0 + wn0), p.ldc, lane);
        else if constexpr (OUT == OUT_FP16)
            store_block_staged<_Float16>(acc, stage, static_cast<_Float16 *>(p.C) + (int64_t)(m0 + wm0) * p.ldc + (n0 + wn0), p.ldc, lane);
        else
            store_block_staged<float>(acc, stage, static_cast<float *>(p.C) + (int64_t)(m0 + wm0) * p.ldc + (n0 + wn0), p.ldc, lane);
        return;
    }
    // lane holds C[m][n .. n+3] for each 4-register group
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
        const int m = m0 + wm0 + fm * 32 + (lane & 31);
        if (m >= p.M)
            continue;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n0 + wn0 + fn * 32 + 8 * g + 4 * (lane >> 5);
                if (n >= p.N)
                    continue;
                f32x4 x = {acc[fn][fm][4 * g], acc[fn][fm][4 * g + 1], acc[fn][fm][4 * g + 2],
                           acc[fn][fm][4 * g + 3]};
                store_result<OUT>(p, split, m, n, x);
            }
        }
    }
}

}  // namespace gnt
