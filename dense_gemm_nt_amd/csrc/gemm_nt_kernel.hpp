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
//  * Split-K (same page, section 9).  With splits > 1 each workgroup reduces a
//    contiguous range of k-slabs and writes its FP32 partial tile to the
//    workspace; a second kernel adds the partials in split order (a fixed
//    order, so results do not depend on scheduling).  No floating-point
//    atomics, no inter-workgroup waiting.
#pragma once

#include <type_traits>

#include "gemm_nt_common.hpp"

namespace gnt {

// ROT: the tiles walk their k-slabs in the rotated order (SlabOrder).
template <int BM, int BN, int BK, int WM, int WN, int STAGES, int IN, int OUT, bool KMASK, bool ROT>
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

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wave_m = wave / WN, wave_n = wave % WN;

    int tm, tn, split;
    if (p.inreduce)       // the K splits of a tile adjacent in launch order (splitk_arrive)
        map_block_split_minor(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, p.splits, tm, tn, split);
    else
        map_block(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn, split);
    const int tile = tm * p.tiles_n + tn;
    const int m0 = tm * BM, n0 = tn * BN;
    const int kt_begin = split * p.kt_per_split;
    const int kt_end = min(p.k_tiles, kt_begin + p.kt_per_split);
    const SlabOrder<ROT> order = slab_order<ROT>(kt_begin, kt_end - kt_begin, p.k_tiles, p.K % BK != 0, n0);

    const int rows_a = min(BM, p.M - m0);
    const int rows_b = min(BN, p.N - n0);
    const __amdgpu_buffer_rsrc_t rsA =
        make_rsrc(p.A + (int64_t)m0 * p.lda, (uint32_t)rows_a * (uint32_t)p.lda * 2u);
    const __amdgpu_buffer_rsrc_t rsB =
        make_rsrc(p.B + (int64_t)n0 * p.ldb, (uint32_t)rows_b * (uint32_t)p.ldb * 2u);

    // Load j of this wave covers LDS rows (j * NWAVES + wave) * RPI .. +RPI.  A
    // row's swizzle key depends on the row mod 16 only, which is the same for
    // every j, so this lane's logical chunk lc is fixed.  Chunks at or past K
    // read as zeros.  Rows past the tile's last valid row re-read that row
    // (their outputs are never stored) rather than reading out of range: a load
    // that touches no memory in any lane may count as done before the loads
    // issued ahead of it, and the vmcnt waits below count on issue order.
    constexpr int RSTEP = NWAVES * RPI;
    const int lrow0 = wave * RPI + lane / CH;
    const int lc = (lane % CH) ^ row_key<CH>(lrow0);
    const uint32_t lda2 = (uint32_t)p.lda * 2u, ldb2 = (uint32_t)p.ldb * 2u;

    const uint32_t lds_base = (uint32_t)(uintptr_t)smem;
    const uint32_t ldsA = lds_base;
    const uint32_t ldsB = lds_base + STAGES * A_BYTES;

    // Load j (0 .. NL-1: A's loads, then B's) of slab kt into stage s; B's
    // take the non-temporal policy `nt` when B is streamed (the policy is an
    // immediate of the instruction, so the main loop exists once per policy).
    constexpr int NL = A_LOADS + B_LOADS;
    auto issue_one = [&](int kt, int s, int j, auto nt) {
        const uint32_t koff = (uint32_t)kt * (uint32_t)(BK * 2);
        const bool kin = lc * 8 < p.K - kt * BK;
        if (j < A_LOADS) {
            const uint32_t r = (uint32_t)min(lrow0 + j * RSTEP, rows_a - 1);
            const uint32_t v = kin ? r * lda2 + (uint32_t)lc * 16u : kOutOfRange;
            load_lds16(rsA, v, koff, ldsA + s * A_BYTES + (j * NWAVES + wave) * 1024);
        } else {
            const int jb = j - A_LOADS;
            const uint32_t r = (uint32_t)min(lrow0 + jb * RSTEP, rows_b - 1);
            const uint32_t v = kin ? r * ldb2 + (uint32_t)lc * 16u : kOutOfRange;
            load_lds16_policy<decltype(nt)::value>(rsB, v, koff,
                                                   ldsB + s * B_BYTES + (jb * NWAVES + wave) * 1024);
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
    // chunks of step ks+1 are read while the MFMAs of step ks run, and
    // `load(j)` (j = 0 .. NL-1, the loads of a later slab) is called between
    // the MFMAs, spread over the k-steps, so that the loads' issue, which the
    // vector memory unit accepts at about one 1 KB load per 25 cycles, can run
    // beside the matrix cores instead of ahead of them.
    auto compute_slab = [&](const uint8_t *sa, const uint8_t *sb, int kvalid, auto load) {
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
            // this k-step's share of the loads, one after each of its first MFMAs
            constexpr int PER = (NL + KSTEPS - 1) / KSTEPS;
            int t = 0;
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int fm = 0; fm < FM; ++fm) {
                    acc[fn][fm] = mfma32x32x16<IN>(bf[cur][fn], af[cur][fm], acc[fn][fm]);
                    if (t < PER && ks * PER + t < NL)
                        load(ks * PER + t);
                    ++t;
                }
            // (a k-step with fewer MFMAs than its share issues the rest here)
#pragma unroll
            for (; t < PER; ++t)
                if (ks * PER + t < NL)
                    load(ks * PER + t);
        }
    };

    const int nkt = kt_end - kt_begin;
    auto main_loop = [&](auto nt) {
        // Where the next slab's loads go.  With B streamed from HBM (the
        // non-temporal policy: one or two tile rows, small M) or a two-stage
        // ring (one slab in flight): all at once after the slab's barrier,
        // which gives them the whole slab to land.  Otherwise: spread between
        // the MFMAs, where their issue no longer holds the matrix cores back
        // (4-16% on 1024 x 4096 x 2048, 1536^3, 2048^3; 1-4% slower on the
        // streamed small-M shapes).
        constexpr bool EARLY = decltype(nt)::value || STAGES <= 2;
        // Spread loads sit inside the slab's code with no branch around them,
        // so every iteration issues NL loads per wave: slabs past the split's
        // last one re-read that slab into a stage no later slab reads.  The
        // wait then has one count: slab i has landed for this wave once at
        // most the (STAGES - 2) NL loads of the slabs after it are in flight.
        // Issued at once, the loads past the end are skipped instead, and the
        // last iterations wait for everything.
        auto slab_kt = [&](int i) { return order(min(i, nkt - 1)); };
#pragma unroll
        for (int s = 0; s < STAGES - 1; ++s)
            if (!EARLY || s < nkt)
#pragma unroll
                for (int j = 0; j < NL; ++j)
                    issue_one(slab_kt(s), s, j, nt);

        // the k-slab of the loads issued in iteration i, computed one iteration
        // ahead so that the loads after the barrier do not wait for it
        int kt_next = slab_kt(STAGES - 1);
        for (int i = 0; i < nkt; ++i) {
            const int s = i % STAGES;
            static_assert((STAGES - 2) * NL <= 63, "vmcnt range");
            if (EARLY && i + STAGES - 2 >= nkt)
                wait_vmcnt<0>();
            else
                wait_vmcnt<(STAGES - 2) * NL>();
            wait_lgkmcnt0();
            wg_barrier();
            const int s_next = (i + STAGES - 1) % STAGES;
            if constexpr (EARLY) {
                if (i + STAGES - 1 < nkt)
#pragma unroll
                    for (int j = 0; j < NL; ++j)
                        issue_one(kt_next, s_next, j, nt);
            }

            const uint8_t *sa = smem + s * A_BYTES + wave_m * WTM * PITCH;
            const uint8_t *sb = smem + STAGES * A_BYTES + s * B_BYTES + wave_n * WTN * PITCH;
            const int kt = order(i);
            // When K is not a multiple of 8 the slab holding column K-1 also holds
            // columns past K in its last chunk (the row's padding); KMASK builds
            // zero those in registers.  Without it K % 8 == 0 is required.
            compute_slab(sa, sb, p.K - kt * BK, [&](int j) {
                if constexpr (!EARLY)
                    issue_one(kt_next, s_next, j, nt);
            });
            kt_next = slab_kt(i + STAGES);
            pin_scalar(kt_next);
        }
        // the re-read loads of the last iterations may still be in flight
        if constexpr (!EARLY)
            wait_vmcnt<0>();
    };
    if (nkt > 0) {
        if (p.nt_b)
            main_loop(std::true_type{});
        else
            main_loop(std::false_type{});
    }

    // K splits reduced here: the last split of the tile to finish adds the
    // others' partials and stores the tile as an unsplit one (the flag word is
    // in the ring, which no wave reads any more once the partials are stored).
    // Not in the two-stage ring, which runs two blocks per compute unit and
    // has no registers for the reduction's buffers.
    if constexpr (STAGES > 2) {
        if (p.inreduce) {
            if (!splitk_arrive<NWAVES, FN, FM>(p, acc, tile, split, wave, lane,
                                               reinterpret_cast<uint32_t *>(smem)))
                return;
            p.splits = 1;
        }
    }

    // Epilogue without a fused epilogue: each wave's block through its share of
    // the (now idle) LDS ring, stored row-contiguously (C, or this split's
    // FP32 partial).  A block-uniform branch, so the barrier that retires the
    // ring's last fragment reads is reached by every wave.
    constexpr int STAGE_BYTES = 4096 * FM * FN;
    if constexpr (NWAVES * STAGE_BYTES <= STAGES * (A_BYTES + B_BYTES)) {
        if (!p.epi) {
            const int r0 = m0 + wave_m * WTM, c0 = n0 + wave_n * WTN;
            wg_barrier();
            uint8_t *stage = smem + wave * STAGE_BYTES;
            if (p.splits > 1)
                store_block_rows<OUT_FP32>(acc, stage, p.partials + (int64_t)split * p.M * p.N + (int64_t)r0 * p.N + c0,
                                           p.N, p.M - r0, p.N - c0, lane);
            else if constexpr (OUT == OUT_FP32)
                store_block_rows<OUT>(acc, stage, static_cast<float *>(p.C) + (int64_t)r0 * p.ldc + c0, p.ldc,
                                      p.M - r0, p.N - c0, lane);
            else
                store_block_rows<OUT>(acc, stage, static_cast<uint16_t *>(p.C) + (int64_t)r0 * p.ldc + c0, p.ldc,
                                      p.M - r0, p.N - c0, lane);
            return;
        }
    }

    // Epilogue: convert and store.  Lane holds C[m][n .. n+3] per 4-register group.
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
                if (n >= p.N)
                    continue;
                f32x4 x = {acc[fn][fm][4 * q], acc[fn][fm][4 * q + 1], acc[fn][fm][4 * q + 2],
                           acc[fn][fm][4 * q + 3]};
                store_result<OUT>(p, split, m, n, x);
            }
        }
    }
}

}  // namespace gnt
