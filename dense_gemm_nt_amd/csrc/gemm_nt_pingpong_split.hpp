// gemm_nt_pingpong_split.hpp -- the eight-wave 256x256x64 ping-pong tile with
// a split LDS ring: the A operand in half-slabs, released one phase earlier.
//
// Same phases as gemm_nt_pingpong.hpp (two wave groups alternating an LDS-read
// phase and an MFMA phase), but the wave layout gives group 0 the tile rows
// 0..127 and group 1 the rows 128..255.  Group 0 therefore reads only the low
// half of A (and all of B) and group 1 only the high half, so a half-slab of A
// is free one phase after it is read, while B stays until both groups have
// read it.  The 160 KB of LDS then hold three B slabs (3 x 32 KB) and four A
// half-slabs (4 x 16 KB), and the loads run further ahead of their use than a
// ring of whole slabs allows ("A Blackwell GEMM by Hand in CuTe DSL", section
// 7: enough stages in flight to cover the load latency):
//
//   phase 2i   : group 0 reads A_lo(i), B(i) and issues A_hi(i+1), B(i+2)
//                group 1 computes slab i-1
//   phase 2i+1 : group 0 computes slab i and issues A_lo(i+2)
//                group 1 reads A_hi(i), B(i)
//
// B(j) is issued 4 phases before its first read, A_lo(j) and A_hi(j) 3 phases
// before theirs (the whole-slab ring of gemm_nt_pingpong.hpp: 2 phases).  Slot
// reuse: B(j) goes to B slot j % 3, whose previous slab j-3 was last read in
// phase 2j-5; the A half issued in phase p goes to A slot p % 4, whose previous
// occupant (issued in phase p-4) was read in phase p-1.  Only group 0 loads;
// it waits, before each barrier, until the half-slabs the next phase reads have
// landed (loads complete in issue order, so that is "at most the loads issued
// after them are still in flight").  Requires K % 8 == 0.
#pragma once

#include "gemm_nt_common.hpp"

namespace gnt {

// s_waitcnt vmcnt(n) for n in {0, 4, ..., 24} (wave-uniform).
__device__ __forceinline__ void wait_vmcnt_4s(int n)
{
    switch (n) {
    case 24: wait_vmcnt<24>(); break;
    case 20: wait_vmcnt<20>(); break;
    case 16: wait_vmcnt<16>(); break;
    case 12: wait_vmcnt<12>(); break;
    case 8: wait_vmcnt<8>(); break;
    case 4: wait_vmcnt<4>(); break;
    default: wait_vmcnt<0>(); break;
    }
}

template <int IN, int OUT>
__global__ __launch_bounds__(512, 1) void gemm_nt_pingpong_split(KernelArgs p)
{
    constexpr int BM = 256, BN = 256, BK = 64;
    constexpr int PITCH = BK * 2;            // 128-byte LDS rows
    constexpr int CH = BK / 8;               // 8 chunks per row
    constexpr int B_SLOT = BN * PITCH;       // 32 KB
    constexpr int A_SLOT = 128 * PITCH;      // 16 KB (half of A)
    constexpr int B_SLOTS = 3, A_SLOTS = 4;
    constexpr int A_BASE = B_SLOTS * B_SLOT; // A ring after the B ring
    constexpr int FM = 2, FN = 4, KSTEPS = BK / 16;
    static_assert(A_BASE + A_SLOTS * A_SLOT <= 160 * 1024, "LDS budget");

    __shared__ __attribute__((aligned(1024))) uint8_t smem[A_BASE + A_SLOTS * A_SLOT];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int group = wave >> 2;
    const int q = wave & 3;
    const int arow = (q >> 1) * 64;          // wave's first row within its A half
    const int wm0 = group * 128 + arow;      // ... within the tile
    const int wn0 = (q & 1) * 128;

    int tm, tn, split;
    map_block(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn, split);
    const int m0 = tm * BM, n0 = tn * BN;
    const int kt0 = split * p.kt_per_split;
    const int nk = min(p.k_tiles, kt0 + p.kt_per_split) - kt0;

    const int rows_a = min(BM, p.M - m0);
    const int rows_b = min(BN, p.N - n0);
    const __amdgpu_buffer_rsrc_t rsA =
        make_rsrc(p.A + (int64_t)m0 * p.lda, (uint32_t)rows_a * (uint32_t)p.lda * 2u);
    const __amdgpu_buffer_rsrc_t rsB =
        make_rsrc(p.B + (int64_t)n0 * p.ldb, (uint32_t)rows_b * (uint32_t)p.ldb * 2u);

    // Group-0 load slots: a 1 KB load covers 8 rows; load j of wave q covers
    // rows 32 j + 8 q .. +8 of its half-slab or slab.  This lane's row offset
    // and swizzled chunk are the same for every j (the key depends on row mod 16).
    const int lrow0 = q * 8 + lane / CH;
    const int lc = (lane % CH) ^ row_key<CH>(lrow0);
    const uint32_t lda2 = (uint32_t)p.lda * 2u, ldb2 = (uint32_t)p.ldb * 2u;
    const uint32_t voffA = (uint32_t)lrow0 * lda2 + (uint32_t)lc * 16u;
    const uint32_t voffB = (uint32_t)lrow0 * ldb2 + (uint32_t)lc * 16u;
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

    // Issue A half h of local slab i into A slot `slot` (4 loads per wave).
    auto issue_a = [&](int i, int h, int slot) {
        const int kt = kt0 + i;
        const uint32_t koff = (uint32_t)kt * (uint32_t)(BK * 2);
        const bool kin = lc * 8 < p.K - kt * BK;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = h * 128 + 32 * j;
            const uint32_t v = (kin && lrow0 + row < rows_a) ? voffA : kOutOfRange;
            load_lds16(rsA, v, koff + (uint32_t)row * lda2,
                       lds0 + A_BASE + slot * A_SLOT + (uint32_t)((j * 4 + q) * 1024));
        }
    };
    // Issue B of local slab i into B slot i % 3 (8 loads per wave).
    auto issue_b = [&](int i) {
        const int kt = kt0 + i;
        const uint32_t koff = (uint32_t)kt * (uint32_t)(BK * 2);
        const bool kin = lc * 8 < p.K - kt * BK;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int row = 32 * j;
            const uint32_t v = (kin && lrow0 + row < rows_b) ? voffB : kOutOfRange;
            load_lds16(rsB, v, koff + (uint32_t)row * ldb2,
                       lds0 + (i % B_SLOTS) * B_SLOT + (uint32_t)((j * 4 + q) * 1024));
        }
    };
    // A half-slab slots: A_lo(j) was issued in phase 2j-3, A_hi(j) in 2j-2.
    auto slot_lo = [](int j) { return (2 * j + 1) & 3; };
    auto slot_hi = [](int j) { return (2 * j + 2) & 3; };

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
    auto read_slab = [&](int i, int aslot) {
        const uint8_t *sa = smem + A_BASE + aslot * A_SLOT + arow * PITCH;
        const uint8_t *sb = smem + (i % B_SLOTS) * B_SLOT + wn0 * PITCH;
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
    auto phase_end = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        wg_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };

    if (nk > 0) {
        if (group == 0) {
            // phases -4 .. -1: B(0); A_lo(0); A_hi(0), B(1); A_lo(1)
            issue_b(0);
            issue_a(0, 0, slot_lo(0));
            issue_a(0, 1, slot_hi(0));
            if (nk > 1) {
                issue_b(1);
                issue_a(1, 0, slot_lo(1));
            }
            wait_vmcnt_4s(nk > 1 ? 16 : 4);    // A_lo(0) and B(0) landed
        }
        phase_end();
        if (group == 0) {
            for (int i = 0; i < nk; ++i) {
                // phase 2i
                if (i + 1 < nk)
                    issue_a(i + 1, 1, slot_hi(i + 1));
                if (i + 2 < nk)
                    issue_b(i + 2);
                read_slab(i, slot_lo(i));
                wait_lgkmcnt0();
                // A_hi(i) landed: after it come B(i+1), A_lo(i+1), A_hi(i+1), B(i+2)
                wait_vmcnt_4s((i + 1 < nk ? 16 : 0) + (i + 2 < nk ? 8 : 0));
                phase_end();
                // phase 2i+1
                if (i + 2 < nk)
                    issue_a(i + 2, 0, slot_lo(i + 2));
                compute_slab();
                __builtin_amdgcn_sched_barrier(0);
                // A_lo(i+1), B(i+1) landed: after A_lo(i+1) come A_hi(i+1), B(i+2), A_lo(i+2)
                wait_vmcnt_4s(i + 1 < nk ? (4 + (i + 2 < nk ? 12 : 0)) : 0);
                phase_end();
            }
        } else {
            for (int i = 0; i < nk; ++i) {
                if (i > 0)
                    compute_slab();            // slab i-1
                phase_end();                   // end of phase 2i
                read_slab(i, slot_hi(i));
                wait_lgkmcnt0();
                phase_end();                   // end of phase 2i+1
            }
            compute_slab();                    // slab nk-1
        }
    }

    // Epilogue (the LDS rings are free after the loop's last barrier).
    const bool full = m0 + BM <= p.M && n0 + BN <= p.N;
    uint8_t *stage = smem + wave * 16384;
    if (full && p.splits > 1 && (p.N & 3) == 0) {
        float *ws = p.partials + (int64_t)split * p.M * p.N;
        store_block_staged<float>(acc, stage, ws + (int64_t)(m0 + wm0) * p.N + (n0 + wn0), p.N, lane);
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
