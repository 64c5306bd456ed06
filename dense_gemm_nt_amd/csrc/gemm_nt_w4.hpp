// gemm_nt_w4.hpp -- four-wave 256 x BN NT GEMM tile for gfx950 (BN = 128):
// one wave per SIMD, each wave owning a 128 x (BN / 2) block of C whose FP32
// accumulators sit in the accumulation registers, over an LDS ring of three
// 32 KB A units and four 16 KB B units.
//
// Why this shape.  Decode batches (M = 256) have few tiles along N, and the
// 256 x 256 ping-pong tile needs many K splits to occupy the machine, each
// split writing an FP32 copy of its tile.  A 256 x 128 tile gives twice the
// tiles, so half the splits for the same occupancy ("A Blackwell GEMM by Hand
// in CuTe DSL", section 9: decode, split-K).  A wave's block needs (FM * FN)
// x 16 FP32 accumulators per lane; with one wave per SIMD there are 512
// registers per lane for them, and the wave itself overlaps everything: its
// MFMAs run while it issues the fragment reads of the next k-step and the
// direct-to-LDS loads of later slabs (section 3: the copies of later stages
// overlap the MMAs of the current one; "Matmul on sm_120", kernel 3: the
// shared-memory and register pipelines nested).
//
// Ring.  A slab is 64 deep: 256 rows of 128 bytes of A (one 32 KB unit) and
// BN rows of B (one 16 KB unit).  Every load instruction fetches whole
// 128-byte rows (8 rows per 1 KB wave-wide load), so each request is one
// cache line.  A(i) lives in A unit i mod 3, B(i) in B unit i mod 4 (96 + 64
// KB).  The barrier of slab i frees both of its units; A(i + 3) and B(i + 4)
// go into them.  Both operands are issued about two slabs before the barrier
// that needs them: B, which a decode-shaped call streams from HBM, and A,
// which it re-reads from L2 for every tile at twice B's bytes (section 7:
// enough stages in flight for the load latency; two A units, one slab ahead,
// measured 3-5% slower on the decode shapes).  Logical 16-byte chunk c of row
// r sits at physical chunk c ^ key(r) (section 6: the XOR swizzle; row_key),
// and the direct-to-LDS load, which writes 1 KB lane-contiguously, applies it
// on the global side: the lane that fills physical chunk p of row r fetches
// logical chunk p ^ key(r).
//
// Hand-off (sections 2-3: full/empty barriers).  One workgroup barrier per
// slab, before the last MFMAs of its third k-step: every wave then holds the
// slab's last fragments in registers (the slab's units may be refilled) and
// has seen its own loads of the next slab land (vmcnt); after it, the next
// slab's first fragments are read under the last k-step's MFMAs.  The loads
// of a slab are spread over its k-steps, beside the MFMAs.
//
// Output: wave w owns rows [128 (w / 2), +128) and columns [(BN / 2) (w % 2),
// +BN / 2) as 4 x (BN / 64) blocks of 32 x 32.  The B fragment is the MFMA's
// first operand, so accumulator register 4q + e of lane l in block (fn, fm)
// holds C[32 fm + l % 32][32 fn + 8 q + 4 (l / 32) + e].  Requires K % 8 == 0.
#pragma once

#include <type_traits>

#include "gemm_nt_common.hpp"

namespace gnt {

// One wave's 128 x (32 FN) block of C stored through its own 32 KB of LDS so
// that each store instruction writes whole row segments ("Optimizing GEMMs
// using tcgen05 - Part 1": the staged store that replaced scattered stores).
// Rows are staged as T values, as many per pass as 32 KB holds; the 16-byte
// chunk c of staged row r sits at chunk c ^ key(r), so that the column-wise
// writes of the accumulator layout spread over the banks.  The read-back gives
// each lane a 16-byte piece of a row.  NT stores with the non-temporal
// policy.  `dst` is the block's first element, in rows of `ld` elements.
template <int CPR>
__device__ __forceinline__ int stage_key(int r)
{
    if constexpr (CPR >= 16)
        return r & 15;
    else
        return row_key<8>(r);
}

template <typename T, int FN, bool NT = false>
__device__ __forceinline__ void store_wave_block_staged(const f32x16 (&acc)[FN][4], uint8_t *stage, T *dst,
                                                        int64_t ld, int lane)
{
    constexpr int ES = sizeof(T);
    constexpr int ROWB = 32 * FN * ES;       // staged row bytes
    constexpr int CPR = ROWB / 16;           // 16-byte chunks per row
    constexpr int ROWS = 32768 / ROWB < 128 ? 32768 / ROWB : 128;   // rows per pass
    constexpr int PASSES = 128 / ROWS;
    static_assert(CPR >= 8, "row of at least 128 bytes");
    const int h = lane >> 5, r0 = lane & 31;
#pragma unroll
    for (int pass = 0; pass < PASSES; ++pass) {
#pragma unroll
        for (int fmp = 0; fmp < ROWS / 32; ++fmp) {
            const int fm = pass * (ROWS / 32) + fmp;
            const int r = fmp * 32 + r0;
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int byte = (fn * 32 + 8 * q + 4 * h) * ES;
                    const int c = (byte >> 4) ^ stage_key<CPR>(r);
                    uint8_t *a = stage + r * ROWB + c * 16 + (byte & 15);
                    if constexpr (ES == 4) {
                        const f32x4 v = {acc[fn][fm][4 * q], acc[fn][fm][4 * q + 1], acc[fn][fm][4 * q + 2],
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
                        const u32x2 w = {(uint32_t)e[0] | ((uint32_t)e[1] << 16),
                                         (uint32_t)e[2] | ((uint32_t)e[3] << 16)};
                        *reinterpret_cast<u32x2 *>(a) = w;
                    }
                }
        }
        wait_lgkmcnt0();
        constexpr int RPR = 64 / CPR;        // rows per read instruction
#pragma unroll
        for (int j = 0; j < ROWS / RPR; ++j) {
            const int r = j * RPR + lane / CPR;
            const int c = lane % CPR;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(stage + r * ROWB + ((c ^ stage_key<CPR>(r)) * 16));
            T *g = dst + (int64_t)(pass * ROWS + r) * ld + c * (16 / ES);
            if constexpr (NT)
                __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(g));
            else
                *reinterpret_cast<u32x4 *>(g) = v;
        }
        wait_lgkmcnt0();
    }
}

// Every other store of a wave's 128 x (32 FN) block: ragged edges, the fused
// epilogue, split-K partials.  The FP32 accumulators go through the wave's 32 KB
// of LDS (128 FN-byte rows, as many per pass as fit; chunk c of row r at
// c ^ (r mod 16)); read back, each lane holds four consecutive columns of one
// row, to which the epilogue is applied (the bias and prior-C reads are then
// row-contiguous) before a predicated store.  Rows at or past M and columns at
// or past N are not stored.  The block's first element is C[r0][c0].
template <int OUT, int FN>
__device__ __forceinline__ void store_wave_block_any(const KernelArgs &p, const f32x16 (&acc)[FN][4],
                                                     uint8_t *stage, int r0, int c0, int split, int lane)
{
    constexpr int ROWB = 128 * FN;           // FP32 row bytes
    constexpr int CPR = ROWB / 16;
    constexpr int ROWS = 32768 / ROWB < 128 ? 32768 / ROWB : 128;
    constexpr int PASSES = 128 / ROWS;
    constexpr int RPR = 64 / CPR;
    const int h = lane >> 5, rl = lane & 31;
#pragma unroll
    for (int pass = 0; pass < PASSES; ++pass) {
#pragma unroll
        for (int fmp = 0; fmp < ROWS / 32; ++fmp) {
            const int fm = pass * (ROWS / 32) + fmp;
            const int r = fmp * 32 + rl;
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int c = (fn * 8 + 2 * q + h) ^ (r & 15);
                    const f32x4 v = {acc[fn][fm][4 * q], acc[fn][fm][4 * q + 1], acc[fn][fm][4 * q + 2],
                                     acc[fn][fm][4 * q + 3]};
                    *reinterpret_cast<f32x4 *>(stage + r * ROWB + c * 16) = v;
                }
        }
        wait_lgkmcnt0();
#pragma unroll 2
        for (int it = 0; it < ROWS / RPR; ++it) {
            const int r = RPR * it + lane / CPR, c = lane % CPR;
            const int m = r0 + ROWS * pass + r, n = c0 + 4 * c;
            if (m < p.M && n < p.N) {
                f32x4 x = *reinterpret_cast<const f32x4 *>(stage + r * ROWB + ((c ^ (r & 15)) * 16));
                store_result<OUT>(p, split, m, n, x);
            }
        }
        wait_lgkmcnt0();
    }
}

template <int IN, int OUT, int BN>
__global__ __launch_bounds__(256, 1) void gemm_nt_w4(KernelArgs p)
{
    constexpr int BM = 256, BK = 64;
    constexpr int PITCH = 128;                // bytes per LDS row (64 16-bit values)
    constexpr int CH = 8;                     // 16-byte chunks per row
    constexpr int UA = BM * PITCH;            // A of one slab, 32 KB
    constexpr int UBB = BN * PITCH;           // B of one slab, 16 KB
    constexpr int NUA = 3;                    // A units
    constexpr int NUB = (160 * 1024 - NUA * UA) / UBB;   // B units: 4
    constexpr int FM = 4, FN = BN / 64;       // wave block 128 x (BN / 2)
    constexpr int LA = BM / 32, LB = BN / 32; // loads per wave and slab
    constexpr int MF = FN * FM;               // MFMAs per k-step
    constexpr int NR = FM + FN;               // fragment reads per k-step
    static_assert(BN == 128, "the 256 x 128 tile is the instantiated and tested one");
    static_assert(NUA == 3 && NUB == 4, "the load schedule below is written for 3 A and 4 B units");
    static_assert(NUA * UA + NUB * UBB <= 160 * 1024, "LDS budget");

    __shared__ __attribute__((aligned(1024))) uint8_t smem[NUA * UA + NUB * UBB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;

    int tm, tn, split;
    if (p.inreduce)
        map_block_split_minor(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, p.splits, tm, tn, split);
    else
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

    // Load j of wave w for one operand covers tile rows 32 j + 8 w + lane / 8:
    // lane l fills physical chunk l % 8 of its row, which holds logical chunk
    // (l % 8) ^ key(row).  The row step 32 keeps the row mod 16, hence the key,
    // the same for every load of the wave.
    const int lr = lane >> 3;
    const int lc = (lane & 7) ^ row_key<CH>(8 * wave + lr);
    const uint32_t lda2 = (uint32_t)p.lda * 2u, ldb2 = (uint32_t)p.ldb * 2u;
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

    // Load j of operand `op` (0: A into A unit u, 1: B into B unit u) of local
    // slab i.  No load is out of range in all its lanes: a load that touches
    // no memory may count as done before the loads issued ahead of it, which
    // would let a vmcnt wait pass too early.  So rows past the tile's valid
    // rows re-read its last valid row (their outputs are never stored), and a
    // slab at or past nk re-reads the split's last slab: the main loop issues
    // the loads of later slabs on every step, and past the last slab they fill
    // a unit no later slab reads, which keeps every wait count of the loop the
    // same.  Only the chunks at or past K of a row read zeros.
    auto issue_one = [&](int op, int i, int u, int j, auto nt) {
        const int kt = kt0 + (i < nk ? i : nk - 1);
        const bool kin = lc * 8 < p.K - kt * BK;
        const uint32_t kb = (uint32_t)kt * (uint32_t)(BK * 2);
        const int row = 32 * j + 8 * wave + lr;
        if (op == 0) {
            const uint32_t v = kin ? (uint32_t)min(row, rows_a - 1) * lda2 + (uint32_t)lc * 16u : kOutOfRange;
            load_lds16(rsA, v, kb, lds0 + (uint32_t)(u * UA + (row - lr) * PITCH));
        } else {
            const uint32_t v = kin ? (uint32_t)min(row, rows_b - 1) * ldb2 + (uint32_t)lc * 16u : kOutOfRange;
            load_lds16_policy<decltype(nt)::value>(rsB, v, kb, lds0 + (uint32_t)(NUA * UA + u * UBB + (row - lr) * PITCH));
        }
    };

    // Fragment read ks (0..3) of a slab: lane l reads row l % 32 of each 32-row
    // block, k 16 ks + 8 (l / 32) .. +8, i.e. logical chunk 2 ks + l / 32.
    const int fr = lane & 31;
    const int roff0 = fr * PITCH + ((lane >> 5) ^ row_key<CH>(fr)) * 16;
    u32x4 fa[2][FM], fb[2][FN];

    f32x16 acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[i][j][e] = 0.0f;

    // Fragment read n (0..NR-1) of k-step ks from A unit ua and B unit ub into
    // buffer `buf`, in the order the MFMAs below consume them: B block 0, A
    // blocks 0..3, then the other B blocks.
    auto read_one = [&](int ua, int ub, int ks, int buf, int n) {
        const int off = roff0 ^ (32 * ks);
        if (n >= 1 && n <= FM)
            fa[buf][n - 1] =
                *reinterpret_cast<const u32x4 *>(smem + ua * UA + off + (wm * 128 + (n - 1) * 32) * PITCH);
        else {
            const int f = n == 0 ? 0 : n - FM;
            fb[buf][f] = *reinterpret_cast<const u32x4 *>(smem + NUA * UA + ub * UBB + off +
                                                          (wn * (BN / 2) + f * 32) * PITCH);
        }
    };
    // MFMA t (0..MF-1) of a k-step on buffer `buf`: B block t / 4 against A block t % 4.
    auto mfma_one = [&](int buf, int t) {
        acc[t >> 2][t & 3] = mfma32x32x16<IN>(fb[buf][t >> 2], fa[buf][t & 3], acc[t >> 2][t & 3]);
    };

    // The main loop for one B load policy (a compile-time flag: the policy is
    // an immediate of the load instruction).  Its body has no branch, so the
    // compiler keeps every accumulator in place across it, and its order is
    // fixed by scheduling barriers: within each k-step the fragment reads of
    // the next k-step go out beside the first MFMAs and the k-step's loads
    // beside the following ones; the slab's barrier comes before the last two
    // MFMAs of k-step 2, which keep the matrix core busy while the waves meet.
    //
    // Loads: A(i) lives in A unit i mod 3, B(i) in B unit i mod 4; the
    // barrier of slab i frees both units of slab i.  A(i + 2) goes into the A
    // unit A(i - 1) left (first half after the barrier of slab i - 1, second
    // half in k-step 0 of slab i), B(i + 3) into the B unit B(i - 1) left
    // (k-steps 1 and 2 of slab i).  So both operands get about two slabs to
    // land: the L2-resident A, which a decode-shaped call re-reads for every
    // tile at twice B's bytes, as well as the streamed B.  In issue order, the
    // loads after the last one of A(i + 1) when the barrier of slab i is
    // reached are B(i + 2), A(i + 2) and B(i + 3): a wave has its loads of
    // slab i + 1 landed once at most LA + 2 LB loads are in flight.
    auto main_loop = [&](auto nt) {
        // Prologue, in the order the loop would have issued it: A(0) first
        // half, B(0), A(0) second half, B(1), A(1), B(2), A(2) first half;
        // then slab 0 landed.
#pragma unroll
        for (int j = 0; j < LA / 2; ++j)
            issue_one(0, 0, 0, j, nt);
#pragma unroll
        for (int j = 0; j < LB; ++j)
            issue_one(1, 0, 0, j, nt);
#pragma unroll
        for (int j = LA / 2; j < LA; ++j)
            issue_one(0, 0, 0, j, nt);
#pragma unroll
        for (int j = 0; j < LB; ++j)
            issue_one(1, 1, 1, j, nt);
#pragma unroll
        for (int j = 0; j < LA; ++j)
            issue_one(0, 1, 1, j, nt);
#pragma unroll
        for (int j = 0; j < LB; ++j)
            issue_one(1, 2, 2, j, nt);
#pragma unroll
        for (int j = 0; j < LA / 2; ++j)
            issue_one(0, 2, 2, j, nt);
        wait_vmcnt<2 * LB + 3 * LA / 2>();
        wg_barrier();
#pragma unroll
        for (int n = 0; n < NR; ++n)
            read_one(0, 0, 0, 0, n);

        // One k-step: MFMAs t0..t1-1 on buffer mbuf, with read t (t < NR) of
        // k-step rks from units (rua, rub) into rbuf and load number k of `load`
        // beside MFMA 1 + k (MF - 3) / nl (k < nl), so that every load of a
        // k-step goes out before its last two MFMAs.
        auto kstep = [&](int mbuf, int rua, int rub, int rks, int rbuf, auto load, int nl, int t0, int t1) {
#pragma unroll
            for (int t = t0; t < t1; ++t) {
                mfma_one(mbuf, t);
                if (t < NR)
                    read_one(rua, rub, rks, rbuf, t);
#pragma unroll
                for (int k = 0; k < nl; ++k)
                    if (t == 1 + k * (MF - 3) / nl)
                        load(k);
                __builtin_amdgcn_sched_barrier(0);
            }
        };

        int ua = 0, ub = 0;                                 // units of slab i
        for (int i = 0; i < nk; ++i) {
            const int ua1 = ua == NUA - 1 ? 0 : ua + 1;     // A(i + 1)
            const int ua2 = ua1 == NUA - 1 ? 0 : ua1 + 1;   // A(i + 2) = A(i - 1)
            const int ub1 = ub == NUB - 1 ? 0 : ub + 1;     // B(i + 1)
            const int ubp = ub == 0 ? NUB - 1 : ub - 1;     // B(i + 3) = B(i - 1)
            // k-step 0: the second half of A(i + 2)
            kstep(0, ua, ub, 1, 1, [&](int k) { issue_one(0, i + 2, ua2, LA / 2 + k, nt); }, LA / 2, 0, MF);
            // k-steps 1, 2: B(i + 3)
            kstep(1, ua, ub, 2, 0, [&](int k) { issue_one(1, i + NUB - 1, ubp, k, nt); }, LB / 2, 0, MF);
            auto load_b2 = [&](int k) { issue_one(1, i + NUB - 1, ubp, LB / 2 + k, nt); };
            kstep(0, ua, ub, 3, 1, load_b2, LB / 2, 0, MF - 2);
            // every wave holds this slab's last fragments and has its own loads
            // of slab i + 1 landed; the barrier publishes both
            wait_lgkmcnt0();
            wait_vmcnt<LA + 2 * LB>();
            wg_barrier();
            __builtin_amdgcn_sched_barrier(0);
            kstep(0, ua, ub, 3, 1, load_b2, LB / 2, MF - 2, MF);
            // k-step 3: the first fragments of slab i + 1, and the first half of
            // A(i + 3) into the unit A(i) has left
            kstep(1, ua1, ub1, 0, 0, [&](int k) { issue_one(0, i + 3, ua, k, nt); }, LA / 2, 0, MF);
            ua = ua1;
            ub = ub1;
        }
    };

    if (nk > 0) {
        if (p.nt_b)
            main_loop(std::true_type{});
        else
            main_loop(std::false_type{});
    }

    if (p.inreduce) {
        // two K splits: the second to arrive holds the sum and stores it as an
        // unsplit tile
        wait_vmcnt<0>();
        if (!splitk2_arrive<4, FN, FM>(p, acc, tm * p.tiles_n + tn, split, wave, lane,
                                       reinterpret_cast<uint32_t *>(smem)))
            return;
        p.splits = 1;
    }
    // Epilogue.  Every wave is past its last fragment read and every load has
    // landed; after the barrier the ring is free for staging (32 KB per wave).
    const bool full = m0 + BM <= p.M && n0 + BN <= p.N;
    const int r0 = m0 + wm * 128, c0 = n0 + wn * (BN / 2);
    uint8_t *stage = smem + wave * 32768;
    wait_vmcnt<0>();
    wg_barrier();
    if (full && p.splits == 1 && p.rows16 && !p.epi) {
        if constexpr (OUT == OUT_BF16)
            store_wave_block_staged<__bf16, FN, true>(
                acc, stage, static_cast<__bf16 *>(p.C) + (int64_t)r0 * p.ldc + c0, p.ldc, lane);
        else if constexpr (OUT == OUT_FP16)
            store_wave_block_staged<_Float16, FN, true>(
                acc, stage, static_cast<_Float16 *>(p.C) + (int64_t)r0 * p.ldc + c0, p.ldc, lane);
        else
            store_wave_block_staged<float, FN, true>(
                acc, stage, static_cast<float *>(p.C) + (int64_t)r0 * p.ldc + c0, p.ldc, lane);
    } else {
        store_wave_block_any<OUT, FN>(p, acc, stage, r0, c0, split, lane);
    }
}

}  // namespace gnt
