// gemm_nt_pp2.hpp -- eight-wave 256x256x64 ping-pong tile in which both wave
// groups issue global loads, over an LDS ring of 16 KB units (gfx950).
//
// Two groups of four waves (one wave of each group per SIMD) alternate between
// a memory phase (LDS -> register fragment reads, plus direct-to-LDS global
// loads) and a compute phase (the 32 MFMAs of one 64-deep k-slab), and a
// workgroup barrier ends every phase.  Both groups load.  Issuing the 64
// wave-wide 1 KB loads of a slab takes longer than one compute phase when a
// single group issues all of them: with the LDS also serving the other
// group's fragment reads, a wave-wide 16-byte-per-lane load costs its wave
// 25-40 cycles of issue (its LDS write queues behind the reads), so the
// loading waves stall on issue, not on latency.  Here each group issues half a slab in its own memory phase, while
// the other group keeps the matrix cores busy ("A Blackwell GEMM by Hand in
// CuTe DSL", section 3: the producer's copies overlap the consumer's MMAs;
// section 7: enough stages in flight for the load latency).
//
// Work split.  Group 0 owns tile rows 0..127 and group 1 rows 128..255, so
// the A half of group g (A_g, 128 rows x 64 k = 16 KB) is read by that group
// only, and B (256 rows, two 16 KB halves) by both.  The ring holds nine
// 16 KB units: B in two slots of two units, A_0 in two units and A_1 in three.
//
//   phase 2i   : group 0 issues B(i+1), reads A_0(i) and B(i);
//                group 1 computes slab i-1
//   phase 2i+1 : group 1 issues A_0(i+2) and A_1(i+2), reads A_1(i) and B(i);
//                group 0 computes slab i, then waits for B(i+1)
//
// Slot reuse: B(i+1) takes the slot of B(i-1), last read in phase 2i-1;
// A_0(i+2) the unit of A_0(i), last read in phase 2i; A_1(i+2) the unit of
// A_1(i-1), last read in phase 2i-1.  Group 1 waits, at the end of phase
// 2i+1, until A(i+1) has landed (only A(i+2) may still be in flight); A(i+1)
// is first read in phase 2i+2.  Each group waits only for its own loads
// (vmcnt counts per wave), and the barrier that ends the phase publishes them.
//
// Output: wave w (group g = w / 4, q = w % 4) owns rows [128 g + 64 (q / 2), +64)
// and columns [128 (q % 2), +128): 2 x 4 blocks of 32 x 32 with FP32
// accumulators.  Requires K % 8 == 0.
//
// FP8 inputs ("CUTLASS Deep Dive", "FP8 and Blockwise Scaling").  A slab is
// still 128 bytes of every row, here 128 k-values, so the loads, the ring and
// the swizzle are the 16-bit kernel's; each MFMA (32x32x64) takes a lane's 32
// consecutive k-values from two 16-byte fragment reads.  Per-tensor scales
// multiply the accumulators once before the store.  Blockwise scales (one per
// 128-deep block, per row or 128 rows of A, per 128 columns of B) are applied
// to each slab's partial sum as it is added to the accumulators.  A lane's 16
// accumulators of a 32x32 block share one output row and one B column block,
// so one scale product s_i per slab; the accumulators are kept in units of
// the current slab's s_i (acc_i = (sum over slabs j <= i of s_j P_j) / s_i),
// which lets the MFMAs add the partial sum P_i in place: acc_i = acc_{i-1} *
// (s_{i-1} / s_i) + P_i, and the store multiplies by the last s.  A slab whose
// s is zero adds nothing: its A fragment is zeroed and the units are kept.
// This needs nonzero scales to be normal FP32 numbers and sum_j s_j P_j / s_i
// to stay in FP32 range (scale ratios along one row below about 2^80).  The
// scales of a slab travel with its
// operands: the waves that load A(i) also load its row scales, and wave 0 of
// group 0 loads B(i)'s two column-block scales, by 4-byte direct-to-LDS loads
// into slots that mirror the operand slots, so the operand waits cover them;
// the memory phase that reads a slab's fragments reads its scales too.
#pragma once

#include <type_traits>

#include "gemm_nt_common.hpp"

#ifdef GNT_PP2_TRACE
#include "gemm_nt_trace.hpp"
#else
// instrumentation hooks (phase timestamps, gemm_nt_trace.hpp); empty in the library
#define GNT_PP2_TRACE_LDS 0
#define GNT_PP2_TRACE_DECL
#define GNT_PP2_EVENT(i, e)
#define GNT_PP2_FLUSH(g, i)
#define GNT_PP2_DUMP
#endif

namespace gnt {

// PS: 0 one tile (split) per block; 1 persistent blocks looping over tiles;
// 2 stream-K segments, each stored as an FP32 partial slot (no epilogue).
template <int IN, int OUT, bool AM = false, bool BNM = false, int SC = 0, bool GR = false,
          int PS = 0>
__global__ __launch_bounds__(512, 1) void gemm_nt_pp2(KernelArgs p0)
{
    constexpr bool F8 = IN >= IN_F8;
    constexpr int ESZ = F8 ? 1 : 2;          // bytes per element
    static_assert(!(F8 && (AM || BNM)), "FP8 operands are K-major");
    static_assert(SC == 0 || F8, "blockwise scales are for FP8 inputs");
    constexpr int BM = 256, BN = 256, BK = 128 / ESZ;   // k-values per slab
    constexpr int PITCH = 128;               // 128-byte LDS rows
    constexpr int CH = 8;                    // 16-byte chunks per row
    constexpr int UNIT = 128 * PITCH;        // 16 KB: 128 rows of one slab
    constexpr int U_B = 0;                   // B slot s: units 2s (rows 0..127), 2s+1
    constexpr int U_A0 = 4;                  // A_0 slot s: unit 4 + s, s < 2
    constexpr int U_A1 = 6;                  // A_1 slot s: unit 6 + s, s < 3
    constexpr int UNITS = 9;
    constexpr int FM = 2, FN = 4, KSTEPS = 4;   // 16-byte fragment reads per row
    // blockwise scales: A_0 rows in two 512-byte slots, A_1 rows in three, B's
    // two column blocks in two 256-byte slots
    constexpr int SA0 = UNITS * UNIT, SA1 = SA0 + 2 * 512, SB = SA1 + 3 * 512;
    constexpr int LDS_USED = UNITS * UNIT + (SC ? 2 * 512 + 3 * 512 + 2 * 256 : 0);
    constexpr int LDS_BYTES = LDS_USED + GNT_PP2_TRACE_LDS;
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");

    __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane_id = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int group = wave >> 2;
    const int q = wave & 3;
    const int wm0 = group * 128 + (q >> 1) * 64;   // wave's first row within the tile
    const int wn0 = (q & 1) * 128;                 // and first column

    KernelArgs p = p0;

    constexpr bool streamk = PS == 2;
    // Grouped launches re-read row 0 for A loads wholly past M (see the loader):
    // most of their tiles are partial.  A plain launch has at most one row of
    // partial tiles, which waits for all loads instead, as with blockwise FP8
    // scales, which have no register to spare for the redirect.
    constexpr bool redirect_a = GR && SC != 1;

    // One output tile (split `split` of tile (tm, tn)): prologue, main loop and
    // epilogue.  Run once per block, or in a loop by persistent blocks.  A
    // stream-K segment is k-slabs [sk_kt0, +sk_nk) of the tile, its FP32
    // partial into slot sk_slot of the workspace.
    // (Always inlined: called from two loops it would otherwise become a real
    // call, which passes the captured arguments through memory.)
    auto tile = [&](int tm, int tn, int split_, int sk_kt0 = 0, int sk_nk = 0,
                    int sk_slot = 0) __attribute__((always_inline)) {
        // Persistent blocks: an opaque copy of the lane id, so the per-lane
        // offsets derived from it are recomputed per work unit instead of
        // being held across the epilogue.
        int lane = lane_id;
        if constexpr (PS != 0)
            asm volatile("" : "+v"(lane));
        const int split = split_;
        const int m0 = tm * BM, n0 = tn * BN;
        const int kt0 = streamk ? sk_kt0 : split * p.kt_per_split;
        const int nk = streamk ? sk_nk : min(p.k_tiles, kt0 + p.kt_per_split) - kt0;

        const int rows_a = min(BM, p.M - m0);
        const int rows_b = min(BN, p.N - n0);
        const uint8_t *Ab = reinterpret_cast<const uint8_t *>(p.A);
        const uint8_t *Bb = reinterpret_cast<const uint8_t *>(p.B);
        const __amdgpu_buffer_rsrc_t rsA =
            make_rsrc(Ab + (int64_t)m0 * p.lda * ESZ, (uint32_t)rows_a * (uint32_t)p.lda * ESZ);
        const __amdgpu_buffer_rsrc_t rsB =
            make_rsrc(Bb + (int64_t)n0 * p.ldb * ESZ, (uint32_t)rows_b * (uint32_t)p.ldb * ESZ);

        // Load slots: within a 128-row unit, load j (0..3) of wave q covers rows
        // 32 j + 8 q .. +8 (one 1 KB wave-wide load, 8 rows x 128 bytes).  The
        // swizzle key depends on the row mod 16 only, so this lane's row offset and
        // swizzled chunk are the same for every j and every unit.
        const int lrow0 = q * 8 + lane / CH;
        const int lc = (lane % CH) ^ row_key<CH>(lrow0);
        const uint32_t lda2 = (uint32_t)p.lda * ESZ, ldb2 = (uint32_t)p.ldb * ESZ;   // row pitch, bytes
        const uint32_t voffA = (uint32_t)lrow0 * lda2 + (uint32_t)lc * 16u;
        const uint32_t voff0 = (uint32_t)lc * 16u;      // the same chunk of the tile's row 0
        const uint32_t voffB = (uint32_t)lrow0 * ldb2 + (uint32_t)lc * 16u;
        const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

        // Load number j (0..3) of the 128-row unit starting at tile row `row0` of
        // A (IS_A) or B at local slab i into LDS unit u.
        //
        // An operand stored MN-major (A as [K][lda], element (m, k) at A[k lda + m];
        // B as [K][ldb]) is staged as 64 k-rows of 128 columns per unit (256-byte
        // LDS rows): load j of wave q covers k-rows 16 j + 4 q .. +4, lane l the
        // 16-byte chunk l % 16 of row l / 16, swizzled on the global side to
        // logical chunk (l % 16) ^ 4 (row mod 4).  Its MFMA fragments (8
        // consecutive k of one column) come from two transposing LDS reads.  A
        // per-slab buffer resource ends with k-row K - 1, so k-rows past K read
        // zeros.
        const int mn_chunk = (lane & 15) ^ (4 * (lane >> 4));
        auto load_one = [&](auto is_a, int i, int row0, int u, int j, auto nt) {
            constexpr bool IS_A = decltype(is_a)::value;
            constexpr bool MN = IS_A ? AM : BNM;
            constexpr bool NT = decltype(nt)::value;
            const int kt = kt0 + i;
            const uint32_t dst = lds0 + (uint32_t)(u * UNIT + (j * 4 + q) * 1024);
            if constexpr (MN) {
                const uint16_t *X = IS_A ? p.A : p.B;
                const int ld = IS_A ? p.lda : p.ldb;
                const int col0 = IS_A ? m0 : n0;
                const int rows_left = min(BK, p.K - kt * BK);
                // the slab's k-rows as whole rows of ld elements (the operand
                // occupies K such rows), seen from the tile's first column
                const __amdgpu_buffer_rsrc_t rs =
                    make_rsrc(X + (int64_t)kt * BK * ld + col0,
                              (uint32_t)(((int64_t)rows_left * ld - col0) * 2));
                const uint32_t ld2 = (uint32_t)ld * 2u;
                // chunks wholly past column M (N) re-read the last valid chunk:
                // they only feed output rows (columns) that are never stored
                const int cmax = ((IS_A ? rows_a : rows_b) - 1) & ~7;
                const int col = min(row0 + 8 * mn_chunk, cmax);
                const uint32_t v = (uint32_t)(4 * q + (lane >> 4)) * ld2 + (uint32_t)col * 2u;
                load_lds16_policy<NT>(rs, v, (uint32_t)(16 * j) * ld2, dst);
            } else {
                // Rows past the tile's valid rows read zeros.  In a grouped
                // launch, an A load all of whose eight rows lie past M re-reads
                // the tile's row 0 instead (its LDS rows feed outputs that are
                // never stored): a load out of range in every lane touches no
                // memory and may count as done ahead of the loads issued before
                // it, and group 1's waits count on the order of its A loads.
                // (Its lane with logical chunk 0 is inside K: kt is below
                // k_tiles.)  B's waits are all for every load, so B keeps the
                // zero reads.
                const uint32_t koff = (uint32_t)kt * (uint32_t)(BK * ESZ);
                const bool kin = lc * 16 < (p.K - kt * BK) * ESZ;
                const int row = row0 + 32 * j;
                const int rows = IS_A ? rows_a : rows_b;
                const uint32_t ld2 = IS_A ? lda2 : ldb2;
                const bool some = !IS_A || !redirect_a || row + 8 * q < rows;   // wave-uniform
                const uint32_t v = some ? ((kin && lrow0 + row < rows) ? (IS_A ? voffA : voffB) : kOutOfRange)
                                        : (kin ? voff0 : kOutOfRange);
                load_lds16_policy<NT>(IS_A ? rsA : rsB, v, some ? koff + (uint32_t)row * ld2 : koff, dst);
            }
        };
        // The eight loads a wave issues in one memory phase, n = 0..7: group 0
        // loads both halves of B(i) into B slot i % 2 (GRP = 0), group 1 both
        // halves of A(i) (GRP = 1).
        auto group_load = [&](auto grp, int i, int n, auto nt) {
            const int j = n & 3, half = n >> 2;
            if constexpr (decltype(grp)::value == 0)
                load_one(std::false_type{}, i, half * 128, U_B + 2 * (i & 1) + half, j, nt);
            else
                load_one(std::true_type{}, i, half * 128, half == 0 ? U_A0 + (i & 1) : U_A1 + (i % 3), j,
                         std::false_type{});
        };

        // Blockwise scales of local slab i (SC == 1).  Group 1 wave q loads the
        // row scales of tile rows 64 q .. +64 (rows of A_0 into the A_0 slot of
        // slab i, rows of A_1 into its A_1 slot); wave 0 of group 0 loads the
        // scales of the tile's two 128-column blocks of B.  Rows past M take the
        // last row's scale and blocks past N read zeros (their outputs are never
        // stored; lane 0's block is always inside N).
        auto scale_load = [&](auto grp, int i) {
            if constexpr (SC == 1) {
                const int kt = kt0 + i;
                if constexpr (decltype(grp)::value == 1) {
                    const int m = min(m0 + 64 * q + lane, p.M - 1);
                    const uint32_t v = ((uint32_t)(m >> p.sfa_shift) * (uint32_t)p.sf_ld + (uint32_t)kt) * 4u;
                    const uint32_t dst = q < 2 ? SA0 + (i & 1) * 512 + q * 256
                                               : SA1 + (i % 3) * 512 + (q - 2) * 256;
                    load_lds4(make_rsrc(p.scale_a, p.sfa_bytes), v, 0, lds0 + dst);
                } else if (q == 0) {
                    const bool ok = lane < 2 && n0 + 128 * lane < p.N;
                    const uint32_t v = ok
                        ? ((uint32_t)((n0 >> 7) + lane) * (uint32_t)p.sf_ld + (uint32_t)kt) * 4u
                        : kOutOfRange;
                    load_lds4(make_rsrc(p.scale_b, p.sfb_bytes), v, 0, lds0 + SB + (i & 1) * 256);
                }
            }
        };
        // This lane's scale products for the two 32-row blocks of local slab i
        // (read in the memory phase that reads the slab's fragments), and the
        // units the accumulators of those blocks are held in.
        float sblk[FM] = {1.0f, 1.0f};
        float unit[FM] = {1.0f, 1.0f};
        auto scale_read = [&](auto grp, int i) {
            if constexpr (SC == 1) {
                const float sb = *reinterpret_cast<const float *>(smem + SB + (i & 1) * 256 + (q & 1) * 4);
                const int slot = decltype(grp)::value == 0 ? SA0 + (i & 1) * 512 : SA1 + (i % 3) * 512;
    #pragma unroll
                for (int fm = 0; fm < FM; ++fm) {
                    const int row = (q >> 1) * 64 + fm * 32 + (lane & 31);   // within the group's half
                    sblk[fm] = *reinterpret_cast<const float *>(smem + slot + row * 4) * sb;
                }
            }
        };

        // Byte offset of this lane's fragment read ks within a block's rows.
        // 16-bit: read ks holds k 16 ks + 8 h .. +8 (chunk 2 ks + h); FP8: read ks
        // holds k 64 (ks / 2) + 32 h + 16 (ks % 2) .. +16 (chunk 4 (ks / 2) + 2 h +
        // ks % 2).  The chunk index of read ks is the one of read 0 with bits
        // flipped (the swizzle is an XOR), so one register carries all four.
        const int roff0 = [&] {
            const int r = lane & 31, h = lane >> 5;
            return r * PITCH + (((F8 ? 2 * h : h) ^ row_key<CH>(r)) * 16);
        }();
        auto roff = [&](int ks) -> int {
            const int flip = F8 ? 4 * (ks >> 1) + (ks & 1) : 2 * ks;
            return roff0 ^ (flip * 16);
        };

        f32x16 acc[FN][FM];
    #pragma unroll
        for (int i = 0; i < FN; ++i)
    #pragma unroll
            for (int j = 0; j < FM; ++j)
    #pragma unroll
                for (int e = 0; e < 16; ++e)
                    acc[i][j][e] = 0.0f;

        u32x4 af[KSTEPS][FM], bf[KSTEPS][FN];
        // Transposing fragment read of an MN-major unit at `base`: the 8
        // consecutive k (16 ks .. +8 (lane / 32) .. +8) of column cb + lane % 32.  Each
        // ds_read_b64_tr_b16 gives lane i of a 16-lane group element i % 4 of the
        // 8-byte pieces addressed by lanes i / 4 + 4 e (e = 0..3) of the group, so
        // lane j addresses k-row 8 (j / 32) + 4 r + (j % 16) / 4 and columns
        // 16 ((j / 16) % 2) + 4 (j % 4) .. +4: read r = 0 brings k .. k+3, r = 1
        // k+4 .. k+7.  Rows 4 apart never share banks under the 4 (row mod 4) chunk
        // swizzle, so each read takes the two-cycle minimum for its 512 bytes.
        const int tr_kq = (lane & 15) >> 2;
        const int tr_lp = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
        const int tr_base = (8 * (lane >> 5) + tr_kq) * 256 + 8 * (lane & 1);
        auto read_mn = [&](const uint8_t *base, int ks, int cb) -> u32x4 {
            const int chunk = 4 * ((cb >> 5) ^ tr_kq) + tr_lp;
            typedef short v4s __attribute__((ext_vector_type(4)));
            typedef __attribute__((address_space(3))) v4s lds_v4s;
            const uint8_t *p0 = base + tr_base + (16 * ks) * 256 + chunk * 16;
            const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_v4s *)(uint32_t)(uintptr_t)p0);
            const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_v4s *)(uint32_t)(uintptr_t)(p0 + 4 * 256));
            const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
            return (u32x4){a[0], a[1], b[0], b[1]};
        };
        // Fragment read number r (0..23) of local slab i: ks = r / 6, then the two
        // A blocks and the four B blocks of that k16 step.
        auto read_one = [&](auto grp, int i, int r) {
            const int ks = r / 6, w = r % 6;
            const int ua = decltype(grp)::value == 0 ? U_A0 + (i & 1) : U_A1 + (i % 3);
            const int ub = U_B + 2 * (i & 1) + (q & 1);
            if (w < FM) {
                if constexpr (AM)
                    af[ks][w] = read_mn(smem + ua * UNIT, ks, (q >> 1) * 64 + w * 32);
                else
                    af[ks][w] = *reinterpret_cast<const u32x4 *>(smem + ua * UNIT + (q >> 1) * 64 * PITCH +
                                                                 w * 32 * PITCH + roff(ks));
            } else {
                if constexpr (BNM)
                    bf[ks][w - FM] = read_mn(smem + ub * UNIT, ks, (w - FM) * 32);
                else
                    bf[ks][w - FM] = *reinterpret_cast<const u32x4 *>(smem + ub * UNIT + (w - FM) * 32 * PITCH +
                                                                      roff(ks));
            }
        };
        // The 8 loads of slab `li` and its scales; `nt` (a compile-time flag)
        // gives group 0's B loads the non-temporal policy.
        auto issue_loads = [&](auto grp, int li, auto nt) {
    #pragma unroll
            for (int n = 0; n < 8; ++n)
                group_load(grp, li, n, nt);
            scale_load(grp, li);
        };
        // One memory phase: the 8 loads of slab `li` (if has_load), then the 24
        // fragment reads of slab i.  Loads first: their issue is what the vector
        // memory unit paces, and the reads overlap it.
        auto memory_phase = [&](auto grp, int i, bool has_load, int li, auto nt, bool reads = true) {
            if (has_load)
                issue_loads(grp, li, nt);
            if (reads) {
    #pragma unroll
                for (int r = 0; r < 24; ++r)
                    read_one(grp, i, r);
                scale_read(grp, i);
            }
        };
        auto compute_slab = [&]() {
            if constexpr (!F8) {
    #pragma unroll
                for (int ks = 0; ks < KSTEPS; ++ks)
    #pragma unroll
                    for (int fn = 0; fn < FN; ++fn)
    #pragma unroll
                        for (int fm = 0; fm < FM; ++fm)
                            acc[fn][fm] = mfma32x32x16<IN>(bf[ks][fn], af[ks][fm], acc[fn][fm]);
            } else if constexpr (SC == 0) {
    #pragma unroll
                for (int k2 = 0; k2 < 2; ++k2)
    #pragma unroll
                    for (int fn = 0; fn < FN; ++fn)
    #pragma unroll
                        for (int fm = 0; fm < FM; ++fm)
                            acc[fn][fm] = mfma32x32x64_f8<IN>(bf[2 * k2][fn], bf[2 * k2 + 1][fn],
                                                              af[2 * k2][fm], af[2 * k2 + 1][fm],
                                                              acc[fn][fm]);
            } else {
                float r[FM];
    #pragma unroll
                for (int fm = 0; fm < FM; ++fm) {
                    const bool zero = sblk[fm] == 0.0f;
                    r[fm] = zero ? 1.0f : unit[fm] * __builtin_amdgcn_rcpf(sblk[fm]);
                    unit[fm] = zero ? unit[fm] : sblk[fm];
                    if (__builtin_amdgcn_ballot_w64(zero)) {
    #pragma unroll
                        for (int ks = 0; ks < KSTEPS; ++ks)
                            af[ks][fm] = zero ? (u32x4){0u, 0u, 0u, 0u} : af[ks][fm];
                    }
                }
    #pragma unroll
                for (int fn = 0; fn < FN; ++fn)
    #pragma unroll
                    for (int fm = 0; fm < FM; ++fm) {
    #pragma unroll
                        for (int e = 0; e < 16; ++e)
                            acc[fn][fm][e] *= r[fm];
                        acc[fn][fm] = mfma32x32x64_f8<IN>(bf[0][fn], bf[1][fn], af[0][fm], af[1][fm],
                                                          acc[fn][fm]);
                        acc[fn][fm] = mfma32x32x64_f8<IN>(bf[2][fn], bf[3][fn], af[2][fm], af[3][fm],
                                                          acc[fn][fm]);
                    }
                // Interleave: the rescale of the next block runs under the MFMAs
                // of the current one (8 multiplies beside each MFMA).
                __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);
    #pragma unroll
                for (int b = 0; b < FN * FM; ++b) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
                }
            }
        };
        // loads a group-1 wave keeps in flight across its compute phase: the
        // eight of the next A slab and, with blockwise scales, its row scales
        constexpr int A_INFLIGHT = SC == 1 ? 9 : 8;
        auto phase_end = [&]() {
            __builtin_amdgcn_sched_barrier(0);
            wg_barrier();
            __builtin_amdgcn_sched_barrier(0);
        };
        using G0 = std::integral_constant<int, 0>;
        using G1 = std::integral_constant<int, 1>;

        // Group 1 owns tile rows 128..255.  When all of them lie past M (a
        // grouped problem with few tokens, the last tile row of a ragged M) its
        // waves skip their fragment reads and MFMAs: they still load A for group
        // 0 and keep every barrier, and their accumulators, never stored, stay 0.
        // (Not in the persistent kernel, whose registers it would overflow.)
        const bool g1_rows = PS != 0 || m0 + 128 < p.M;
        // Group 1 waits with the loads of a later A slab in flight.  A load out
        // of range in every lane touches no memory and may count as done ahead
        // of the loads issued before it, which would let such a wait pass
        // early.  No MN-major A load is (columns past M are clamped), nor a
        // K-major one with the row-0 redirect; without it the count-based waits
        // need every A row inside M.  The k-rows past K of an MN-major A's last
        // slab are such loads too: the count-based waits are never used with
        // that slab in flight.
        const bool a_exact = AM || redirect_a || rows_a == BM;
        GNT_PP2_TRACE_DECL
        if (nk > 0) {
            // Prologue: B(0) by group 0; A(0), A(1) by group 1.  Slab 0 lands before
            // phase 0; A(1) by the end of phase 1 (the steady-state wait).
            if (group == 0) {
                if (SC != 1 && p.nt_b)
                    issue_loads(G0{}, 0, std::integral_constant<bool, SC != 1>{});
                else
                    issue_loads(G0{}, 0, std::false_type{});
                wait_vmcnt<0>();
            } else {
                issue_loads(G1{}, 0, std::false_type{});
                if (nk > 1)
                    issue_loads(G1{}, 1, std::false_type{});
                if (a_exact && (nk > 2 || (nk == 2 && !AM)))
                    wait_vmcnt<A_INFLIGHT>();
                else
                    wait_vmcnt<0>();
            }
            phase_end();
            if (group == 0) {
                // two copies of the loop, for the two policies of the B loads
                auto g0_loop = [&](auto nt) {
                    for (int i = 0; i < nk; ++i) {
                        GNT_PP2_EVENT(i, 0);
                        memory_phase(G0{}, i, i + 1 < nk, i + 1, nt);    // B(i+1)
                        wait_lgkmcnt0();
                        GNT_PP2_FLUSH(0, i);
                        GNT_PP2_EVENT(i, 1);
                        phase_end();                               // end of phase 2i
                        GNT_PP2_EVENT(i, 2);
                        compute_slab();
                        __builtin_amdgcn_sched_barrier(0);
                        GNT_PP2_EVENT(i, 3);
                        wait_vmcnt<0>();                           // B(i+1) landed
                        GNT_PP2_EVENT(i, 4);
                        phase_end();                               // end of phase 2i+1
                    }
                };
                // (blockwise FP8 keeps one copy, with the default policy: a second
                // one does not fit its registers)
                if (SC != 1 && p.nt_b)
                    g0_loop(std::integral_constant<bool, SC != 1>{});
                else
                    g0_loop(std::false_type{});
            } else {
                for (int i = 0; i < nk; ++i) {
                    GNT_PP2_EVENT(i, 0);
                    if (i > 0 && g1_rows)
                        compute_slab();                        // slab i-1
                    __builtin_amdgcn_sched_barrier(0);
                    GNT_PP2_EVENT(i, 1);
                    phase_end();                               // end of phase 2i
                    GNT_PP2_EVENT(i, 2);
                    memory_phase(G1{}, i, i + 2 < nk, i + 2, std::false_type{}, g1_rows);   // A(i+2)
                    wait_lgkmcnt0();
                    GNT_PP2_FLUSH(1, i);
                    GNT_PP2_EVENT(i, 3);
                    if (a_exact && (i + 3 < nk || (i + 2 < nk && !AM)))   // A(i+1) landed
                        wait_vmcnt<A_INFLIGHT>();
                    else
                        wait_vmcnt<0>();
                    GNT_PP2_EVENT(i, 4);
                    phase_end();                               // end of phase 2i+1
                }
                if (g1_rows)
                    compute_slab();                            // slab nk-1
            }
        }

        GNT_PP2_DUMP
        // Epilogue (the ring is free: the last fragment read and the last load
        // completed before the loop's last barrier).  Each wave stages its own
        // 64 x 128 block in its own 16 KB of LDS.
        if constexpr (F8) {
            // per-tensor scales (every load of the main loop has completed), or
            // the blockwise accumulators' last units
            float s[FM];
            if constexpr (SC == 0)
                s[0] = s[1] = p.scale_a[0] * p.scale_b[0];
            else
                s[0] = unit[0], s[1] = unit[1];
    #pragma unroll
            for (int fn = 0; fn < FN; ++fn)
    #pragma unroll
                for (int fm = 0; fm < FM; ++fm)
    #pragma unroll
                    for (int e = 0; e < 16; ++e)
                        acc[fn][fm][e] *= s[fm];
        }
        if constexpr (PS == 0 && !GR) {
            if (p.inreduce) {
                // two K splits: the second to arrive holds the sum and stores it
                // as an unsplit tile (the flag lives in unit 8, past the staging
                // area)
                if (!splitk2_arrive<8, FN, FM>(p, acc, tm * p.tiles_n + tn, split, wave, lane,
                                               reinterpret_cast<uint32_t *>(smem + 8 * UNIT)))
                    return;
                p.splits = 1;
            }
        }
        uint8_t *stage = smem + wave * 16384;
        if constexpr (streamk) {
            // a whole 256 x 256 slot per segment, ragged tiles included
            float *ws = p.partials + (int64_t)sk_slot * (BM * BN);
            store_block_staged<float>(acc, stage, ws + wm0 * BN + wn0, BN, lane);
        } else {
            const bool full = m0 + BM <= p.M && n0 + BN <= p.N;
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
                    store_block_staged<__bf16, true>(acc, stage, static_cast<__bf16 *>(p.C) + (int64_t)(m0 + wm0) * p.ldc + (n0 + wn0), p.ldc, lane);
                else if constexpr (OUT == OUT_FP16)
                    store_block_staged<_Float16, true>(acc, stage, static_cast<_Float16 *>(p.C) + (int64_t)(m0 + wm0) * p.ldc + (n0 + wn0), p.ldc, lane);
                else
                    store_block_staged<float, true>(acc, stage, static_cast<float *>(p.C) + (int64_t)(m0 + wm0) * p.ldc + (n0 + wn0), p.ldc, lane);
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
    };

    int tm, tn, split;
    if constexpr (GR) {
        // Grouped launch: this block's launch position names its problem and
        // the tile within it; the problem's fields replace the launch's.
        const int v = xcd_order(blockIdx.x, gridDim.x);
        const int g = __builtin_amdgcn_readfirstlane(p0.tile_group[v]);
        const GroupDesc *d = p0.groups + g;
        auto u32 = [](int x) { return __builtin_amdgcn_readfirstlane(x); };
        auto uptr = [](const void *x) {
            const uint64_t a = (uint64_t)(uintptr_t)x;
            const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
            const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
            return (void *)(uintptr_t)(((uint64_t)hi << 32) | lo);
        };
        p.A = static_cast<const uint16_t *>(uptr(d->A));
        p.B = static_cast<const uint16_t *>(uptr(d->B));
        p.C = uptr(d->C);
        p.bias = static_cast<const float *>(uptr(d->bias));
        p.M = u32(d->M), p.N = u32(d->N), p.K = u32(d->K);
        p.lda = u32(d->lda), p.ldb = u32(d->ldb), p.ldc = u32(d->ldc);
        p.tiles_m = u32(d->tiles_m), p.tiles_n = u32(d->tiles_n), p.k_tiles = u32(d->k_tiles);
        p.splits = 1;
        p.kt_per_split = p.k_tiles;
        const int flags = u32(d->flags);
        p.vec_store = flags & GD_VEC_STORE ? 1 : 0;
        p.rows16 = flags & GD_ROWS16 ? 1 : 0;
        p.bias_vec = flags & GD_BIAS_VEC ? 1 : 0;
        p.nt_b = flags & GD_NT_B ? 1 : 0;
        if constexpr (F8) {
            p.scale_a = static_cast<const float *>(uptr(d->scale_a));
            p.scale_b = static_cast<const float *>(uptr(d->scale_b));
            p.sf_ld = u32(d->sf_ld);
            p.sfa_bytes = (uint32_t)u32((int)d->sfa_bytes);
            p.sfb_bytes = (uint32_t)u32((int)d->sfb_bytes);
        }
        split = 0;
        tile_order(v - u32(d->tile_start), p.tiles_m, p.tiles_n, p.group_m, tm, tn);
        tile(tm, tn, split);
    } else if constexpr (PS == 2) {
        // Stream-K: block b takes the contiguous units [b T / G, (b + 1) T / G)
        // of the T = tiles * k_tiles (tile, k-slab) units in tile-major order,
        // one segment per tile it touches; a barrier between segments, as
        // between the persistent loop's units below.
        // (T < 2^31, checked by the host; the values are wave-uniform)
        auto uni = [](int x) { return __builtin_amdgcn_readfirstlane(x); };
        const int T = uni(p.sk_units), G = uni((int)gridDim.x);
        int u = uni((int)((int64_t)blockIdx.x * T / G));
        const int end = uni((int)((int64_t)(blockIdx.x + 1) * T / G));
        for (int seg = 0; u < end; ++seg) {
            const int t = uni(u / p.k_tiles);
            const int e = min(end, (t + 1) * p.k_tiles);
            tile(uni(t / p.tiles_n), uni(t % p.tiles_n), 0, uni(u - t * p.k_tiles), uni(e - u),
                 uni((int)blockIdx.x * p.sk_maxseg + seg));
            wg_barrier();
            u = e;
        }
    } else if constexpr (PS == 1) {
        // Persistent blocks (grid a multiple of 8, at most the work units):
        // XCD x (the blocks with id % 8 == x) owns the contiguous run
        // [x T / 8, (x + 1) T / 8) of the T work units in tile order, and its
        // blocks take every (grid / 8)-th unit of the run, so the tiles in
        // flight on one XCD stay neighbours that share operand panels in its
        // L2.  A barrier between units: the epilogue's LDS staging is read
        // before the next unit's loads land in the ring.
        const int T = p.tiles_m * p.tiles_n * p.splits;
        const int tiles = p.tiles_m * p.tiles_n;
        const int x = blockIdx.x & 7, j = blockIdx.x >> 3, per = gridDim.x >> 3;
        const int c0 = (int)((int64_t)x * T / 8), c1 = (int)((int64_t)(x + 1) * T / 8);
        for (int v = c0 + j; v < c1; v += per) {
            split = v / tiles;
            tile_order(v - split * tiles, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
            tile(tm, tn, split);
            wg_barrier();
        }
    } else {
        if (p.inreduce)
            map_block_split_minor(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, p.splits, tm, tn,
                                  split);
        else
            map_block(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn, split);
        tile(tm, tn, split);
    }
}

}  // namespace gnt
