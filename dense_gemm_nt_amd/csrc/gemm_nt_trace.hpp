// gemm_nt_trace.hpp -- phase timestamps of the ping-pong kernel, compiled only
// into a separately built, instrumented copy of the library (-DGNT_PP2_TRACE,
// dense_gemm_nt_amd/phase_trace.py); the library itself has empty hooks.
//
// Every wave reads the shader clock (s_memtime) at five points of each slab
// iteration i of its main loop, and the 100 MHz reference clock
// (s_memrealtime) at the first:
//   group 0: e0 memory phase starts, e1 its fragment reads are done, e2 the
//            barrier has passed (compute starts), e3 the MFMAs are issued,
//            e4 the wait for B(i+1) is over (then the barrier);
//   group 1: e0 compute starts, e1 the MFMAs are issued, e2 the barrier has
//            passed (memory phase starts), e3 the fragment reads are done,
//            e4 the wait for A(i+1) is over (then the barrier).
// The values stay in scalar registers and are written to an LDS area past
// the ring only right after the memory phase's own lgkmcnt(0) wait, by when
// every earlier clock read has returned: no wait is added anywhere (a clock
// read is a scalar memory operation, and using its value at once would stall
// the wave).  Slabs TRACE_T0 .. +TRACE_TN are kept.  After its main loop,
// every wave of blocks 0..31 copies its records to global memory just past
// the end of C (the caller allocates TRACE_BYTES more after C's M x ldc
// elements): record (block b, wave w, slab t) is 6 unsigned 64-bit values
// (e0..e4, reference clock at e0) at index ((b * 8 + w) * TRACE_TN + t) * 6.
#pragma once

namespace gnt {
constexpr int TRACE_T0 = 16, TRACE_TN = 16, TRACE_REC = 6, TRACE_BLOCKS = 32;
constexpr int TRACE_BYTES = TRACE_BLOCKS * 8 * TRACE_TN * TRACE_REC * 8;
}

#define GNT_PP2_TRACE_LDS (8 * gnt::TRACE_TN * gnt::TRACE_REC * 8)
#define GNT_PP2_TRACE_DECL unsigned long long gnt_tr_[6] = {0ull, 0ull, 0ull, 0ull, 0ull, 0ull};
#define GNT_PP2_EVENT(i, e)                                                              \
    do {                                                                                 \
        gnt_tr_[(e)] = __builtin_amdgcn_s_memtime();                                     \
        if ((e) == 0)                                                                    \
            gnt_tr_[5] = __builtin_amdgcn_s_memrealtime();                               \
    } while (0)
#define GNT_TRACE_SLOT(i, e)                                                             \
    (reinterpret_cast<unsigned long long *>(smem + LDS_USED)[(wave * gnt::TRACE_TN + ((i) - gnt::TRACE_T0)) * gnt::TRACE_REC + (e)])
#define GNT_TRACE_KEPT(i) ((i) >= gnt::TRACE_T0 && (i) < gnt::TRACE_T0 + gnt::TRACE_TN)
// group 0 writes e0 of this slab and e1..e4 of the previous one; group 1 e0..e2
// of this slab and e3, e4 of the previous one (the later events of a slab are
// read after this point)
#define GNT_PP2_FLUSH(g, i)                                                              \
    do {                                                                                 \
        if (lane_id == 0) {                                                              \
            constexpr int last_ = (g) == 0 ? 0 : 2;                                      \
            if (GNT_TRACE_KEPT(i)) {                                                     \
                for (int e_ = 0; e_ <= last_; ++e_)                                      \
                    GNT_TRACE_SLOT(i, e_) = gnt_tr_[e_];                                 \
                GNT_TRACE_SLOT(i, 5) = gnt_tr_[5];                                       \
            }                                                                            \
            if (GNT_TRACE_KEPT((i) - 1))                                                 \
                for (int e_ = last_ + 1; e_ <= 4; ++e_)                                  \
                    GNT_TRACE_SLOT((i) - 1, e_) = gnt_tr_[e_];                           \
        }                                                                                \
    } while (0)
#define GNT_PP2_DUMP                                                                     \
    {                                                                                    \
        wait_lgkmcnt0();                                                                 \
        if (blockIdx.x < gnt::TRACE_BLOCKS) {                                            \
            constexpr int n_ = gnt::TRACE_TN * gnt::TRACE_REC;                           \
            unsigned long long *out_ = reinterpret_cast<unsigned long long *>(           \
                static_cast<char *>(p.C) + (size_t)p.M * p.ldc * (OUT == OUT_FP32 ? 4 : 2)); \
            for (int t_ = lane_id; t_ < n_; t_ += 64)                                    \
                out_[(blockIdx.x * 8 + wave) * n_ + t_] =                                \
                    reinterpret_cast<const unsigned long long *>(smem + LDS_USED)[wave * n_ + t_]; \
        }                                                                                \
    }
