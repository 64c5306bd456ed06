/*
 * gemm_nt.h -- C ABI of the MI355X (gfx950) NT GEMM library.
 *
 * Operation (all three pages that write the kernel out agree on it):
 *   C[i, j] = out( sum_{k=0}^{K-1} A[i, k] * B[j, k] ),   0 <= i < M, 0 <= j < N
 * "A Blackwell GEMM by Hand in CuTe DSL: TMA, mbarriers, TMEM, and tcgen05",
 * section 1 (C = A . B^T, 2MNK operations) and section 3 (A and B both K-major,
 * 16-bit inputs, FP32 accumulation); "Matmul on sm_120", The tiled view (the
 * per-element sum, and the tiled form the kernels compute it in).
 *
 * Storage: row-major with element strides.  A is M rows of lda elements, B is N
 * rows of ldb elements (the [out, in] weight layout of a linear layer), C is M
 * rows of ldc elements; only the first K columns of A and B and the first N
 * columns of C are touched.  Inputs are both BF16 or both FP16; products are
 * exact and accumulate in FP32; the FP32 sum is written as FP32 or rounded to
 * BF16/FP16 with round-to-nearest-even.  The summation order is unspecified
 * (any order the tiling chooses), but for given arguments every call on the
 * same device returns the same bits.
 *
 * The other entry points widen this product: gemm_run_ex adds a fused
 * epilogue (scale, prior C, bias, activation), gemm_run_layout lets either
 * operand be stored MN-major, gemm_run_fp8 takes FP8 operands with per-tensor
 * or blockwise scales, and gemm_run_grouped / gemm_run_grouped_fp8 run a list
 * of such products in one launch.
 *
 * Ownership: A, B and C are device pointers owned by the caller.  The handle
 * owns its workspace (FP32 split-K partial sums, or a grouped launch's problem
 * list) and a pinned staging buffer for grouped problem lists.
 *
 * Streams: every run call only enqueues work on `stream` (0 = the null stream)
 * and never synchronises (a grouped call waits only for the copy out of its
 * staging buffer made by the previous grouped call).  One handle must not be
 * used by two calls that may run concurrently (its workspace is shared); use
 * one handle per stream.
 *
 * Errors: every argument error is returned before any device work is enqueued.
 */
#ifndef GEMM_NT_H
#define GEMM_NT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t;
typedef struct ihipStream_t *hipStream_t;

typedef struct gemm_handle_s *gemm_handle_t;

typedef enum {
    GEMM_BF16 = 0,
    GEMM_FP16 = 1,
    GEMM_FP32 = 2,
    GEMM_FP8_E4M3 = 3, /* inputs of gemm_run_fp8 only: OCP E4M3 (bias 7, no infinities, max 448) */
    GEMM_FP8_E5M2 = 4  /* OCP E5M2 (bias 15, IEEE-style infinities and NaNs, max 57344) */
} gemm_dtype_t;

typedef enum {
    GEMM_OK = 0,
    GEMM_ERR_INVALID_ARG = 1, /* null pointer, negative size, leading dimension too small */
    GEMM_ERR_UNSUPPORTED = 2, /* unknown dtype enum, FP32 inputs, a size beyond the limits */
    GEMM_ERR_MISALIGNED = 3,  /* A/B base or row pitch not a multiple of 16 bytes */
    GEMM_ERR_ALLOC = 4,       /* workspace allocation failed */
    GEMM_ERR_HIP = 5          /* a HIP runtime call or a launch failed */
} gemm_status_t;

/* Create a handle on the current device: allocates the workspace for split-K
 * and stream-K partials (128 MiB by default; GEMM_WORKSPACE_MB overrides) and
 * 64 KiB of per-tile counters, which it zeroes (synchronously) and which every
 * call leaves at zero.  GEMM_INREDUCE=0 turns the in-kernel reduction of K
 * splits off (two on the 256-row tiles, any number on the 32 x 128 and
 * 128 x 128 tiles; every split plan then takes the second pass, with the
 * same bits).
 * *out is NULL on error.  For measurement, GEMM_CONFIG=<name> forces one kernel
 * configuration, GEMM_SPLITS=<n> a K split on every call of this handle, and
 * GEMM_STREAMK=0/1/2 turns stream-K off, leaves it to the plan (default) or
 * uses it whenever the 256 x 256 ping-pong tile is planned; a GEMM_CONFIG that
 * names no configuration makes gemm_create return GEMM_ERR_INVALID_ARG.
 * GEMM_PERSIST=1 runs planned 256 x 256 ping-pong grids of more than 256
 * blocks with 256 persistent blocks.  GEMM_ROTATE=0/1/2 sets the order in
 * which the 32 x 128 and 128 x 128 tiles walk their K slabs: from the first
 * slab, from a start rotated per 256-column block when M <= 128 (default), or
 * rotated always (the 256-row tiles always start at the first slab); the
 * order is the FP32 summation order, so it changes the bits.  GEMM_LOG=1 prints each call's plan to
 * stderr.  GEMM_TEST_FAIL_ALLOC=1 makes gemm_create fail as a failed workspace
 * allocation does (GEMM_ERR_ALLOC, *out NULL), to test callers' error paths. */
gemm_status_t gemm_create(gemm_handle_t *out);

/* C = A . B^T (see the top of this file).
 *   A, B      device pointers, 16-byte aligned; lda, ldb multiples of 8 elements
 *   C         device pointer, any alignment of its element type; ldc >= N
 *   M, N, K   >= 0; M = 0 or N = 0 enqueues nothing; K = 0 writes zeros
 *   lda >= K, ldb >= K, ldc >= N (elements); lda and ldb below 2^22
 *   in_dtype  GEMM_BF16 or GEMM_FP16 (both operands)
 *   out_dtype GEMM_BF16, GEMM_FP16 or GEMM_FP32
 * Returns GEMM_OK after enqueueing, or an error status with nothing enqueued. */
gemm_status_t gemm_run(gemm_handle_t h, const void *A, const void *B, void *C,
                       int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                       int in_dtype, int out_dtype, hipStream_t stream);

/* gemm_run for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  No handle:
 * split-K and stream-K partials go to a static scratch array of
 * GEMM_NOALLOC_SCRATCH_BYTES (64 MiB) per device, which the library's code
 * object holds on each device it runs on from the first call there until the
 * process ends.  The call itself allocates nothing (no hipMalloc, hipFree or
 * allocating library routine).
 *   Arguments, results and errors as gemm_run on the current device (with a
 *   handle made without GEMM_* switches), with one difference in the plan: a
 *   stream-K plan whose partials would exceed the scratch takes the split plan
 *   instead, so its results may differ from gemm_run's in the summation order
 *   (within the same bound); every other plan is gemm_run's, with the same
 *   bits.  A plan that still needed more scratch would return
 *   GEMM_ERR_UNSUPPORTED with nothing enqueued.
 *   Every call on one device shares that device's scratch: two calls that may
 *   run concurrently on one device (different streams, or different host
 *   threads without ordering) race on it.  Serialise them, e.g. on one stream.
 *   Each call writes every partial it reads; the array's per-tile counters
 *   start at zero when the library is loaded and every call leaves them at
 *   zero. */
#define GEMM_NOALLOC_SCRATCH_BYTES ((int64_t)64 << 20)   /* partials; plus 64 KiB of counters */
gemm_status_t gemm_run_noalloc(const void *A, const void *B, void *C,
                               int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                               int64_t ldc, int in_dtype, int out_dtype, hipStream_t stream);

/* Fused epilogue ("CUTLASS Deep Dive: From CuTe Layouts to Blackwell tcgen05",
 * the Tutorial 01/05 epilogues, "Epilogue Visitor Trees (EVT)" and "Classic
 * Fused Epilogue: Bias + ReLU"): as each output tile is written back,
 *     C[i,j] = act( alpha * sum_k A[i,k] B[j,k] + beta * C_old[i,j] + bias )
 * computed in FP32 and rounded once to out_dtype (round to nearest even).
 *   alpha, beta  FP32 scalars; beta != 0 reads the prior contents of C
 *   bias         device pointer to FP32 values, 4-byte aligned, caller-owned:
 *                N of them (bias_along GEMM_BIAS_N: one per output column, the
 *                bias of a linear layer whose weights are the rows of B) or M
 *                (GEMM_BIAS_M: one per output row); NULL when GEMM_BIAS_NONE
 *   activation   GEMM_ACT_NONE, GEMM_ACT_RELU (max(0, x)) or GEMM_ACT_GELU
 *                (x * Phi(x) = x / 2 * (1 + erf(x / sqrt(2))))  */
typedef enum { GEMM_BIAS_NONE = 0, GEMM_BIAS_N = 1, GEMM_BIAS_M = 2 } gemm_bias_t;
typedef enum { GEMM_ACT_NONE = 0, GEMM_ACT_RELU = 1, GEMM_ACT_GELU = 2 } gemm_act_t;
typedef struct {
    float alpha;
    float beta;
    const float *bias;
    int bias_along;  /* gemm_bias_t */
    int activation;  /* gemm_act_t */
} gemm_epilogue_t;

/* gemm_run with a fused epilogue.  epi == NULL is the plain product
 * (alpha = 1, beta = 0, no bias, no activation).  Errors as gemm_run, plus
 * GEMM_ERR_INVALID_ARG for an unknown bias_along or activation, a missing or
 * misaligned bias, and GEMM_ERR_UNSUPPORTED for a non-finite alpha or beta.
 * With beta != 0, C must hold the prior output values. */
gemm_status_t gemm_run_ex(gemm_handle_t h, const void *A, const void *B, void *C,
                          int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                          int in_dtype, int out_dtype, const gemm_epilogue_t *epi,
                          hipStream_t stream);

/* Operand layouts.  The NT form keeps both operands K-major ("A Blackwell GEMM
 * by Hand in CuTe DSL", the header of its kernel listing); "Optimizing GEMMs
 * using tcgen05 - Part 1" ("What I am measuring") multiplies a row-major A
 * [M][K] by a row-major B [K][N], which is B stored N-major; "Steps for Writing
 * a Speed-of-Light GEMM kernel: Part 1" (its CuTe introduction) defines a
 * layout as the map from a logical coordinate to a storage offset.
 *   GEMM_K_MAJOR   A is M rows of lda elements (element (i,k) at A[i*lda + k]),
 *                  B is N rows of ldb elements (element (j,k) at B[j*ldb + k])
 *   GEMM_MN_MAJOR  A is K rows of lda elements (element (i,k) at A[k*lda + i]),
 *                  B is K rows of ldb elements (element (j,k) at B[k*ldb + j])
 * so NT = (K, K) and the row-major "A times B" with B [K][N] is (K, MN). */
typedef enum { GEMM_K_MAJOR = 0, GEMM_MN_MAJOR = 1 } gemm_layout_t;

/* gemm_run_ex for any operand layouts: C[i,j] = act(alpha sum_k a(i,k) b(j,k)
 * + beta C_old + bias) with a, b read as layout_a / layout_b (gemm_layout_t)
 * say; C and the epilogue as in gemm_run_ex.
 *   lda >= K (K-major A) or >= M (MN-major A); ldb >= K or >= N likewise;
 *   lda, ldb multiples of 8 below 2^22 and A, B 16-byte aligned.
 * Layouts other than (K, K) need K % 8 == 0 (else GEMM_ERR_UNSUPPORTED) and run
 * on the 256 x 256 ping-pong tile (a handle forced to another configuration
 * returns GEMM_ERR_UNSUPPORTED); a layout value outside gemm_layout_t is
 * GEMM_ERR_INVALID_ARG.  (K, K) is exactly gemm_run_ex. */
gemm_status_t gemm_run_layout(gemm_handle_t h, int layout_a, int layout_b, const void *A,
                              const void *B, void *C, int64_t M, int64_t N, int64_t K,
                              int64_t lda, int64_t ldb, int64_t ldc, int in_dtype, int out_dtype,
                              const gemm_epilogue_t *epi, hipStream_t stream);

/* FP8 scaling ("CUTLASS Deep Dive: From CuTe Layouts to Blackwell tcgen05",
 * "FP8 and Blockwise Scaling": one scale per tensor, or one per (block_m,
 * block_k) tile of A and per (block_n, block_k) tile of B, applied while
 * accumulating).  Here block_k = block_n = 128 and the scales are FP32 device
 * arrays, row-major:
 *   GEMM_SCALE_TENSOR  a, b: one value each
 *   GEMM_SCALE_BLOCK   a: [ceil(M / block_m)][ceil(K / 128)], block_m 1 or 128
 *                      b: [ceil(N / 128)][ceil(K / 128)]
 * Blockwise scales must be finite and either zero or normal (|s| >= 2^-126);
 * the kernel holds each accumulator in units of the current block's scale
 * product, so along one output row the ratio between scale products of
 * different k-blocks must stay below about 2^80. */
typedef enum { GEMM_SCALE_TENSOR = 0, GEMM_SCALE_BLOCK = 1 } gemm_scale_mode_t;
typedef struct {
    int mode;        /* gemm_scale_mode_t */
    const float *a;  /* device pointer, 4-byte aligned */
    const float *b;  /* device pointer, 4-byte aligned */
    int block_m;     /* GEMM_SCALE_BLOCK: rows of A per scale, 1 or 128 */
} gemm_fp8_scales_t;

/* FP8 GEMM with scales: C[i,j] = act(alpha sum_k sa(i,k) a(i,k) sb(j,k) b(j,k)
 * + beta C_old + bias), a and b decoded from the a_dtype / b_dtype FP8 codes
 * (GEMM_FP8_E4M3 or GEMM_FP8_E5M2 each, K-major: A is M rows of lda bytes, B
 * N rows of ldb bytes), sa / sb from `scales`; FP32 accumulation; C and the
 * epilogue (NULL = identity) as in gemm_run_ex.
 *   K % 16 == 0 and lda, ldb multiples of 16 (else GEMM_ERR_UNSUPPORTED /
 *   GEMM_ERR_MISALIGNED); A, B 16-byte aligned; lda, ldb >= K, below 2^22.
 *   scales NULL, a null scale pointer, an unknown mode or block_m:
 *   GEMM_ERR_INVALID_ARG.  Runs on the 256 x 256 ping-pong tile. */
gemm_status_t gemm_run_fp8(gemm_handle_t h, int a_dtype, int b_dtype, const void *A,
                           const void *B, void *C, int64_t M, int64_t N, int64_t K, int64_t lda,
                           int64_t ldb, int64_t ldc, int out_dtype,
                           const gemm_fp8_scales_t *scales, const gemm_epilogue_t *epi,
                           hipStream_t stream);

/* One problem of a grouped launch: C = A . B^T with A M rows of lda elements,
 * B N rows of ldb, C M rows of ldc (K-major, as gemm_run). */
typedef struct {
    const void *A;
    const void *B;
    void *C;
    const float *bias;  /* this group's FP32 bias when the epilogue has a bias axis, else unused */
    int64_t M, N, K;
    int64_t lda, ldb, ldc;
} gemm_group_problem_t;

/* Grouped GEMM ("CUTLASS Deep Dive: From CuTe Layouts to Blackwell tcgen05",
 * "Grouped GEMM -- MoE's workhorse": many GEMMs of different shapes, e.g. one
 * per expert, in one kernel launch whose tiles each look up their problem).
 * For g < num_groups: C_g = act(alpha A_g . B_g^T + beta C_g_old + bias_g),
 * all groups in in_dtype (BF16 or FP16) -> out_dtype with one epilogue
 * (epi->bias must be NULL: group g's bias is problems[g].bias).
 *   problems: host array, read before the call returns.  Each group passes the
 *   checks of gemm_run_ex and needs K % 8 == 0 (else GEMM_ERR_UNSUPPORTED);
 *   empty groups (M, N or K = 0; K = 0 writes the epilogue of zero) are allowed.
 *   The problem list and a per-tile lookup table are copied into the handle's
 *   workspace on `stream` (one call at a time per handle, as for split-K)
 *   through the handle's pinned staging buffer: the call waits only when the
 *   previous grouped call's copy has not run yet.  A list that does not fit
 *   the workspace returns GEMM_ERR_UNSUPPORTED.  Every group runs
 *   on the 256 x 256 ping-pong tile without K splits. */
gemm_status_t gemm_run_grouped(gemm_handle_t h, const gemm_group_problem_t *problems,
                               int num_groups, int in_dtype, int out_dtype,
                               const gemm_epilogue_t *epi, hipStream_t stream);

/* One FP8 problem of a grouped launch: as gemm_group_problem_t with 8-bit A
 * and B (lda, ldb in elements = bytes) and the group's own scales, laid out as
 * gemm_fp8_scales_t describes for the call's scale mode and block_m. */
typedef struct {
    const void *A;
    const void *B;
    void *C;
    const float *bias;
    const float *scale_a;
    const float *scale_b;
    int64_t M, N, K;
    int64_t lda, ldb, ldc;
} gemm_group_problem_fp8_t;

/* Grouped FP8 GEMM (the grouped example of "CUTLASS Deep Dive", "Grouped GEMM
 * -- MoE's workhorse", runs FP8 problems): gemm_run_grouped's one launch over
 * a host list of problems, with the operands and scales of gemm_run_fp8.  One
 * format pair, scale mode (gemm_scale_mode_t) and block_m (1 or 128, used by
 * GEMM_SCALE_BLOCK) for the whole list; per group the checks of gemm_run_fp8
 * (K % 16 == 0, lda and ldb multiples of 16, scales non-null and 4-byte
 * aligned) and the staging of gemm_run_grouped. */
gemm_status_t gemm_run_grouped_fp8(gemm_handle_t h, int a_dtype, int b_dtype,
                                   const gemm_group_problem_fp8_t *problems, int num_groups,
                                   int out_dtype, int scale_mode, int block_m,
                                   const gemm_epilogue_t *epi, hipStream_t stream);

/* Release the handle and its workspace.  NULL is a no-op.  The caller must make
 * sure no call enqueued with this handle is still running. */
gemm_status_t gemm_destroy(gemm_handle_t h);

/* Host-only argument check that gemm_run performs first (no device access). */
gemm_status_t gemm_validate(const void *A, const void *B, void *C, int64_t M, int64_t N,
                            int64_t K, int64_t lda, int64_t ldb, int64_t ldc, int in_dtype,
                            int out_dtype);

/* The kernel configuration gemm_run would launch for a shape (host only). */
typedef struct {
    int block_m, block_n, block_k; /* output tile and K depth of one LDS stage */
    int waves;                     /* wavefronts per workgroup */
    int stages;                    /* LDS ring slots (the 256x256 ping-pong kernel: 16 KB units) */
    int splits;                    /* K splits per output tile (1 = none) */
    int lds_bytes;                 /* LDS the kernel allocates per workgroup */
    int64_t tiles;                 /* output tiles */
    int64_t workgroups;            /* grid size */
    int64_t workspace_bytes;       /* split-K partials used (splits * M * N * 4; with
                                      inreduce, tiles * 2 * block_m * block_n * 4), or the
                                      stream-K slots (workgroups * segments * 256 KB) */
    char name[48];                 /* kernel configuration name */
    int streamk;                   /* 1: stream-K (each workgroup an equal run of the
                                      tiles * k-slabs units, then a reduction kernel) */
    int inreduce;                  /* 1: two K splits whose second to finish adds the
                                      first's partial and stores the tile (no second pass) */
} gemm_plan_t;

gemm_status_t gemm_plan(int64_t M, int64_t N, int64_t K, int in_dtype, int out_dtype,
                        gemm_plan_t *plan);

/* Human-readable name of a status code (static storage). */
const char *gemm_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_NT_H */
