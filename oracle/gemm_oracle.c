/*
 * gemm_oracle.c -- plain CPU oracle for the NT GEMM  C[M,N] = A[M,K] . B[N,K]^T.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the GPU library includes, links or calls
 * this file; only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark load it.  It shares no header, table or helper with the HIP code.
 *
 * What it computes (the plain definition, written out):
 *   - "A Blackwell GEMM by Hand in CuTe DSL: TMA, mbarriers, TMEM, and tcgen05",
 *     section 1 (Two regimes): C (M x N) equals A (M x K) times the transpose of
 *     B (N x K); section 3 (The kernel), file header: A and B are both K-major,
 *     16-bit inputs, FP32 accumulation is the intended arithmetic.
 *   - "Steps for Writing a Speed-of-Light GEMM kernel: Part 1", Intro to Matrix
 *     Multiplication: one scalar sum per output element over the whole K range
 *     (the naive three-loop form); Kernel 1 + Specifications: bf16 entries,
 *     products accumulated at higher precision.
 *   - "Matmul on sm_120", The tiled view: C_ij is the sum over k of A_ik B_kj; the
 *     printed upper limit K is read as K-1 (k runs over the K columns of A).
 *
 * Arithmetic: every 16-bit input is decoded exactly to binary64; each product of
 * two decoded values is exact in binary64 (at most 11+11 significant bits); the
 * sum runs in increasing k in binary64.  Alongside C the oracle returns
 * S[i,j] = sum_k |a(i,k) b(j,k)|, the scale the acceptance tolerance is stated in.
 *
 * Parity pins (tests marked "not gpu"): exhaustive decode of all 65536 codes of
 * each format against library conversions; exact rational brute force on tiny
 * shapes; closed forms (all-ones gives K, identity B gives A, rank-1 gives a
 * product of sums); numpy float64 products; RNE encoding against library
 * float32 -> bf16/fp16 conversion.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Input formats accepted by the oracle (same numbering as the public enum, but
 * declared here independently). */
enum { ORACLE_BF16 = 0, ORACLE_FP16 = 1 };

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits. */
double oracle_decode_bf16(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 7) & 0xFF;
    int f = h & 0x7F;
    double v;
    if (e == 0xFF)
        v = f ? NAN : INFINITY;
    else if (e == 0)
        v = ldexp((double)f, 1 - 127 - 7);          /* subnormal: 0.f x 2^-126 */
    else
        v = ldexp((double)(f | 0x80), e - 127 - 7); /* 1.f x 2^(e-127) */
    return sign ? -v : v;
}

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_decode_fp16(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    double v;
    if (e == 0x1F)
        v = f ? NAN : INFINITY;
    else if (e == 0)
        v = ldexp((double)f, 1 - 15 - 10);
    else
        v = ldexp((double)(f | 0x400), e - 15 - 10);
    return sign ? -v : v;
}

/* Round a binary64 value to a binary format with `ebits` exponent bits and
 * `fbits` fraction bits, round-to-nearest, ties-to-even, and return its code.
 * Written from the IEEE-754 definition: find the quantum of the binade the value
 * falls in (clamped to the subnormal quantum), scale to an integer multiple of
 * it, pick the nearer integer (the even one on a tie), and re-encode; a carry
 * out of the significand moves to the next binade, beyond the largest finite
 * value the result is infinity. */
static uint16_t encode_rne(double x, int ebits, int fbits)
{
    const int bias = (1 << (ebits - 1)) - 1;
    const int emin = 1 - bias;
    const int emax = bias;
    const uint16_t sign = signbit(x) ? (uint16_t)(1u << (ebits + fbits)) : 0;
    const uint16_t inf_code = (uint16_t)(((1u << ebits) - 1) << fbits);
    if (isnan(x))
        return (uint16_t)(inf_code | (1u << (fbits - 1))); /* quiet NaN */
    double a = fabs(x);
    if (isinf(a))
        return sign | inf_code;
    if (a == 0.0)
        return sign;
    int e2;
    (void)frexp(a, &e2); /* a = m * 2^e2, m in [0.5, 1) */
    int E = e2 - 1;      /* a in [2^E, 2^(E+1)) */
    if (E < emin)
        E = emin;
    double n = ldexp(a, fbits - E); /* a / quantum, exact (power-of-two scale) */
    double r = floor(n);
    double frac = n - r;
    if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0))
        r += 1.0;
    const double one = ldexp(1.0, fbits); /* hidden bit position */
    if (r >= 2.0 * one) {                 /* carried into the next binade */
        r = one;
        E += 1;
    }
    if (E > emax)
        return sign | inf_code;
    if (r < one) /* subnormal (or rounded to zero): exponent field 0 */
        return sign | (uint16_t)r;
    return sign | (uint16_t)((unsigned)(E + bias) << fbits) | (uint16_t)(r - one);
}

uint16_t oracle_encode_bf16(double x) { return encode_rne(x, 8, 7); }
uint16_t oracle_encode_fp16(double x) { return encode_rne(x, 5, 10); }

static int fill_table(int dtype, double *table)
{
    if (dtype != ORACLE_BF16 && dtype != ORACLE_FP16)
        return -1;
    for (uint32_t c = 0; c < 65536u; ++c)
        table[c] = dtype == ORACLE_BF16 ? oracle_decode_bf16((uint16_t)c)
                                        : oracle_decode_fp16((uint16_t)c);
    return 0;
}

/* One output element: the sum over k in increasing order, and the sum of the
 * absolute products. */
static void dot_one(const double *table, const uint16_t *arow, const uint16_t *brow,
                    int64_t K, double *c, double *s)
{
    double acc = 0.0, mag = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double p = table[arow[k]] * table[brow[k]];
        acc += p;
        mag += fabs(p);
    }
    *c = acc;
    *s = mag;
}

/* Full product.  A is M rows of lda codes, B is N rows of ldb codes (only the
 * first K of each row are read).  C and S are dense M x N row-major binary64
 * (S may be NULL).  Returns 0, or -1 on a bad argument. */
int oracle_gemm_nt(const uint16_t *A, const uint16_t *B, int64_t M, int64_t N, int64_t K,
                   int64_t lda, int64_t ldb, int dtype, double *C, double *S)
{
    if (M < 0 || N < 0 || K < 0 || lda < K || ldb < K || !C)
        return -1;
    double *table = (double *)malloc(65536 * sizeof(double));
    if (!table)
        return -1;
    if (fill_table(dtype, table)) {
        free(table);
        return -1;
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            double c, s;
            dot_one(table, A + i * lda, B + j * ldb, K, &c, &s);
            C[i * N + j] = c;
            if (S)
                S[i * N + j] = s;
        }
    }
    free(table);
    return 0;
}

/* Selected rows only: C and S are nrows x N (row r of the result is row rows[r]
 * of the product).  Used where the full product would take too long. */
int oracle_gemm_nt_rows(const uint16_t *A, const uint16_t *B, int64_t M, int64_t N,
                        int64_t K, int64_t lda, int64_t ldb, int dtype,
                        const int64_t *rows, int64_t nrows, double *C, double *S)
{
    if (M < 0 || N < 0 || K < 0 || lda < K || ldb < K || !C || (nrows > 0 && !rows))
        return -1;
    for (int64_t r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= M)
            return -1;
    double *table = (double *)malloc(65536 * sizeof(double));
    if (!table)
        return -1;
    if (fill_table(dtype, table)) {
        free(table);
        return -1;
    }
    /* Columns outermost so each row of B is streamed from memory once for all
     * the selected rows; every element is still one dot_one() in k order. */
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t j = 0; j < N; ++j) {
        for (int64_t r = 0; r < nrows; ++r) {
            const int64_t i = rows[r];
            double c, s;
            dot_one(table, A + i * lda, B + j * ldb, K, &c, &s);
            C[r * N + j] = c;
            if (S)
                S[r * N + j] = s;
        }
    }
    free(table);
    return 0;
}

/* Selected (i, j) points: C[p], S[p] for p < npts. */
int oracle_gemm_nt_points(const uint16_t *A, const uint16_t *B, int64_t M, int64_t N,
                          int64_t K, int64_t lda, int64_t ldb, int dtype,
                          const int64_t *ii, const int64_t *jj, int64_t npts, double *C,
                          double *S)
{
    if (M < 0 || N < 0 || K < 0 || lda < K || ldb < K || !C || (npts > 0 && (!ii || !jj)))
        return -1;
    for (int64_t p = 0; p < npts; ++p)
        if (ii[p] < 0 || ii[p] >= M || jj[p] < 0 || jj[p] >= N)
            return -1;
    double *table = (double *)malloc(65536 * sizeof(double));
    if (!table)
        return -1;
    if (fill_table(dtype, table)) {
        free(table);
        return -1;
    }
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < npts; ++p) {
        double c, s;
        dot_one(table, A + ii[p] * lda, B + jj[p] * ldb, K, &c, &s);
        C[p] = c;
        if (S)
            S[p] = s;
    }
    free(table);
    return 0;
}

/* Number of threads an OpenMP parallel region uses here (1 without OpenMP). */
int oracle_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}
