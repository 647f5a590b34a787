/*
 * oracle.c -- CPU reference for the small-M bf16 "skinny" GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: it is used by the tests, by the smoke check and by the
 * bench's CPU-baseline leg, and by nothing else.  It shares no code, header
 * or constant with the HIP library.
 *
 * What it computes (plain definition, no blocking, no fusion, no reordering):
 *
 *     C[m, n] = sum_{k = 0 .. K-1} dec(A[m, k]) * dec(B[n, k])
 *
 * with A an M x K and B an N x K row-major bf16 matrix, i.e. C = A . B^T.
 *   - PR #42562 page ("Add generic cuteDSL LL BF16 router (GEMM)"),
 *     section 实现拆解 items 1-2 and the _ll_bf16_dotprod.py excerpt under
 *     关键源码片段: the dot-product kernel loads B and A, widens both to
 *     fp32 and accumulates acc[m] += a * b per token m; the split-K kernel
 *     splits the same sum over K.  The tests of that PR compare against a
 *     plain PyTorch matmul reference.
 *   - PR #48597 page ("GLM-5.2 Blackwell decode optimizations"), section
 *     实现拆解 item 3: bf16 A and B for the decode projections.
 *
 * The sum is taken in IEEE binary64, in ascending k.  A bf16 x bf16 product
 * has at most 16 significant bits, so each product is exact in binary64;
 * only the additions round (relative error bounded by K * 2^-53).
 *
 * dec(h): a bf16 value is the upper half of an IEEE binary32 word, so the
 * decode places the 16 stored bits in the high half of a 32-bit word and
 * reinterprets it (exact; widened to binary64 without rounding).
 *
 * The same sum with binary32 weights W[n, k] in place of dec(B[n, k])
 * (oracle_gemm_f32w_f64, oracle_gemm_f32w_f64_points): the router GEMM over
 * weights kept in fp32.  The PR #48597 page names such a router GEMM, and the
 * keeping of the router weights in fp32, among the parts of that PR (section
 * 关联脉络) without printing any of it; the reading taken is the same
 * product C = A . W^T with W read as binary32.  A bf16 x binary32
 * product has at most 8 + 24 significant bits, so it is exact in binary64
 * too, and again only the additions round.
 *
 * oracle_round_bf16: binary64 -> bf16 round-to-nearest, ties-to-even, via
 * scaling by the quantum of the value's binade and rint().  Used only to
 * predict bf16 outputs in cases where the fp32 result is exact.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static double dec_bf16(uint16_t h)
{
    uint32_t w = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

double oracle_bf16_decode(uint16_t h) { return dec_bf16(h); }

/*
 * C[m*ldc + n] (binary64) for m < M, n < N.  A is read at A[m*lda + k],
 * B at B[n*ldb + k], k < K.  Returns 0, or -1 on bad arguments.
 * nthreads > 1 splits the independent columns n across OpenMP threads; each
 * C[m, n] is still one sequential loop over k.
 */
int oracle_gemm_f64(const uint16_t *A, const uint16_t *B, double *C,
                    int M, int N, int K, int64_t lda, int64_t ldb,
                    int64_t ldc, int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || lda < K || ldb < K || ldc < N)
        return -1;
    if (nthreads < 1)
        nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (int n = 0; n < N; ++n) {
        for (int m = 0; m < M; ++m) {
            double s = 0.0;
            for (int k = 0; k < K; ++k)
                s += dec_bf16(A[(int64_t)m * lda + k]) *
                     dec_bf16(B[(int64_t)n * ldb + k]);
            C[(int64_t)m * ldc + n] = s;
        }
    }
    return 0;
}

/*
 * Same sum for an explicit list of (m, n) pairs: out[i] = C[ms[i], ns[i]].
 * Used to check sampled outputs of the largest shapes one by one.
 */
int oracle_gemm_f64_points(const uint16_t *A, const uint16_t *B, int K,
                           int64_t lda, int64_t ldb, const int *ms,
                           const int *ns, int npts, double *out, int nthreads)
{
    if (K < 0 || lda < K || ldb < K || npts < 0)
        return -1;
    if (nthreads < 1)
        nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (int i = 0; i < npts; ++i) {
        double s = 0.0;
        for (int k = 0; k < K; ++k)
            s += dec_bf16(A[(int64_t)ms[i] * lda + k]) *
                 dec_bf16(B[(int64_t)ns[i] * ldb + k]);
        out[i] = s;
    }
    return 0;
}

/*
 * C[m*ldc + n] = sum_k dec(A[m*lda + k]) * W[n*ldw + k] (binary64, k
 * ascending), W binary32.  Returns 0, or -1 on bad arguments.
 */
int oracle_gemm_f32w_f64(const uint16_t *A, const float *W, double *C,
                         int M, int N, int K, int64_t lda, int64_t ldw,
                         int64_t ldc, int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || lda < K || ldw < K || ldc < N)
        return -1;
    if (nthreads < 1)
        nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (int n = 0; n < N; ++n) {
        for (int m = 0; m < M; ++m) {
            double s = 0.0;
            for (int k = 0; k < K; ++k)
                s += dec_bf16(A[(int64_t)m * lda + k]) *
                     (double)W[(int64_t)n * ldw + k];
            C[(int64_t)m * ldc + n] = s;
        }
    }
    return 0;
}

/* The same for an explicit list of (m, n) pairs: out[i] = C[ms[i], ns[i]]. */
int oracle_gemm_f32w_f64_points(const uint16_t *A, const float *W, int K,
                                int64_t lda, int64_t ldw, const int *ms,
                                const int *ns, int npts, double *out,
                                int nthreads)
{
    if (K < 0 || lda < K || ldw < K || npts < 0)
        return -1;
    if (nthreads < 1)
        nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (int i = 0; i < npts; ++i) {
        double s = 0.0;
        for (int k = 0; k < K; ++k)
            s += dec_bf16(A[(int64_t)ms[i] * lda + k]) *
                 (double)W[(int64_t)ns[i] * ldw + k];
        out[i] = s;
    }
    return 0;
}

/*
 * Nearest bf16 to x, ties to even; returns the 16-bit pattern.
 * bf16 keeps 8 significant bits (7 stored) and binary32's exponent range:
 * normal binades [2^e, 2^(e+1)) for e >= -126 have quantum 2^(e-7); below
 * 2^-126 the quantum stays 2^-133 (subnormals).  A result of 2^128 or more
 * is +-infinity.  NaN maps to the canonical quiet NaN with x's sign.
 */
uint16_t oracle_round_bf16(double x)
{
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x))
        return (uint16_t)(sign | 0x7FC0u);
    double a = fabs(x);
    if (isinf(a))
        return (uint16_t)(sign | 0x7F80u);
    if (a == 0.0)
        return sign;
    int E;
    (void)frexp(a, &E); /* a = f * 2^E, f in [0.5, 1) => binade exponent E-1 */
    int e = E - 1;
    if (e < -126)
        e = -126;
    double q = ldexp(1.0, e - 7);
    double r = rint(a / q) * q; /* rint: nearest, ties to even (default mode) */
    if (r >= ldexp(1.0, 128))
        return (uint16_t)(sign | 0x7F80u);
    float f = (float)r; /* exact: r is a bf16 value */
    uint32_t w;
    memcpy(&w, &f, sizeof w);
    return (uint16_t)(sign | (uint16_t)(w >> 16));
}
