/*
 * CPU oracle for the dense GEMM and fully-connected-layer hot path.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may link, load or
 * call this file: only the tests, the package's smoke check and the bench's
 * CPU-baseline leg use it. It shares no code, header, table or helper with
 * the HIP kernels.
 *
 * What it computes (float64 throughout, k summed in increasing order):
 *
 *   GEMM (fp32, binary16 or bfloat16 inputs), page "GEMM 优化详解" (GEMM
 *   optimisation in detail), section "GEMM 基础理论 / 数学定义"
 *   (mathematical definition): the full form is
 *   C = alpha*A*B + beta*C, with A M-by-K, B K-by-N, C M-by-N and
 *   C(m,n) = sum over k of A(m,k)*B(k,n). Page "第5章-基础Kernel" section 1.1
 *   gives the same sum with k running from 0 to K-1, and its section 7.1
 *   gives a CPU triple loop (which accumulates in float; the oracle
 *   accumulates in float64 instead, so it is the reference the GPU is held to).
 *
 *   Fully-connected layer, page "GEMM 优化详解", table "为什么 GEMM 重要"
 *   (FC layer Y = X*W + b) and section "Level 6: Kernel Fusion": the fused
 *   output is ReLU(X*W + bias) with the bias indexed by output column and the
 *   bias added before the ReLU.
 *
 * Readings where the pages leave a step open:
 *   - beta == 0 means C is not read (so NaN in C does not propagate);
 *     alpha == 0 (or K == 0) means the result is beta*C and A, B are not read.
 *   - ReLU returns +0.0 for y <= 0.
 *   - Every product of two fp32 (24-bit), binary16 (11-bit) or bfloat16
 *     (8-bit) significands is exact in a double, so only the additions round;
 *     no fast-math may be used to build this file, because reassociating k
 *     changes the result.
 *
 * B (or W) is K-by-N, or, with b_trans (w_trans) set, stored N-by-K so that
 * element (k, n) is at B[n*ldb + k] (the product is then A*B^T, X*W^T).
 *
 * Besides the value r, every routine returns t = sum over k of |A(m,k)*B(k,n)|,
 * which is the basis of the parity tolerance |C_gpu - r| <= 1e-4 * t.
 *
 * Blocking: the full-matrix routines first decode A and B to double (exact for
 * every input format; B into K-by-N order), then split the output over row
 * blocks and column blocks for cache reuse and threads and walk k in chunks
 * within a block, but each element still receives its products in increasing
 * k, so the result is bitwise that of the plain triple loop.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* IEEE 754 binary16 to double, from the format's definition: 1 sign bit,
 * 5 exponent bits (bias 15), 10 fraction bits; exponent 0 is subnormal
 * (f * 2^-24), exponent 31 is infinity (f == 0) or NaN. */
double oracle_half_to_double(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int e = (h >> 10) & 0x1f;
    const int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(f + 1024), e - 25);
    return sign ? -v : v;
}

/* bfloat16 to double, from the format's definition: 1 sign bit, 8 exponent
 * bits (bias 127), 7 fraction bits; exponent 0 is subnormal (f * 2^-133),
 * exponent 255 is infinity (f == 0) or NaN. */
double oracle_bf16_to_double(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int e = (h >> 7) & 0xff;
    const int f = h & 0x7f;
    double v;
    if (e == 0)
        v = ldexp((double)f, -133);
    else if (e == 255)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(f + 128), e - 134);
    return sign ? -v : v;
}

static inline double ld_f32(const void *p, int64_t i) { return (double)((const float *)p)[i]; }
static inline double ld_bf16(const void *p, int64_t i) { return oracle_bf16_to_double(((const uint16_t *)p)[i]); }
static inline double ld_f16(const void *p, int64_t i) { return oracle_half_to_double(((const uint16_t *)p)[i]); }

typedef double (*loader_fn)(const void *, int64_t);

enum { EPI_GEMM = 0, EPI_LINEAR = 1 };

typedef struct {
    int kind;            /* EPI_GEMM or EPI_LINEAR */
    double alpha, beta;  /* gemm */
    const float *cin;    /* gemm, read only when beta != 0 */
    int64_t ldc;
    const float *bias;   /* linear, may be NULL */
    int act;             /* linear: 0 none, 1 ReLU */
} epilogue_t;

static void set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* The epilogue applied to one element once its sum s over k is known. */
static inline double finish(const epilogue_t *e, int64_t m, int64_t n, double s)
{
    if (e->kind == EPI_GEMM) {
        double r = e->alpha * s;
        if (e->beta != 0.0)
            r += e->beta * (double)e->cin[m * e->ldc + n];
        return r;
    }
    double y = s;
    if (e->bias)
        y += (double)e->bias[n];
    if (e->act == 1)
        y = (y > 0.0) ? y : 0.0;
    return y;
}

/* Whether the sum over k is needed at all (gemm with alpha == 0 skips it). */
static inline int needs_sum(const epilogue_t *e)
{
    return !(e->kind == EPI_GEMM && e->alpha == 0.0);
}

#define NB 64 /* output columns per block */
#define MB 16 /* output rows per block */
#define KB 256 /* k values per chunk of a block */

/* A (M-by-K) decoded to double, row-major with leading dimension K. Every
 * input format converts to double exactly, so the decoded operands are the
 * values of the definition themselves. */
static double *decode_a(int64_t M, int64_t K, const void *A, int64_t lda, loader_fn la)
{
    double *Ad = malloc((size_t)(M * K > 0 ? M * K : 1) * sizeof(double));
    if (!Ad)
        abort();
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k)
            Ad[m * K + k] = la(A, m * lda + k);
    return Ad;
}

/* B decoded to double in K-by-N order (leading dimension N), whether it is
 * stored K-by-N or, with b_trans, N-by-K. */
static double *decode_b(int64_t K, int64_t N, const void *B, int64_t ldb, loader_fn lb, int b_trans)
{
    double *Bd = malloc((size_t)(K * N > 0 ? K * N : 1) * sizeof(double));
    if (!Bd)
        abort();
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < K; ++k)
        for (int64_t col = 0; col < N; ++col)
            Bd[k * N + col] = lb(B, b_trans ? col * ldb + k : k * ldb + col);
    return Bd;
}

/* Full M-by-N result into R (row-major, ld N) and T (same layout). */
static void full_product(int64_t M, int64_t N, int64_t K,
                         const void *A, int64_t lda, loader_fn la,
                         const void *B, int64_t ldb, loader_fn lb, int b_trans,
                         const epilogue_t *e, double *R, double *T, int nthreads)
{
    if (M <= 0 || N <= 0)
        return;
    set_threads(nthreads);
    const int sum = needs_sum(e) && K > 0;
    double *Ad = sum ? decode_a(M, K, A, lda, la) : NULL;
    double *Bd = sum ? decode_b(K, N, B, ldb, lb, b_trans) : NULL;
    const int64_t nmb = (M + MB - 1) / MB, nnb = (N + NB - 1) / NB;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t task = 0; task < nmb * nnb; ++task) {
        const int64_t n0 = (task % nnb) * NB, m0 = (task / nnb) * MB;
        const int64_t nb = (N - n0 < NB) ? N - n0 : NB;
        const int64_t mb = (M - m0 < MB) ? M - m0 : MB;
        double s[MB][NB], t[MB][NB];
        for (int64_t i = 0; i < mb; ++i)
            for (int64_t j = 0; j < nb; ++j) {
                s[i][j] = 0.0;
                t[i][j] = 0.0;
            }
        /* k in chunks of KB, each chunk over every row of the block: every
         * element still receives its products in increasing k */
        for (int64_t k0 = 0; sum && k0 < K; k0 += KB) {
            const int64_t k1 = (K - k0 < KB) ? K : k0 + KB;
            for (int64_t i = 0; i < mb; ++i) {
                const int64_t m = m0 + i;
                for (int64_t k = k0; k < k1; ++k) {
                    const double a = Ad[m * K + k];
                    const double *brow = Bd + k * N + n0;
                    for (int64_t j = 0; j < nb; ++j) {
                        const double p = a * brow[j];
                        s[i][j] += p;
                        t[i][j] += fabs(p);
                    }
                }
            }
        }
        for (int64_t i = 0; i < mb; ++i)
            for (int64_t j = 0; j < nb; ++j) {
                R[(m0 + i) * N + n0 + j] = finish(e, m0 + i, n0 + j, s[i][j]);
                T[(m0 + i) * N + n0 + j] = t[i][j];
            }
    }
    free(Ad);
    free(Bd);
}

/* Selected elements (rows[p], cols[p]): each is one plain dot product over k. */
static void sampled_product(int64_t K, const void *A, int64_t lda, loader_fn la,
                            const void *B, int64_t ldb, loader_fn lb, int b_trans,
                            const epilogue_t *e, int64_t P, const int64_t *rows,
                            const int64_t *cols, double *R, double *T, int nthreads)
{
    set_threads(nthreads);
    const int sum = needs_sum(e);
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t p = 0; p < P; ++p) {
        const int64_t m = rows[p], n = cols[p];
        double s = 0.0, t = 0.0;
        if (sum) {
            for (int64_t k = 0; k < K; ++k) {
                const double prod = la(A, m * lda + k) * lb(B, b_trans ? n * ldb + k : k * ldb + n);
                s += prod;
                t += fabs(prod);
            }
        }
        R[p] = finish(e, m, n, s);
        T[p] = t;
    }
}

static epilogue_t gemm_epi(double alpha, double beta, const float *cin, int64_t ldc)
{
    epilogue_t e;
    memset(&e, 0, sizeof e);
    e.kind = EPI_GEMM;
    e.alpha = alpha;
    e.beta = beta;
    e.cin = cin;
    e.ldc = ldc;
    return e;
}

static epilogue_t linear_epi(const float *bias, int act)
{
    epilogue_t e;
    memset(&e, 0, sizeof e);
    e.kind = EPI_LINEAR;
    e.bias = bias;
    e.act = act;
    return e;
}

/* ---- exported entry points (called from Python through ctypes) ---- */

/* C = alpha*A*B + beta*Cin with fp32 A, B, Cin; results in float64. */
void oracle_gemm_f32(int64_t M, int64_t N, int64_t K, double alpha,
                     const float *A, int64_t lda, const float *B, int64_t ldb, int b_trans,
                     double beta, const float *Cin, int64_t ldc,
                     double *R, double *T, int nthreads)
{
    epilogue_t e = gemm_epi(alpha, beta, Cin, ldc);
    full_product(M, N, K, A, lda, ld_f32, B, ldb, ld_f32, b_trans, &e, R, T, nthreads);
}

/* As oracle_gemm_f32 but A and B hold IEEE binary16 bit patterns. */
void oracle_gemm_f16(int64_t M, int64_t N, int64_t K, double alpha,
                     const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb, int b_trans,
                     double beta, const float *Cin, int64_t ldc,
                     double *R, double *T, int nthreads)
{
    epilogue_t e = gemm_epi(alpha, beta, Cin, ldc);
    full_product(M, N, K, A, lda, ld_f16, B, ldb, ld_f16, b_trans, &e, R, T, nthreads);
}

/* As oracle_gemm_f32 but A and B hold bfloat16 bit patterns. */
void oracle_gemm_bf16(int64_t M, int64_t N, int64_t K, double alpha,
                      const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb, int b_trans,
                      double beta, const float *Cin, int64_t ldc,
                      double *R, double *T, int nthreads)
{
    epilogue_t e = gemm_epi(alpha, beta, Cin, ldc);
    full_product(M, N, K, A, lda, ld_bf16, B, ldb, ld_bf16, b_trans, &e, R, T, nthreads);
}

/* Y = act(X*W + bias); bias may be NULL; act 0 = none, 1 = ReLU. */
void oracle_linear(int64_t M, int64_t N, int64_t K,
                   const float *X, int64_t ldx, const float *W, int64_t ldw, int w_trans,
                   const float *bias, int act, double *R, double *T, int nthreads)
{
    epilogue_t e = linear_epi(bias, act);
    full_product(M, N, K, X, ldx, ld_f32, W, ldw, ld_f32, w_trans, &e, R, T, nthreads);
}

void oracle_gemm_f32_at(int64_t K, double alpha, const float *A, int64_t lda,
                        const float *B, int64_t ldb, int b_trans, double beta, const float *Cin,
                        int64_t ldc, int64_t P, const int64_t *rows, const int64_t *cols,
                        double *R, double *T, int nthreads)
{
    epilogue_t e = gemm_epi(alpha, beta, Cin, ldc);
    sampled_product(K, A, lda, ld_f32, B, ldb, ld_f32, b_trans, &e, P, rows, cols, R, T, nthreads);
}

void oracle_gemm_f16_at(int64_t K, double alpha, const uint16_t *A, int64_t lda,
                        const uint16_t *B, int64_t ldb, int b_trans, double beta, const float *Cin,
                        int64_t ldc, int64_t P, const int64_t *rows, const int64_t *cols,
                        double *R, double *T, int nthreads)
{
    epilogue_t e = gemm_epi(alpha, beta, Cin, ldc);
    sampled_product(K, A, lda, ld_f16, B, ldb, ld_f16, b_trans, &e, P, rows, cols, R, T, nthreads);
}

void oracle_gemm_bf16_at(int64_t K, double alpha, const uint16_t *A, int64_t lda,
                         const uint16_t *B, int64_t ldb, int b_trans, double beta, const float *Cin,
                         int64_t ldc, int64_t P, const int64_t *rows, const int64_t *cols,
                         double *R, double *T, int nthreads)
{
    epilogue_t e = gemm_epi(alpha, beta, Cin, ldc);
    sampled_product(K, A, lda, ld_bf16, B, ldb, ld_bf16, b_trans, &e, P, rows, cols, R, T, nthreads);
}

void oracle_linear_at(int64_t K, const float *X, int64_t ldx, const float *W, int64_t ldw,
                      int w_trans, const float *bias, int act, int64_t P, const int64_t *rows,
                      const int64_t *cols, double *R, double *T, int nthreads)
{
    epilogue_t e = linear_epi(bias, act);
    sampled_product(K, X, ldx, ld_f32, W, ldw, ld_f32, w_trans, &e, P, rows, cols, R, T, nthreads);
}
