/*
 * Reference GEMM oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * This file is the plain, slow, obviously correct CPU definition of what the
 * GPU library computes.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load it.  The GPU library never links,
 * calls or includes anything from here, and this file includes nothing from
 * the GPU library.
 *
 * What it computes ("naive vs persistent matmul" post, Hugging Face activity
 * feed page: the MxK . KxN product, each output tile a sum-reduction across
 * K; Triton issue #1393 "Stream-k matmul implementation very slow...", final
 * revision: the accumulator is fp32 for fp16/bf16/fp32 inputs and the result
 * is checked against A @ B):
 *
 *     C[i][j] = sum_{k=0}^{K-1} a[i][k] * b[k][j]
 *     S[i][j] = sum_{k=0}^{K-1} |a[i][k]| * |b[k][j]|
 *
 * a and b are the input values exactly as stored (fp32, fp16 or bf16 bit
 * patterns, decoded here by hand, or two's-complement int8, whose products
 * the same revision accumulates in int32).  Every product and every partial
 * sum is an IEEE double, summed in ascending k.  Products of two
 * fp32/fp16/bf16 values have at most 48 significant bits, so each product is
 * exact in fp64 and the only rounding is in the sum (|error| <= (K-1) *
 * 2^-53 * S); int8 products are at most 2^14 in magnitude, so int8 sums are
 * exact integers for any K below 2^39.
 *
 * S is the scale used by the acceptance bound |C_gpu - C| <= tol * S.
 *
 * Layouts: A is M x K row-major, B is K x N row-major, C and S are M x N
 * row-major doubles.  Threads split output rows (full mode) or samples
 * (sampled mode); each output element is still one sequential loop, so the
 * result does not depend on the thread count.
 *
 * Parity pins: decoders against numpy over every 16-bit pattern; sums against
 * exact rational arithmetic on tiny shapes; identity, permutation,
 * small-integer, closed-form and scaling cases; sampled mode against full
 * mode.  See tests/test_oracle.py.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_F16 1
#define ORACLE_BF16 2
#define ORACLE_I8 3

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double decode_f16(uint16_t h)
{
    int sign = h >> 15;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);            /* subnormal: f * 2^(1-15-10) */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25); /* (1 + f/2^10) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits. */
static double decode_bf16(uint16_t b)
{
    int sign = b >> 15;
    int e = (b >> 7) & 0xff;
    int f = b & 0x7f;
    double v;
    if (e == 0)
        v = ldexp((double)f, -133);           /* subnormal: f * 2^(1-127-7) */
    else if (e == 255)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + f), e - 134); /* (1 + f/2^7) * 2^(e-127) */
    return sign ? -v : v;
}

/* IEEE binary32: 1 sign bit, 8 exponent bits (bias 127), 23 fraction bits. */
static double decode_f32(uint32_t u)
{
    int sign = u >> 31;
    int e = (u >> 23) & 0xff;
    int32_t f = (int32_t)(u & 0x7fffff);
    double v;
    if (e == 0)
        v = ldexp((double)f, -149);
    else if (e == 255)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(0x800000 + f), e - 150);
    return sign ? -v : v;
}

static double elem(int dtype, const void *p, int64_t idx)
{
    if (dtype == ORACLE_F32)
        return decode_f32(((const uint32_t *)p)[idx]);
    if (dtype == ORACLE_F16)
        return decode_f16(((const uint16_t *)p)[idx]);
    if (dtype == ORACLE_I8)
        return (double)((const int8_t *)p)[idx];
    return decode_bf16(((const uint16_t *)p)[idx]);
}

int oracle_decode_array(int dtype, const void *p, int64_t n, double *out)
{
    if (dtype < ORACLE_F32 || dtype > ORACLE_I8 || n < 0 || (n && (!p || !out)))
        return -1;
    for (int64_t i = 0; i < n; ++i)
        out[i] = elem(dtype, p, i);
    return 0;
}

/* ---------------------------------------------------------------- full mode */

typedef struct {
    int64_t M, N, K;
    const double *a;   /* M x K, decoded */
    const double *bt;  /* N x K, decoded, b transposed so column j is contiguous */
    double *C, *S;
    int64_t row_begin, row_end;
} full_job;

static void *full_worker(void *arg)
{
    full_job *jb = (full_job *)arg;
    for (int64_t i = jb->row_begin; i < jb->row_end; ++i) {
        const double *ai = jb->a + i * jb->K;
        for (int64_t j = 0; j < jb->N; ++j) {
            const double *bj = jb->bt + j * jb->K;
            double c = 0.0, s = 0.0;
            for (int64_t k = 0; k < jb->K; ++k) {
                c += ai[k] * bj[k];
                s += fabs(ai[k]) * fabs(bj[k]);
            }
            jb->C[i * jb->N + j] = c;
            if (jb->S)
                jb->S[i * jb->N + j] = s;
        }
    }
    return NULL;
}

int oracle_gemm_full(int dtype, int64_t M, int64_t N, int64_t K, const void *A, const void *B,
                     double *C, double *S, int nthreads)
{
    if (dtype < ORACLE_F32 || dtype > ORACLE_I8 || M < 0 || N < 0 || K < 0 || !C)
        return -1;
    if (M == 0 || N == 0)
        return 0;
    if (nthreads < 1)
        nthreads = 1;
    double *a = (double *)malloc(sizeof(double) * (size_t)(M * K > 0 ? M * K : 1));
    double *bt = (double *)malloc(sizeof(double) * (size_t)(N * K > 0 ? N * K : 1));
    if (!a || !bt) {
        free(a);
        free(bt);
        return -2;
    }
    for (int64_t i = 0; i < M; ++i)
        for (int64_t k = 0; k < K; ++k)
            a[i * K + k] = elem(dtype, A, i * K + k);
    for (int64_t k = 0; k < K; ++k)
        for (int64_t j = 0; j < N; ++j)
            bt[j * K + k] = elem(dtype, B, k * N + j);

    if (nthreads > M)
        nthreads = (int)M;
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    full_job *jobs = (full_job *)calloc((size_t)nthreads, sizeof(full_job));
    int rc = 0;
    for (int t = 0; t < nthreads; ++t) {
        full_job jb = {M, N, K, a, bt, C, S, M * t / nthreads, M * (t + 1) / nthreads};
        jobs[t] = jb;
        if (pthread_create(&th[t], NULL, full_worker, &jobs[t]) != 0) {
            full_worker(&jobs[t]);
            th[t] = 0;
        }
    }
    for (int t = 0; t < nthreads; ++t)
        if (th[t])
            pthread_join(th[t], NULL);
    free(th);
    free(jobs);
    free(a);
    free(bt);
    return rc;
}

/* ------------------------------------------------------------- sampled mode */

typedef struct {
    int dtype;
    int64_t N, K;
    const void *A, *B;
    const int64_t *rows, *cols;
    double *C, *S;
    int64_t begin, end;
} sample_job;

static void *sample_worker(void *arg)
{
    sample_job *jb = (sample_job *)arg;
    for (int64_t s = jb->begin; s < jb->end; ++s) {
        int64_t i = jb->rows[s], j = jb->cols[s];
        double c = 0.0, sc = 0.0;
        for (int64_t k = 0; k < jb->K; ++k) {
            double a = elem(jb->dtype, jb->A, i * jb->K + k);
            double b = elem(jb->dtype, jb->B, k * jb->N + j);
            c += a * b;
            sc += fabs(a) * fabs(b);
        }
        jb->C[s] = c;
        if (jb->S)
            jb->S[s] = sc;
    }
    return NULL;
}

/* C[s] (and S[s]) for the output element (rows[s], cols[s]), s < n. */
int oracle_gemm_sampled(int dtype, int64_t M, int64_t N, int64_t K, const void *A, const void *B,
                        int64_t n, const int64_t *rows, const int64_t *cols, double *C, double *S,
                        int nthreads)
{
    if (dtype < ORACLE_F32 || dtype > ORACLE_I8 || M < 0 || N < 0 || K < 0 || n < 0)
        return -1;
    if (n == 0)
        return 0;
    if (!rows || !cols || !C)
        return -1;
    for (int64_t s = 0; s < n; ++s)
        if (rows[s] < 0 || rows[s] >= M || cols[s] < 0 || cols[s] >= N)
            return -3;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > n)
        nthreads = (int)n;
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    sample_job *jobs = (sample_job *)calloc((size_t)nthreads, sizeof(sample_job));
    for (int t = 0; t < nthreads; ++t) {
        sample_job jb = {dtype, N, K, A, B, rows, cols, C, S, n * t / nthreads, n * (t + 1) / nthreads};
        jobs[t] = jb;
        if (pthread_create(&th[t], NULL, sample_worker, &jobs[t]) != 0) {
            sample_worker(&jobs[t]);
            th[t] = 0;
        }
    }
    for (int t = 0; t < nthreads; ++t)
        if (th[t])
            pthread_join(th[t], NULL);
    free(th);
    free(jobs);
    return 0;
}
