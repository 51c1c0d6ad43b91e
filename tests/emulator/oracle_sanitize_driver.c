/* Drives the oracle's entry points under AddressSanitizer and
 * UndefinedBehaviorSanitizer (test infrastructure): ragged tiny shapes, every
 * dtype, one and several threads, sampled mode against full mode bitwise.
 * Exit status 0 means every call returned 0 and every comparison held; a
 * sanitizer finding aborts with a non-zero status. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_gemm_full(int dtype, int64_t M, int64_t N, int64_t K, const void *A, const void *B,
                     double *C, double *S, int nthreads);
int oracle_gemm_sampled(int dtype, int64_t M, int64_t N, int64_t K, const void *A, const void *B,
                        int64_t n, const int64_t *rows, const int64_t *cols, double *C, double *S,
                        int nthreads);

static uint32_t rng = 12345u;
static uint32_t next(void)
{
    rng = rng * 1664525u + 1013904223u;
    return rng >> 8;
}

int main(void)
{
    const int64_t shapes[][3] = {{1, 1, 1}, {3, 5, 7}, {17, 9, 33}, {64, 40, 130}, {5, 70, 1}};
    for (int dt = 0; dt < 3; ++dt)
        for (size_t si = 0; si < sizeof shapes / sizeof shapes[0]; ++si) {
            const int64_t M = shapes[si][0], N = shapes[si][1], K = shapes[si][2];
            const size_t e = dt == 0 ? 4 : 2;
            unsigned char *A = malloc((size_t)(M * K) * e), *B = malloc((size_t)(K * N) * e);
            for (int64_t i = 0; i < M * K; ++i) {
                uint32_t v = next();
                /* finite values: clear the top exponent bit of each pattern */
                if (e == 4) { v &= 0xBFFFFFFFu; memcpy(A + 4 * i, &v, 4); }
                else { uint16_t h = (uint16_t)(v & 0xBFFF); memcpy(A + 2 * i, &h, 2); }
            }
            for (int64_t i = 0; i < K * N; ++i) {
                uint32_t v = next();
                if (e == 4) { v &= 0xBFFFFFFFu; memcpy(B + 4 * i, &v, 4); }
                else { uint16_t h = (uint16_t)(v & 0xBFFF); memcpy(B + 2 * i, &h, 2); }
            }
            double *C1 = malloc(sizeof(double) * (size_t)(M * N));
            double *S1 = malloc(sizeof(double) * (size_t)(M * N));
            double *C3 = malloc(sizeof(double) * (size_t)(M * N));
            double *S3 = malloc(sizeof(double) * (size_t)(M * N));
            if (oracle_gemm_full(dt, M, N, K, A, B, C1, S1, 1) ||
                oracle_gemm_full(dt, M, N, K, A, B, C3, S3, 3))
                return 1;
            if (memcmp(C1, C3, sizeof(double) * (size_t)(M * N)) ||
                memcmp(S1, S3, sizeof(double) * (size_t)(M * N)))
                return 2;
            const int64_t n = M * N;
            int64_t *rows = malloc(sizeof(int64_t) * (size_t)n), *cols = malloc(sizeof(int64_t) * (size_t)n);
            for (int64_t s = 0; s < n; ++s) {
                rows[s] = s / N;
                cols[s] = s % N;
            }
            double *Cs = malloc(sizeof(double) * (size_t)n), *Ss = malloc(sizeof(double) * (size_t)n);
            if (oracle_gemm_sampled(dt, M, N, K, A, B, n, rows, cols, Cs, Ss, 2))
                return 3;
            if (memcmp(Cs, C1, sizeof(double) * (size_t)n) || memcmp(Ss, S1, sizeof(double) * (size_t)n))
                return 4;
            free(A); free(B); free(C1); free(S1); free(C3); free(S3);
            free(rows); free(cols); free(Cs); free(Ss);
        }
    /* argument checks: bad dtype, out-of-range sample */
    double c, s;
    int64_t r = 5, k = 0;
    if (oracle_gemm_full(7, 1, 1, 1, &c, &c, &c, &s, 1) == 0)
        return 5;
    if (oracle_gemm_sampled(0, 2, 2, 1, &c, &c, 1, &r, &k, &c, &s, 1) == 0)
        return 6;
    puts("ok");
    return 0;
}
