/*
 * CPU oracle for the W4A16 GEMM -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load this library. The product path (the HIP library) never calls it and
 * shares no code with it.
 *
 * What it computes is the plain definition, in double precision:
 *
 *   w[k][n] = (q[k][n] - z[k/G][n]) * s[k/G][n]
 *   Y[m][n] = sum over k = 0 .. K-1, in increasing k, of X[m][k] * w[k][n]
 *
 * The dequantization formula is the one in "LMDeploy Guide: Fast
 * Mixed-Precision LLM Inference Engine", section 3 "Instruction-Level
 * Parallelism (ILP) for Zero-Overhead Dequantization" (FP16 = (INT4 -
 * ZeroPoint) x Scale). Groups of G consecutive rows along K share one scale
 * and one zero per output column ("LMDeploy, in depth", section
 * "Quantization: AWQ weights and KV cache": 4-bit weights in groups of 128
 * with a scale per group; the axis is this oracle's reading). The product is
 * an ordinary matmul of 16-bit activations with the dequantized weights
 * ("LMDeploy" interview notes, answer to why W4A16 raises throughput
 * although FLOPs do not change: dequantize, then multiply in FP16).
 *
 * The subtraction of the integer zero happens before the scale. (q - z) is an
 * integer in [-15, 15] and s is an fp16 value, so w is exact in double; the
 * products X * w are exact too (11 + 11 + 4 significant bits), so the only
 * rounding is in the running sum. Compile with -ffp-contract=off so that the
 * sum is the plain "acc = acc + x * w" in increasing k.
 *
 * fp16 values arrive as raw IEEE binary16 bit patterns (uint16) and are
 * decoded here from the format's definition.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int f = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24); /* subnormal: f * 2^-24 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25); /* (1 + f/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* Returns 0 on success, -1 if any code is outside 0..15, -2 on bad shape. */
static int check_args(const uint8_t *q, const uint8_t *z, int64_t K, int64_t N, int64_t G)
{
    if (K <= 0 || N <= 0 || G <= 0 || K % G)
        return -2;
    for (int64_t i = 0; i < K * N; ++i)
        if (q[i] > 15)
            return -1;
    for (int64_t i = 0; i < (K / G) * N; ++i)
        if (z[i] > 15)
            return -1;
    return 0;
}

/* W[k][n] (K x N doubles) = (q[k][n] - z[k/G][n]) * s[k/G][n]. */
int oracle_dequant(const uint8_t *q, const uint8_t *z, const uint16_t *s,
                   int64_t K, int64_t N, int64_t G, double *W)
{
    int rc = check_args(q, z, K, N, G);
    if (rc)
        return rc;
    for (int64_t k = 0; k < K; ++k) {
        int64_t g = k / G;
        for (int64_t n = 0; n < N; ++n) {
            int diff = (int)q[k * N + n] - (int)z[g * N + n];
            W[k * N + n] = (double)diff * oracle_half_to_double(s[g * N + n]);
        }
    }
    return 0;
}

/*
 * Y (M x (n1 - n0) doubles, row-major) = X[M][K] . W[K][n0:n1].
 * Columns are split into blocks across OpenMP threads; each output element
 * is still summed by one thread in increasing k. nthreads <= 0 means the
 * OpenMP default.
 */
int oracle_gemm(const uint16_t *X, const uint8_t *q, const uint8_t *z, const uint16_t *s,
                int64_t M, int64_t N, int64_t K, int64_t G, int64_t n0, int64_t n1,
                double *Y, int nthreads)
{
    int rc = check_args(q, z, K, N, G);
    if (rc)
        return rc;
    if (M <= 0 || n0 < 0 || n1 > N || n0 >= n1)
        return -2;
    const int64_t NC = n1 - n0;
    double *Xd = (double *)malloc(sizeof(double) * (size_t)(M * K));
    if (!Xd)
        return -3;
    for (int64_t i = 0; i < M * K; ++i)
        Xd[i] = oracle_half_to_double(X[i]);

    const int64_t NB = 64; /* columns per work item */
    const int64_t nblocks = (NC + NB - 1) / NB;
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int64_t blk = 0; blk < nblocks; ++blk) {
        const int64_t c0 = n0 + blk * NB;
        const int64_t c1 = c0 + NB < n1 ? c0 + NB : n1;
        const int64_t w = c1 - c0;
        double *acc = (double *)calloc((size_t)(M * w), sizeof(double));
        double *wrow = (double *)malloc(sizeof(double) * (size_t)w);
        for (int64_t k = 0; k < K; ++k) {
            const int64_t g = k / G;
            for (int64_t j = 0; j < w; ++j) {
                const int64_t n = c0 + j;
                int diff = (int)q[k * N + n] - (int)z[g * N + n];
                wrow[j] = (double)diff * oracle_half_to_double(s[g * N + n]);
            }
            for (int64_t m = 0; m < M; ++m) {
                const double xm = Xd[m * K + k];
                double *am = acc + m * w;
                for (int64_t j = 0; j < w; ++j)
                    am[j] = am[j] + xm * wrow[j];
            }
        }
        for (int64_t m = 0; m < M; ++m)
            memcpy(Y + m * NC + (c0 - n0), acc + m * w, sizeof(double) * (size_t)w);
        free(wrow);
        free(acc);
    }
    free(Xd);
    return 0;
}

/* Threads OpenMP would use by default (1 when built without OpenMP). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
