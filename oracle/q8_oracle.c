/*
 * q8_oracle.c -- plain, slow CPU oracle for Q8_0 weight-only GEMV.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or
 * call this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg do. It shares no code, header or table with the HIP
 * library.
 *
 * What it computes (the plain definition, nothing approximated):
 *   Q8_0 block = one fp16 scale d followed by 32 int8 quants q; the weight
 *   is d*q. This is the GGUF Q8_0 format that memra decodes and runs through
 *   its decode matvecs (memra wiki, feature list: the NVFP4/Q4_0/Q8_0
 *   decode item and the loaders item; topairepos memra listing, crate
 *   table row memra-gguf).
 *   y[n][m] = sum_{k=0}^{K-1} (d[m][k/32] * q[m][k]) * x[n][k]
 *   A[n][m] = sum_{k=0}^{K-1} |d[m][k/32] * q[m][k] * x[n][k]|
 *
 * Arithmetic: every term is formed exactly in fp64 (d*q needs 11+8 bits,
 * times an fp16 x another 11 bits: 30 bits < 53), and the terms are summed
 * sequentially in increasing k, so the only rounding is that of the running
 * sum: |y_fp64 - y_exact| <= (K-1) * 2^-53 * A. Build with
 * -ffp-contract=off and no fast-math so no fused or reordered operation
 * changes that.
 *
 * fp16 decoding is written out from the IEEE 754 binary16 definition
 * (1 sign bit, 5 exponent bits with bias 15, 10 fraction bits; exponent 0
 * means subnormal 0.f * 2^-14) and handles subnormals and signed zeros.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_QK 32

double or_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24); /* 0.f * 2^-14 = f * 2^-24 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25); /* 1.f * 2^(e-15) */
    return sign ? -v : v;
}

/* Decode GGUF Q8_0 blocks: blk is M rows of K/32 blocks of 34 bytes
 * (little-endian fp16 scale, then 32 int8). Writes q [M][K] and the scale
 * bit patterns d [M][K/32]. Returns 0, or -1 if K is not a multiple of 32. */
int or_decode_blocks(const uint8_t *blk, int64_t M, int64_t K, int8_t *q, uint16_t *d)
{
    if (K % OR_QK)
        return -1;
    int64_t nb = K / OR_QK;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t *p = blk + (m * nb + b) * (2 + OR_QK);
            d[m * nb + b] = (uint16_t)(p[0] | (p[1] << 8));
            for (int i = 0; i < OR_QK; ++i)
                q[m * K + b * OR_QK + i] = (int8_t)p[2 + i];
        }
    }
    return 0;
}

/* One output: token row xn (fp16 bits or fp32 values), weight row m. */
static void dot_row(const int8_t *qrow, const uint16_t *drow, int64_t K,
                    const uint16_t *x16, const float *x32, double *y, double *a)
{
    double s = 0.0, t = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double w = or_half_to_double(drow[k / OR_QK]) * (double)qrow[k];
        double xv = x16 ? or_half_to_double(x16[k]) : (double)x32[k];
        double p = w * xv;
        s = s + p;
        t = t + fabs(p);
    }
    *y = s;
    *a = t;
}

typedef struct {
    const int8_t *q;
    const uint16_t *d;
    int64_t K, ldq, ldd;
    const uint16_t *x16;
    const float *x32;
    int64_t N, ldx;
    const int64_t *rows; /* NULL: rows r0..r1-1 are all rows */
    int64_t R;           /* number of output columns (rows or sampled rows) */
    double *y, *a;       /* [N][R] */
    int64_t r0, r1;      /* this thread's slice of output columns */
} job_t;

static void *run_job(void *arg)
{
    job_t *j = (job_t *)arg;
    for (int64_t i = j->r0; i < j->r1; ++i) {
        int64_t m = j->rows ? j->rows[i] : i;
        for (int64_t n = 0; n < j->N; ++n) {
            dot_row(j->q + m * j->ldq, j->d + m * j->ldd, j->K,
                    j->x16 ? j->x16 + n * j->ldx : NULL,
                    j->x32 ? j->x32 + n * j->ldx : NULL,
                    &j->y[n * j->R + i], &j->a[n * j->R + i]);
        }
    }
    return NULL;
}

/* Shared driver: splits output columns over `threads` pthreads (each runs
 * the same scalar loop; results do not depend on the split). */
static int run(const int8_t *q, const uint16_t *d, int64_t M, int64_t K,
               const uint16_t *x16, const float *x32, int64_t N,
               const int64_t *rows, int64_t R, double *y, double *a, int threads)
{
    if (K % OR_QK || M < 0 || N < 0 || R < 0)
        return -1;
    if (rows)
        for (int64_t i = 0; i < R; ++i)
            if (rows[i] < 0 || rows[i] >= M)
                return -2;
    if (threads < 1)
        threads = 1;
    if (threads > 256)
        threads = 256;
    if (threads > R)
        threads = R > 0 ? (int)R : 1;
    job_t jobs[256];
    pthread_t tid[256];
    for (int t = 0; t < threads; ++t) {
        job_t *j = &jobs[t];
        j->q = q;
        j->d = d;
        j->K = K;
        j->ldq = K;
        j->ldd = K / OR_QK;
        j->x16 = x16;
        j->x32 = x32;
        j->N = N;
        j->ldx = K;
        j->rows = rows;
        j->R = R;
        j->y = y;
        j->a = a;
        j->r0 = R * t / threads;
        j->r1 = R * (t + 1) / threads;
    }
    if (threads == 1) {
        run_job(&jobs[0]);
        return 0;
    }
    int started = 0;
    for (int t = 0; t < threads; ++t) {
        if (pthread_create(&tid[t], NULL, run_job, &jobs[t]) != 0)
            break;
        ++started;
    }
    for (int t = started; t < threads; ++t) /* could not spawn: run inline */
        run_job(&jobs[t]);
    for (int t = 0; t < started; ++t)
        pthread_join(tid[t], NULL);
    return 0;
}

/* y, a: [N][M] fp64. x: fp16 bits [N][K]. */
int or_gemv_f16x(const int8_t *q, const uint16_t *d, int64_t M, int64_t K,
                 const uint16_t *x, int64_t N, double *y, double *a, int threads)
{
    return run(q, d, M, K, x, NULL, N, NULL, M, y, a, threads);
}

/* Same with fp32 activations (each fp32 value is exact in fp64; the product
 * w*x needs up to 19+24 = 43 bits, still exact). */
int or_gemv_f32x(const int8_t *q, const uint16_t *d, int64_t M, int64_t K,
                 const float *x, int64_t N, double *y, double *a, int threads)
{
    return run(q, d, M, K, NULL, x, N, NULL, M, y, a, threads);
}

/* Sampled rows: y, a are [N][R], column i is weight row rows[i]. */
int or_gemv_rows_f16x(const int8_t *q, const uint16_t *d, int64_t M, int64_t K,
                      const uint16_t *x, int64_t N, const int64_t *rows, int64_t R,
                      double *y, double *a, int threads)
{
    return run(q, d, M, K, x, NULL, N, rows, R, y, a, threads);
}
