/*
 * Sanitizer driver for the CPU oracle (oracle/skinny_oracle.c), built with gcc
 * -fsanitize=address,undefined together with it by tests/test_sanitizers.py.
 *
 * Every buffer is a heap allocation of exactly the size the oracle's contract
 * names, so a read or write past it is reported. It runs every bfloat16 pattern
 * through the round trip, special and random doubles through the rounding, and
 * the row-selecting product over random small shapes, row subsets and thread
 * counts (more threads than rows, zero rows, K = 0), comparing each result
 * element with the same definition evaluated here in plain loops, bit for bit
 * (the oracle's result does not depend on its thread count); invalid arguments
 * must return -1.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_bf16_to_f64(uint16_t h);
uint16_t oracle_f64_to_bf16(double v);
int oracle_gemm_bf16_rows(const uint16_t *x, const uint16_t *W, const int64_t *rows, int64_t nrows,
                          int M, int K, uint16_t *y, double *ref64, double *mag, double *x64,
                          int nthreads);
int oracle_gemm_bf16(const uint16_t *x, const uint16_t *W, int M, int N, int K, uint16_t *y,
                     double *ref64, double *mag, double *x64, int nthreads);

static uint64_t s = 0x243F6A8885A308D3ull;
static uint64_t next(void)
{
    s ^= s << 13;
    s ^= s >> 7;
    s ^= s << 17;
    return s;
}

static int failures = 0;
static void fail(const char *what, long i)
{
    fprintf(stderr, "oracle_check: %s (case %ld)\n", what, i);
    if (++failures > 20)
        exit(1);
}

/* a random finite bfloat16 of moderate size: sign, exponent 2^-8 .. 2^7 */
static uint16_t rnd_bf16(void)
{
    uint16_t sign = (uint16_t)((next() & 1) << 15);
    uint16_t e = (uint16_t)(127 - 8 + next() % 16);
    return (uint16_t)(sign | (e << 7) | (next() & 0x7F));
}

int main(void)
{
    /* every pattern round-trips (NaNs stay NaN) */
    for (uint32_t h = 0; h < 65536; ++h) {
        double v = oracle_bf16_to_f64((uint16_t)h);
        uint16_t back = oracle_f64_to_bf16(v);
        if (isnan(v) ? !isnan(oracle_bf16_to_f64(back)) : back != (uint16_t)h)
            fail("bf16 round trip", (long)h);
    }
    /* specials and random bit patterns through the rounding */
    const double specials[] = {0.0, -0.0, INFINITY, -INFINITY, NAN, 1e-320, -1e-320, 3.0e38, 3.4e38,
                               -3.4e38, 1.7976931348623157e308, 5e-324};
    for (size_t i = 0; i < sizeof specials / sizeof specials[0]; ++i)
        (void)oracle_f64_to_bf16(specials[i]);
    for (long i = 0; i < 200000; ++i) {
        uint64_t bits = next();
        double v;
        memcpy(&v, &bits, sizeof v);
        (void)oracle_f64_to_bf16(v);
    }

    /* the product over random shapes, row subsets and thread counts */
    for (long c = 0; c < 3000; ++c) {
        int M = (int)(next() % 5), K = (int)(next() % 41), N = 1 + (int)(next() % 20);
        int64_t nrows = (int64_t)(next() % 24);
        int use_rows = (int)(next() % 2);
        int nthreads = (int)(next() % 6) + (next() % 8 == 0 ? 300 : 0) - 1;
        uint16_t *x = malloc(sizeof(uint16_t) * (size_t)(M * K + 1));
        uint16_t *W = malloc(sizeof(uint16_t) * (size_t)(N * K + 1));
        int64_t *rows = malloc(sizeof(int64_t) * (size_t)(nrows + 1));
        int64_t nout = use_rows ? nrows : N;
        uint16_t *y = malloc(sizeof(uint16_t) * (size_t)(M * nout + 1));
        double *ref = malloc(sizeof(double) * (size_t)(M * nout + 1));
        double *mag = malloc(sizeof(double) * (size_t)(M * nout + 1));
        double *x64 = malloc(sizeof(double) * (size_t)(M * K + 1));
        for (int i = 0; i < M * K; ++i)
            x[i] = rnd_bf16();
        for (int i = 0; i < N * K; ++i)
            W[i] = rnd_bf16();
        for (int64_t i = 0; i < nrows; ++i)
            rows[i] = (int64_t)(next() % (uint64_t)N);
        int rc = oracle_gemm_bf16_rows(x, W, use_rows ? rows : NULL, nout, M, K, y, ref, mag, x64, nthreads);
        if (rc != 0)
            fail("valid call refused", c);
        for (int m = 0; m < M; ++m)
            for (int64_t i = 0; i < nout; ++i) {
                int64_t n = use_rows ? rows[i] : i;
                double sum = 0.0, a = 0.0;
                for (int k = 0; k < K; ++k) {
                    double p = oracle_bf16_to_f64(x[m * K + k]) * oracle_bf16_to_f64(W[n * K + k]);
                    sum += p;
                    a += fabs(p);
                }
                size_t o = (size_t)m * (size_t)nout + (size_t)i;
                if (memcmp(&sum, &ref[o], sizeof sum) != 0 || memcmp(&a, &mag[o], sizeof a) != 0 ||
                    y[o] != oracle_f64_to_bf16(sum))
                    fail("element differs from the definition", c);
            }
        if (!use_rows && oracle_gemm_bf16(x, W, M, N, K, y, NULL, NULL, x64, nthreads) != 0)
            fail("full product refused", c);
        free(x);
        free(W);
        free(rows);
        free(y);
        free(ref);
        free(mag);
        free(x64);
    }
    /* invalid arguments */
    uint16_t b[4] = {0};
    double d[4];
    if (oracle_gemm_bf16_rows(NULL, b, NULL, 1, 1, 1, b, d, d, d, 1) != -1 ||
        oracle_gemm_bf16_rows(b, b, NULL, -1, 1, 1, b, d, d, d, 1) != -1 ||
        oracle_gemm_bf16_rows(b, b, NULL, 1, -1, 1, b, d, d, d, 1) != -1 ||
        oracle_gemm_bf16_rows(b, b, NULL, 1, 1, -1, b, d, d, d, 1) != -1 ||
        oracle_gemm_bf16_rows(b, b, NULL, 1, 1, 1, b, d, d, NULL, 1) != -1)
        fail("invalid arguments accepted", -1);
    printf("oracle_check: %d failures\n", failures);
    return failures == 0 ? 0 : 1;
}
