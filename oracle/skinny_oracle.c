/*
 * CPU oracle for the BF16 skinny GEMM  y[M,N] = x[M,K] . W[N,K]^T.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the plain, slow, obviously correct
 * definition that the HIP kernels are checked against. It shares no code,
 * header, table or helper with the HIP library, and only tests, the smoke
 * check and the benchmark's CPU-baseline leg may load it.
 *
 * What it computes (the definition written out, no blocking or reordering):
 *
 *   ref64[m,n] = sum_{k=0..K-1} double(x[m,k]) * double(W[n,k])   (k ascending)
 *   mag[m,n]   = sum_{k=0..K-1} |double(x[m,k]) * double(W[n,k])| (tolerance scale)
 *   y[m,n]     = bf16_rne(ref64[m,n])                               (one rounding)
 *
 * Sources: the operation is F.linear on bfloat16 tensors at 1..4 tokens (vLLM
 * PR #62949, SM121 skinny GEMM plans, section Validation: outputs compared with
 * F.linear); the reference precision is float64 (vLLM PR #65306, SM90 skinny
 * GEMM plans, section Validation: elementwise comparison with a float64
 * reference). Each product of two bfloat16 values is exact in double (8 + 8
 * significant bits), so only the sums round, at double precision.
 *
 * Rounding to bfloat16 (the reading taken where the cited pull requests are
 * silent):
 * IEEE-754 round-to-nearest, ties-to-even, applied once, directly from the
 * double value (no intermediate float rounding); results beyond the largest
 * finite bfloat16 by half an ulp or more become +-Inf; NaN becomes a quiet NaN
 * with the input's sign; subnormal bfloat16 results are kept, not flushed.
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared -pthread  (no fast-math).
 */
#include <math.h>
#include <pthread.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

/* bfloat16 bit pattern -> double. A bfloat16 value is the top half of a
 * binary32 value, so the widening is exact. */
double oracle_bf16_to_f64(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* double -> bfloat16 bit pattern, round-to-nearest-even, one rounding step.
 *
 * bfloat16 has 8 significant bits: for |v| in [2^e, 2^(e+1)) with e >= -126 the
 * spacing of representable values is q = 2^(e-7); below 2^-126 (subnormals) it
 * is 2^-133. v/q is then computed exactly (q is a power of two and the quotient
 * stays far inside double's range), rint() rounds it to an integer with ties to
 * even under the default rounding mode, and n*q is exactly representable in
 * binary32, so the final narrowing to float is exact and its top half is the
 * bfloat16 pattern. */
uint16_t oracle_f64_to_bf16(double v)
{
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    if (isnan(v))
        return (uint16_t)(sign | 0x7FC0u);
    double a = fabs(v);
    if (isinf(a))
        return (uint16_t)(sign | 0x7F80u);
    if (a == 0.0)
        return sign;

    int E;
    (void)frexp(a, &E);          /* a = f * 2^E, f in [0.5, 1)  ->  floor(log2 a) = E - 1 */
    int e = E - 1;
    if (e < -126)
        e = -126;                /* subnormal range shares the spacing of the smallest normal binade */
    double q = ldexp(1.0, e - 7);
    double n = rint(a / q);      /* exact quotient, ties to even */
    double r = n * q;            /* exact */
    if (r >= ldexp(1.0, 128))    /* rounded past the largest finite value */
        return (uint16_t)(sign | 0x7F80u);

    float f = (float)r;          /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (uint16_t)(u >> 16));
}

/* Vector forms, used by the Python wrapper for the exhaustive rounding pins. */
void oracle_bf16_to_f64_array(const uint16_t *h, double *out, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        out[i] = oracle_bf16_to_f64(h[i]);
}

void oracle_f64_to_bf16_array(const double *v, uint16_t *out, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        out[i] = oracle_f64_to_bf16(v[i]);
}

/* One output element: the definition above, k ascending. */
static void dot_row(const double *x64, const uint16_t *w_row, int K, double *sum, double *mag)
{
    double s = 0.0, a = 0.0;
    for (int k = 0; k < K; ++k) {
        double p = x64[k] * oracle_bf16_to_f64(w_row[k]);
        s += p;
        a += fabs(p);
    }
    *sum = s;
    *mag = a;
}

typedef struct {
    const double *x64;        /* [M, K] activations widened to double */
    const uint16_t *W;        /* [N, K] weight bits */
    const int64_t *rows;      /* rows of W to evaluate (NULL = 0..nrows-1) */
    int64_t nrows;
    int M, K;
    int64_t lo, hi;           /* this worker's slice of [0, nrows) */
    uint16_t *y;              /* [M, nrows] */
    double *ref64;            /* [M, nrows] or NULL */
    double *mag;              /* [M, nrows] or NULL */
} job_t;

static void *worker(void *arg)
{
    job_t *j = (job_t *)arg;
    for (int64_t i = j->lo; i < j->hi; ++i) {
        int64_t n = j->rows ? j->rows[i] : i;
        const uint16_t *w_row = j->W + (size_t)n * (size_t)j->K;
        for (int m = 0; m < j->M; ++m) {
            double s, a;
            dot_row(j->x64 + (size_t)m * (size_t)j->K, w_row, j->K, &s, &a);
            size_t o = (size_t)m * (size_t)j->nrows + (size_t)i;
            j->y[o] = oracle_f64_to_bf16(s);
            if (j->ref64)
                j->ref64[o] = s;
            if (j->mag)
                j->mag[o] = a;
        }
    }
    return NULL;
}

#define ORACLE_MAX_THREADS 256

/* Evaluate the definition for the selected rows of W (rows == NULL: all rows
 * 0..nrows-1, i.e. the full product with N = nrows). Outputs are [M, nrows],
 * row-major. x64 is scratch of M*K doubles owned by the caller. Returns 0, or -1
 * on invalid arguments. The work is split over `nthreads` POSIX threads by
 * output row; every element is still computed by the same sequential loop, so
 * the result does not depend on the thread count. */
int oracle_gemm_bf16_rows(const uint16_t *x, const uint16_t *W, const int64_t *rows,
                          int64_t nrows, int M, int K, uint16_t *y, double *ref64,
                          double *mag, double *x64, int nthreads)
{
    if (!x || !W || !y || !x64 || M < 0 || K < 0 || nrows < 0)
        return -1;
    for (size_t i = 0; i < (size_t)M * (size_t)K; ++i)
        x64[i] = oracle_bf16_to_f64(x[i]);

    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > ORACLE_MAX_THREADS)
        nthreads = ORACLE_MAX_THREADS;
    if ((int64_t)nthreads > nrows)
        nthreads = nrows > 0 ? (int)nrows : 1;

    job_t jobs[ORACLE_MAX_THREADS];
    pthread_t tids[ORACLE_MAX_THREADS];
    int started[ORACLE_MAX_THREADS];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = (job_t){x64, W, rows, nrows, M, K,
                          nrows * t / nthreads, nrows * (t + 1) / nthreads, y, ref64, mag};
        started[t] = 0;
    }
    for (int t = 1; t < nthreads; ++t)
        started[t] = pthread_create(&tids[t], NULL, worker, &jobs[t]) == 0;
    worker(&jobs[0]);
    for (int t = 1; t < nthreads; ++t) {
        if (started[t])
            pthread_join(tids[t], NULL);
        else
            worker(&jobs[t]);    /* thread creation failed: do the slice here */
    }
    return 0;
}

/* Full product y[M,N] = x[M,K] . W[N,K]^T. */
int oracle_gemm_bf16(const uint16_t *x, const uint16_t *W, int M, int N, int K, uint16_t *y,
                     double *ref64, double *mag, double *x64, int nthreads)
{
    return oracle_gemm_bf16_rows(x, W, NULL, N, M, K, y, ref64, mag, x64, nthreads);
}
