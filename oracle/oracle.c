/*
 * oracle.c -- plain, slow, obviously correct CPU reference for the
 * batch-invariant linear-layer GEMM.  TEST INFRASTRUCTURE ONLY: the tests,
 * the smoke check and the bench's CPU-baseline leg may call it; the product
 * path never does.  It shares no code, header or table with the HIP library.
 *
 * What it computes (the real-valued definition, to fp64 accuracy):
 *
 *   y[i][n] = sum_k x[i][k] * w[n][k]          (x: [M,K] bf16, w: [N,K] bf16)
 *
 * i.e. the linear layer y = x W^T whose GEMMs dominate an FFN (LLM-42 reading
 * notes, §2.1 and §2.3 Fig. 4a).  A row's result is a function of that row of
 * x alone (Detent, §3: each request's output is mathematically a function of
 * its own input; CoRun, §III-B Definition 1).  Alongside each value it returns
 * a[i][n] = sum_k |x[i][k] * w[n][k]|, the scale of the accuracy bound the GPU
 * result is judged by.
 *
 * Floating-point addition is not associative (LLM-42 notes §2.2; CoRun §III-A
 * Fig. 3), so the pages fix no particular fp32 result; the oracle therefore
 * sums in fp64, where every bf16*bf16 product is exact and the rounding error
 * of the K-term sum is at most (K-1) * 2^-53 * a.  The k loop is sequential
 * and ascending; OpenMP only spreads independent (row, column) pairs.  Build
 * without -ffast-math and with -ffp-contract=off.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* bf16 bits -> fp64, exactly: bf16 is the top half of an fp32. */
static double bf16_to_f64(uint16_t b)
{
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static void set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

/* Number of threads an OpenMP region of this library would use. */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * y[r][n], a[r][n] for the rows rows[0..nrows-1] of x (all M rows when rows is
 * NULL, then nrows must equal M).  Returns 0, or -1 on a bad argument.
 */
int oracle_gemm_f64(const uint16_t *x, const uint16_t *w, long M, long N, long K,
                    const long *rows, long nrows, double *y, double *a, int nthreads)
{
    if (!x || !w || !y || M < 0 || N < 0 || K < 0 || nrows < 0)
        return -1;
    if (!rows && nrows != M)
        return -1;
    for (long r = 0; r < nrows; ++r)
        if (rows && (rows[r] < 0 || rows[r] >= M))
            return -1;
    set_threads(nthreads);
    long total = nrows * N;
#pragma omp parallel for schedule(static)
    for (long p = 0; p < total; ++p) {
        long r = p / N, n = p % N;
        long i = rows ? rows[r] : r;
        const uint16_t *xi = x + i * K;
        const uint16_t *wn = w + n * K;
        double s = 0.0, abs_s = 0.0;
        for (long k = 0; k < K; ++k) {
            double prod = bf16_to_f64(xi[k]) * bf16_to_f64(wn[k]); /* exact */
            s += prod;
            abs_s += fabs(prod);
        }
        y[p] = s;
        if (a)
            a[p] = abs_s;
    }
    return 0;
}

/*
 * Integer-valued inputs: the same sum in int64, exact.  Every x and w value
 * must be an integer of magnitude <= 256 (exact in bf16).  Returns 0, -1 on a
 * bad argument, -2 if some input is not such an integer.
 */
int oracle_gemm_i64(const uint16_t *x, const uint16_t *w, long M, long N, long K,
                    const long *rows, long nrows, int64_t *y, int nthreads)
{
    if (!x || !w || !y || M < 0 || N < 0 || K < 0 || nrows < 0)
        return -1;
    if (!rows && nrows != M)
        return -1;
    for (long r = 0; r < nrows; ++r)
        if (rows && (rows[r] < 0 || rows[r] >= M))
            return -1;
    for (long j = 0; j < M * K; ++j) {
        double v = bf16_to_f64(x[j]);
        if (v != floor(v) || fabs(v) > 256.0)
            return -2;
    }
    for (long j = 0; j < N * K; ++j) {
        double v = bf16_to_f64(w[j]);
        if (v != floor(v) || fabs(v) > 256.0)
            return -2;
    }
    set_threads(nthreads);
    long total = nrows * N;
#pragma omp parallel for schedule(static)
    for (long p = 0; p < total; ++p) {
        long r = p / N, n = p % N;
        long i = rows ? rows[r] : r;
        int64_t s = 0;
        for (long k = 0; k < K; ++k)
            s += (int64_t)bf16_to_f64(x[i * K + k]) * (int64_t)bf16_to_f64(w[n * K + k]);
        y[p] = s;
    }
    return 0;
}

/*
 * Grouped (MoE expert) GEMM: rows are grouped by expert, expert e owning rows
 * offsets[e] .. offsets[e+1]-1 of x (R rows in all); each such row is
 * multiplied by that expert's weight w[e] ([N,K]).  The routing that produces
 * the grouping happens outside the GEMM.  Returns 0, or -1 on a bad argument
 * (offsets must start at 0, end at R and never decrease).
 */
int oracle_grouped_f64(const uint16_t *x, const uint16_t *w, long E, long N, long K,
                       const int32_t *offsets, long R, const long *rows, long nrows,
                       double *y, double *a, int nthreads)
{
    if (!x || !w || !offsets || !y || E <= 0 || N < 0 || K < 0 || R < 0 || nrows < 0)
        return -1;
    if (!rows && nrows != R)
        return -1;
    if (offsets[0] != 0 || offsets[E] != R)
        return -1;
    for (long e = 0; e < E; ++e)
        if (offsets[e + 1] < offsets[e])
            return -1;
    for (long r = 0; r < nrows; ++r)
        if (rows && (rows[r] < 0 || rows[r] >= R))
            return -1;
    set_threads(nthreads);
    long total = nrows * N;
#pragma omp parallel for schedule(static)
    for (long p = 0; p < total; ++p) {
        long r = p / N, n = p % N;
        long i = rows ? rows[r] : r;
        long e = 0;
        while (!(offsets[e] <= i && i < offsets[e + 1]))
            ++e;
        const uint16_t *xi = x + i * K;
        const uint16_t *wn = w + (e * N + n) * K;
        double s = 0.0, abs_s = 0.0;
        for (long k = 0; k < K; ++k) {
            double prod = bf16_to_f64(xi[k]) * bf16_to_f64(wn[k]);
            s += prod;
            abs_s += fabs(prod);
        }
        y[p] = s;
        if (a)
            a[p] = abs_s;
    }
    return 0;
}

/*
 * The in-order combine of split partial sums, in fp32 round-to-nearest-even:
 * out = (((p[0] + p[1]) + p[2]) + ...) + p[S-1].  A split kernel fixes its
 * split boundaries and adds the partial sums in that fixed order (CoRun,
 * §III-A Fig. 3b keeps (a+b)+(c+d) at every batch size; Detent, Fig. 2b
 * combines the splits in order).  parts is [S][count]; out is [count].
 */
int oracle_fold_f32(const float *parts, long S, long count, float *out)
{
    if (!parts || !out || S <= 0 || count < 0)
        return -1;
    for (long j = 0; j < count; ++j) {
        volatile float t = parts[j];
        for (long s = 1; s < S; ++s)
            t = t + parts[s * count + j];
        out[j] = t;
    }
    return 0;
}
