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

/* ------------------------------------------------------------------------
 * The MoE layer around the grouped GEMM.  The fused MoE is one of the kernel
 * families whose selection reads the batch (Detent, §2 Obs. 1 and Fig. 3a:
 * it takes the tuned row nearest the batch's token count); each step below is
 * a function of one token's own values, so the whole layer is too.  The steps
 * follow a Qwen3-30B-A3B-style expert layer (Detent, §8.1: the MoE deployment;
 * CoRun, §VII-C: a router perturbation changes the experts a token uses):
 * router logits, top-k, grouping of the rows by expert, up projection, SwiGLU,
 * down projection, and the weighted combine of each token's k expert outputs.
 * ------------------------------------------------------------------------ */

/*
 * Top-k routing of each token: the k experts with the largest logits, best
 * first, an equal logit going to the lower expert id; the decision compares
 * the fp32 logits as given.  weights w[t][j] = exp(l_j - l_0) / sum_i exp(l_i
 * - l_0) over the k chosen logits, in fp64 (the softmax over all experts,
 * renormalised over the chosen ones, is the same number).  k passes over the
 * logits, each taking the best expert not yet chosen.  Returns 0, -1 on a bad
 * argument, -3 when a logit is not finite.
 */
int oracle_moe_topk(const float *logits, long T, long E, long k, int32_t *ids, double *w)
{
    if (!logits || !ids || !w || T < 0 || E <= 0 || k <= 0 || k > E || k > 1024)
        return -1;
    for (long i = 0; i < T * E; ++i)
        if (!isfinite(logits[i]))
            return -3;
    for (long t = 0; t < T; ++t) {
        const float *l = logits + t * E;
        int32_t *id = ids + t * k;
        for (long j = 0; j < k; ++j) {
            long best = -1;
            for (long e = 0; e < E; ++e) {
                int taken = 0;
                for (long q = 0; q < j; ++q)
                    taken |= id[q] == e;
                if (taken)
                    continue;
                if (best < 0 || l[e] > l[best])  /* ties keep the lower id found first */
                    best = e;
            }
            id[j] = (int32_t)best;
        }
        double z[1024];
        double s = 0.0;
        for (long j = 0; j < k; ++j) {
            z[j] = exp((double)l[id[j]] - (double)l[id[0]]);
            s += z[j];
        }
        for (long j = 0; j < k; ++j)
            w[t * k + j] = z[j] / s;
    }
    return 0;
}

/*
 * Rows grouped by expert: every (token t, slot j) pair becomes one row of its
 * expert ids[t][j]; experts in ascending id, and inside an expert the pairs
 * in ascending (t, j) -- a stable counting sort.  offsets[E+1] delimits each
 * expert's rows, token_of_row[R] names a row's token and row_of[t*k + j] the
 * row of pair (t, j).  Returns 0, or -1 on a bad argument or an id outside
 * 0..E-1.
 */
int oracle_moe_permute(const int32_t *ids, long T, long E, long k, int32_t *offsets,
                       int32_t *token_of_row, int32_t *row_of)
{
    if (!ids || !offsets || !token_of_row || !row_of || T < 0 || E <= 0 || k <= 0)
        return -1;
    for (long i = 0; i < T * k; ++i)
        if (ids[i] < 0 || ids[i] >= E)
            return -1;
    for (long e = 0; e <= E; ++e)
        offsets[e] = 0;
    for (long i = 0; i < T * k; ++i)
        offsets[ids[i] + 1] += 1;
    for (long e = 0; e < E; ++e)
        offsets[e + 1] += offsets[e];
    for (long e = 0; e < E; ++e) {
        long r = offsets[e];
        for (long t = 0; t < T; ++t)
            for (long j = 0; j < k; ++j)
                if (ids[t * k + j] == e) {
                    token_of_row[r] = (int32_t)t;
                    row_of[t * k + j] = (int32_t)r;
                    ++r;
                }
    }
    return 0;
}

/*
 * SwiGLU of the up projection's output h [R, 2I] (gate columns 0..I-1, up
 * columns I..2I-1): a[r][i] = silu(g) * u with silu(g) = g / (1 + exp(-g)),
 * in fp64.  Returns 0 or -1.
 */
int oracle_swiglu_f64(const float *h, long R, long I, double *a)
{
    if (!h || !a || R < 0 || I <= 0)
        return -1;
    for (long r = 0; r < R; ++r)
        for (long i = 0; i < I; ++i) {
            double g = h[r * 2 * I + i];
            double u = h[r * 2 * I + I + i];
            a[r * I + i] = g / (1.0 + exp(-g)) * u;
        }
    return 0;
}

/*
 * Weighted combine of each token's k expert outputs:
 *   y[t][n] = sum_j w[t][j] * o[row_of[t][j]][n]
 * in fp64, and s[t][n] = sum_j |w[t][j] * o[row_of[t][j]][n]|, the scale of
 * the bound a fixed-order fp32 sum is judged by.  Returns 0, or -1 on a bad
 * argument or a row outside 0..R-1.
 */
int oracle_moe_combine_f64(const float *o, long R, const float *w, const int32_t *row_of, long T,
                           long k, long H, double *y, double *s)
{
    if (!o || !w || !row_of || !y || R < 0 || T < 0 || k <= 0 || H < 0)
        return -1;
    for (long i = 0; i < T * k; ++i)
        if (row_of[i] < 0 || row_of[i] >= R)
            return -1;
    for (long t = 0; t < T; ++t)
        for (long n = 0; n < H; ++n) {
            double acc = 0.0, mag = 0.0;
            for (long j = 0; j < k; ++j) {
                double p = (double)w[t * k + j] * (double)o[(long)row_of[t * k + j] * H + n];
                acc += p;
                mag += fabs(p);
            }
            y[t * H + n] = acc;
            if (s)
                s[t * H + n] = mag;
        }
    return 0;
}

/* ------------------------------------------------------------------------
 * RMSNorm, the step before the gate+up projection.  A token-wise reduction
 * over the hidden dimension whose stock kernels split a row across blocks
 * when the batch is small, so the tree (and the bits) follow the batch
 * (CoRun, §III-A Fig. 3; the pages measure batch-invariant RMSNorm against
 * stock kernels in CoRun §II Fig. 2a and LLM-42 notes §2.3 Fig. 4b).
 * ------------------------------------------------------------------------ */

/*
 * y[t][h] = x[t][h] * g[h] / sqrt(ms[t] + eps), ms[t] = (1/H) sum_h x[t][h]^2,
 * in fp64 over bf16 inputs (each square is exact in fp64; the H-term sum of
 * non-negative terms is within (H-1) * 2^-53 of its value, relatively).  ms
 * is returned too.  Returns 0, or -1 on a bad argument.
 */
int oracle_rmsnorm_f64(const uint16_t *x, const uint16_t *g, long T, long H, double eps, double *y,
                       double *ms)
{
    if (!x || !g || !y || !ms || T < 0 || H <= 0 || !(eps >= 0.0))
        return -1;
    for (long t = 0; t < T; ++t) {
        double s = 0.0;
        for (long h = 0; h < H; ++h) {
            double v = bf16_to_f64(x[t * H + h]);
            s += v * v;
        }
        ms[t] = s / (double)H;
        double inv = 1.0 / sqrt(ms[t] + eps);
        for (long h = 0; h < H; ++h)
            y[t * H + h] = bf16_to_f64(x[t * H + h]) * bf16_to_f64(g[h]) * inv;
    }
    return 0;
}

/* ------------------------------------------------------------------------
 * Decode attention: one new query token per sequence against its KV cache.
 * Split-KV kernels partition a sequence's keys across blocks when the batch
 * is small; batch invariance needs split boundaries that do not depend on
 * the batch -- a fixed split size (Detent, §8.1 Kernels: a rebuilt FA3 that
 * keeps split-KV with the fixed split-size principle; CoRun, §IV-C and
 * §V-F: Split-KV turned off for decode instead).  The oracle is the
 * definition, with no split at all.
 * ------------------------------------------------------------------------ */

/*
 * For sequence b (keys seq_start[b] .. seq_start[b+1]-1 of the cache) and
 * query head h (kv head h / (Hq / Hkv)), in fp64:
 *   s_t = scale * sum_i q[b][h][i] * k[t][kvh][i]
 *   p_t = exp(s_t - max_u s_u) / sum_u exp(s_u - max_u s_u)
 *   out[b][h][i] = sum_t p_t * v[t][kvh][i]
 * and, for the accuracy bound, mag[b][h][i] = sum_t p_t |v[t][kvh][i]| and
 * qk[b][h] = max_t scale * sum_i |q[b][h][i] * k[t][kvh][i]|.  q: bf16
 * [B, Hq, D]; k, v: bf16 [Ntok, Hkv, D]; a sequence with no keys gives
 * out = mag = qk = 0.  Returns 0, or -1 on a bad argument (Hq not a multiple
 * of Hkv, offsets outside 0..Ntok or decreasing).
 */
int oracle_decode_attn_f64(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                           const int32_t *seq_start, long B, long Hq, long Hkv, long D, long Ntok,
                           double scale, double *out, double *mag, double *qk)
{
    if (!q || !k || !v || !seq_start || !out || !mag || !qk || B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 ||
        Hq % Hkv != 0 || Ntok < 0)
        return -1;
    for (long b = 0; b < B; ++b)
        if (seq_start[b] < 0 || seq_start[b + 1] < seq_start[b] || seq_start[b + 1] > Ntok)
            return -1;
    const long G = Hq / Hkv;
#pragma omp parallel for schedule(dynamic)
    for (long bh = 0; bh < B * Hq; ++bh) {
        const long b = bh / Hq, h = bh % Hq, kvh = h / G;
        const long t0 = seq_start[b], n = seq_start[b + 1] - t0;
        const uint16_t *qv = q + (b * Hq + h) * D;
        double *o = out + (b * Hq + h) * D;
        double *mg = mag + (b * Hq + h) * D;
        for (long i = 0; i < D; ++i)
            o[i] = mg[i] = 0.0;
        qk[bh] = 0.0;
        if (n == 0)
            continue;
        double smax = -INFINITY, amax = 0.0;
        for (long t = 0; t < n; ++t) {
            const uint16_t *kt = k + ((t0 + t) * Hkv + kvh) * D;
            double s = 0.0, a = 0.0;
            for (long i = 0; i < D; ++i) {
                double p = bf16_to_f64(qv[i]) * bf16_to_f64(kt[i]);
                s += p;
                a += fabs(p);
            }
            s *= scale;
            a *= fabs(scale);
            if (s > smax)
                smax = s;
            if (a > amax)
                amax = a;
        }
        qk[bh] = amax;
        double den = 0.0;
        for (long t = 0; t < n; ++t) {
            const uint16_t *kt = k + ((t0 + t) * Hkv + kvh) * D;
            const uint16_t *vt = v + ((t0 + t) * Hkv + kvh) * D;
            double s = 0.0;
            for (long i = 0; i < D; ++i)
                s += bf16_to_f64(qv[i]) * bf16_to_f64(kt[i]);
            const double e = exp(s * scale - smax);
            den += e;
            for (long i = 0; i < D; ++i) {
                const double vi = bf16_to_f64(vt[i]);
                o[i] += e * vi;
                mg[i] += e * fabs(vi);
            }
        }
        for (long i = 0; i < D; ++i) {
            o[i] /= den;
            mg[i] /= den;
        }
    }
    return 0;
}
