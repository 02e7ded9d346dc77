/*
 * bi_norm.h -- C ABI of the batch-invariant RMSNorm for MI355X (gfx950), the
 * step before a gate+up projection.
 *
 * RMSNorm reduces each token's hidden vector.  A stock kernel splits that
 * reduction over several blocks when the batch holds few tokens and keeps a
 * row in one block when it holds many, so the summation tree, and with it
 * the low-order bits of a token's result, follow the batch (CoRun, §III-A
 * Fig. 3a).  A batch-invariant kernel keeps one partition and one combine
 * order for every batch (CoRun, §III-A Fig. 3b).  The pages measure what
 * that costs against stock kernels: CoRun, §II Fig. 2a (Mean, RMSNorm and
 * Softmax 2.12-5.61x) and LLM-42 notes, §2.3 Fig. 4b.
 *
 * Here the tree depends on H alone: one block of 256 threads per row;
 * thread t sums the squares of 16-byte chunks t, t+256, t+512, ... of the
 * row in ascending order (the eight values of a chunk in order), in fp32,
 * one multiply and one add each; inside each 64-thread wave the sums are
 * combined by a butterfly over lane distances 32, 16, 8, 4, 2, 1 (every lane
 * ends with its wave's total), and the four wave totals are added in order,
 * ((w0 + w1) + w2) + w3.  Then r = 1 / sqrt(total / H + eps) and
 * y = bf16((x * r) * g), every operation IEEE fp32 round-to-nearest-even,
 * the last one rounding to bf16 the same way.
 *
 * Conventions (as bi_gemm.h): device pointers, row-major, `stream` is a
 * hipStream_t (NULL: the null stream); every argument is checked on the host
 * before any HIP call, a failure launches nothing, detail in bi_last_error().
 * The call neither allocates nor synchronises.
 */
#ifndef BI_NORM_H
#define BI_NORM_H

#include "bi_gemm.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * y[t] = RMSNorm(x[t]) * gain for t < T.  x: bf16 [T, H]; gain: bf16 [H];
 * y: bf16 [T, H] out (may not overlap x).  8 <= H <= 65536, H a multiple of
 * 8; T >= 0 (T == 0 launches nothing), T*H < 2^31; eps finite and >= 0 (a
 * zero row with eps == 0 gives NaN, as the formula does); x, gain and y
 * 16-byte aligned.  A row's output is a function of that row and gain only.
 */
bi_status_t bi_rmsnorm(const void *x, const void *gain, int T, int H, float eps, void *y, void *stream);

/*
 * The RMSNorm fused into the prologue of the projection that follows it
 * (the gate+up projection of a Llama block): y = bf16(RMSNorm(x) * gain) W^T
 * for the M raw rows of x, bit for bit what bi_rmsnorm into a bf16 buffer
 * followed by bi_gemm_run on it gives, without that buffer.  A row pass
 * writes each row's r = 1 / sqrt(mean(x^2) + eps) (the tree above) to rstd;
 * the GEMM then loads the raw rows into LDS and rewrites each stage's x tile
 * in place as bf16((x * r) * g), the rounding bi_rmsnorm uses, before its
 * MFMAs read it.  The pages measure a separate batch-invariant norm against
 * stock kernels (CoRun, §II Fig. 2a; LLM-42 notes, §2.3 Fig. 4b).
 *   h: dense handle of a layer [N, K]; H = K (8 <= K <= 65536).
 *   x: bf16 [M, K] raw rows; gain: bf16 [K]; both 16-byte aligned.
 *   rstd: fp32 [M] out, 4-byte aligned (the rows' r; also what a backward
 *         pass of the norm keeps).
 *   y: fp32 [M, N] out, 16-byte aligned; must not overlap x or rstd.
 *   eps: finite, >= 0.  M: 0 <= M, M * max(N, K) < 2^31; M == 0 launches
 *   nothing.
 * The GEMM runs the handle's tree; where the handle's tiling names a
 * streaming or four-wave kernel, the tiled kernel that normalises its tiles
 * runs instead (64x32, or 128x128 with eight waves): same tree, other speed.
 * Asynchronous and allocation-free like bi_gemm_run.
 */
bi_status_t bi_rmsnorm_gemm_run(bi_gemm_t h, const void *x, const void *gain, float eps, int M, float *rstd,
                                float *y, void *stream);

/* The GEMM kernel bi_rmsnorm_gemm_run launches for M rows ("" for an
 * invalid handle or M <= 0). */
const char *bi_rmsnorm_gemm_kernel_name(bi_gemm_t h, int M);

#ifdef __cplusplus
}
#endif

#endif /* BI_NORM_H */
