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

#ifdef __cplusplus
}
#endif

#endif /* BI_NORM_H */
