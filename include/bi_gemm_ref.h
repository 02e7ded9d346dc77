/*
 * bi_gemm_ref.h -- the NON-invariant comparison GEMM of this library, for
 * measuring what batch invariance costs on MI355X (gfx950).
 *
 * The pages measure the price of invariance against the fastest GEMM the
 * vendor library picks per shape: a batch-invariant kernel gives up split-K
 * and shape-adapted tiles, and loses most at small and mid batch sizes
 * (LLM-42 reading notes, §2.3 Fig. 4a: 527 against 194 TFLOPS on the
 * Llama-3.1-8B down-projection; CoRun, §I Fig. 1b and §II Fig. 2b).  This
 * entry point is that comparison written with this library's own kernels:
 * the caller picks, per call, the kernel and a number of CONCURRENT K splits
 * (more workgroups over the same tiles, each summing its own K range), the
 * way a batch-dependent selector would.  Because the split count may follow
 * M, a row's bits may follow the batch: never use it where invariance is
 * required.  It exists for the benchmark's cost-of-invariance figure.
 *
 * Conventions as bi_gemm.h: host-side checks before any HIP call, a failure
 * launches nothing, detail in bi_last_error(); no allocation, no
 * synchronisation.
 */
#ifndef BI_GEMM_REF_H
#define BI_GEMM_REF_H

#include "bi_gemm.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * y = x W^T on a dense handle's weights, with kernel `kind`
 * (bi_kernel_kind_t) and `splits` concurrent K splits: split s sums
 * k in [s K / splits, (s + 1) K / splits) as one MFMA chain; split 0 writes
 * y, splits 1.. write their partials into `workspace`, and a final kernel adds
 * them to y in ascending split order.  The handle's own pin (its tree and
 * tiling) is not used.
 *   x, y, M: as bi_gemm_run.
 *   kind: 0 .. BI_KERNEL_COUNT-1.
 *   splits: 1 .. 16 with K % (64 * splits) == 0.
 *   workspace: device fp32 [(splits-1) * M * N], 16-byte aligned, not
 *       overlapping y; unused (may be NULL) when splits == 1.  Caller-owned.
 * Returns BI_ERR_INVALID_ARGUMENT for a grouped handle or bad sizes.
 */
bi_status_t bi_gemm_run_splitk(bi_gemm_t h, const void *x, int M, float *y, int kind, int splits,
                               float *workspace, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* BI_GEMM_REF_H */
