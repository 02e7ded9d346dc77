/*
 * bi_moe.h -- C ABI of the batch-invariant MoE expert layer for MI355X
 * (gfx950), built around the grouped GEMM of bi_gemm.h.
 *
 * The layer a token goes through (a Qwen3-30B-A3B-style expert block, the MoE
 * deployment of Detent, §8.1):
 *
 *   logits = x W_r^T                        router, the dense GEMM [E, H]
 *   (ids, w) = top-k(logits)                k experts, weights softmax(chosen)
 *   rows grouped by expert                  (token, slot) pairs, stable
 *   h = x_row W_up[e]^T                     grouped GEMM [E, 2I, H], each row
 *                                           read from its token's row of x
 *   a = bf16(silu(h[:, :I]) * h[:, I:])     SwiGLU
 *   o = a W_down[e]^T                       grouped GEMM [E, H, I]
 *   y[t] = sum_j w[t][j] o[row(t, j)]       in ascending expert id
 *
 * Why each step is pinned: the stock fused MoE picks its kernel
 * configuration from the row of its tuned table nearest the batch's token
 * count (Detent, §2 Obs. 1 and Fig. 3a), and Detent pins that row key (§5);
 * here no step reads the token count at all.  The routing is where a
 * numerical difference turns into different work: a perturbed router logit
 * changes the experts a token uses (CoRun, §VII-C, on Qwen3-30B-A3B).  So
 * every step computes a token's values from that token's inputs alone, in a
 * fixed order: a token's outputs keep their bits whatever other tokens share
 * the call.
 *
 * Conventions (as bi_gemm.h): device pointers, row-major, `stream` is a
 * hipStream_t (NULL: the null stream); every argument is checked on the host
 * before any HIP call and a failure launches nothing (Detent, §5); detail of
 * a failure in bi_last_error().  The step functions enqueue kernels and
 * neither allocate nor synchronise.  Device data (logits, ids, offsets) is
 * never read by the host: kernels clamp it so that bad values cannot send
 * them outside the buffers named here.
 */
#ifndef BI_MOE_H
#define BI_MOE_H

#include "bi_gemm.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct bi_moe *bi_moe_t;

/*
 * Top-k routing of each token (Detent, §2 Obs. 1: the MoE step whose choice
 * must not depend on the batch).
 *   logits: fp32 [T, E], 4-byte aligned.  ids: int32 [T, k] out, the k
 *   experts with the largest logits, best first, an equal logit to the lower
 *   expert id (a NaN logit ranks as -inf).  weights: fp32 [T, k] out,
 *   exp(l_j - l_0) / sum_i exp(l_i - l_0) over the chosen logits, summed in
 *   the order chosen (equal to the softmax over all experts renormalised
 *   over the chosen ones).
 *   1 <= E <= 1024, 1 <= k <= min(E, 64), 0 <= T, T*E < 2^31.  T == 0 launches
 *   nothing.
 */
bi_status_t bi_moe_topk(const float *logits, int T, int E, int k, int32_t *ids, float *weights,
                        void *stream);

/*
 * Rows grouped by expert: pair (t, j) becomes one row of expert ids[t][j];
 * experts ascending, inside an expert pairs ascending in (t, j) -- a stable
 * grouping, the row order bi_grouped_gemm_run takes.
 *   ids: int32 [T, k].  offsets: int32 [E+1] out (expert e owns rows
 *   offsets[e] .. offsets[e+1]-1; always written, all zero for T == 0).
 *   token_of_row: int32 [T*k] out (first offsets[E] entries written).
 *   row_of: int32 [T, k] out, the row of each pair; -1 for an id outside
 *   0..E-1, which gets no row.  1 <= E <= 1024, 1 <= k <= 64, T*k < 2^31;
 *   4-byte aligned.
 */
bi_status_t bi_moe_permute(const int32_t *ids, int T, int E, int k, int32_t *offsets,
                           int32_t *token_of_row, int32_t *row_of, void *stream);

/*
 * Row gather: dst[r] = src[idx[r]] for bf16 rows of K values; an index
 * outside 0..nsrc-1 gives a zero row.  src and dst 16-byte aligned,
 * K > 0 a multiple of 8, R >= 0, R*K < 2^31.
 */
bi_status_t bi_gather_rows(const void *src, int nsrc, const int32_t *idx, int R, int K, void *dst,
                           void *stream);

/*
 * SwiGLU of an up projection h: fp32 [R, 2I] (gate columns 0..I-1, up
 * columns I..2I-1) into a: bf16 [R, I], a = bf16(silu(g) * u), silu(g) =
 * g / (1 + exp(-g)) in fp32, rounded to nearest even.  I > 0 a multiple of
 * 4, h 16-byte and a 8-byte aligned, R*2I < 2^31.
 */
bi_status_t bi_swiglu(const float *h, int R, int I, void *a, void *stream);

/*
 * Weighted combine: y[t] = sum_j weights[t][j] * o[row_of[t][j]], the k terms
 * taken in ascending expert id ids[t][j] (the slot breaks a tie), one fp32
 * multiply and one fp32 add each, in that order.  A row outside 0..R-1
 * contributes nothing.  o: fp32 [R, H]; y: fp32 [T, H] out; H > 0 a multiple
 * of 4; o and y 16-byte aligned; 1 <= k <= 64; R*H and T*H < 2^31.
 */
bi_status_t bi_moe_combine(const float *o, int R, const int32_t *ids, const float *weights,
                           const int32_t *row_of, int T, int k, int H, float *y, void *stream);

/*
 * The whole expert layer on one device.  W_router: bf16 [E, H]; W_up: bf16
 * [E, 2I, H] (gate rows 0..I-1 then up rows of each expert); W_down: bf16
 * [E, H, I]; all 16-byte aligned.  The router and the two expert
 * projections are bi_gemm handles with the pins of their shapes, so create
 * packs copies of all three weights (bi_gemm_create) and they may be freed
 * once it returns.  Create allocates the layer's workspace for up to max_tokens
 * tokens once; run allocates nothing.  Limits: E a multiple of 16 within
 * 16..1024; 1 <= k <= min(E, 64); H a multiple of 64; I a multiple of 64;
 * 1 <= max_tokens, max_tokens*k*max(H, 2I) < 2^31.
 */
bi_status_t bi_moe_create(int E, int k, int H, int I, const void *W_router, const void *W_up,
                          const void *W_down, int max_tokens, bi_moe_t *out);

/*
 * y: fp32 [T, H] = the layer applied to x: bf16 [T, H]; 0 <= T <= max_tokens
 * (T == 0 launches nothing).  A token's row of y is a function of its row of
 * x and the weights only: the steps above, bit for bit as the step functions
 * and bi_grouped_gemm_run compute them.  (The layer packs W_up with its gate
 * and up rows interleaved 16 at a time; when the rows average at least 16 per
 * expert, or no expert can have more than 16 rows (T <= 16: a token's k
 * experts are distinct), the up projection's epilogue applies SwiGLU in
 * registers and writes a directly; for T <= 8 one kernel does the top-k and
 * the grouping.  Each product element keeps its tree, SwiGLU its arithmetic
 * and the top-k and grouping their results, so none changes a bit.)  One
 * handle runs one call at a time: its
 * workspace is shared by the calls, so calls on one handle must not overlap.
 */
bi_status_t bi_moe_run(bi_moe_t h, const void *x, int T, float *y, void *stream);

/* Release a layer (NULL is ignored). */
void bi_moe_destroy(bi_moe_t h);

#ifdef __cplusplus
}
#endif

#endif /* BI_MOE_H */
