/*
 * bi_attn.h -- C ABI of batch-invariant decode attention for MI355X (gfx950):
 * one new query token per sequence against that sequence's KV cache, with
 * grouped-query heads.
 *
 * Split-KV kernels partition a sequence's keys across blocks when the batch
 * offers too little parallelism, and pick the number of partitions from the
 * batch, so a request's reduction tree follows its co-runners (CoRun, §III-A;
 * LLM-42 notes, §4.4, which set the number of KV splits to one while
 * verifying).  The fixed split-size principle keeps split-KV but makes the
 * split boundaries a function of the sequence alone: every split holds S keys
 * (the last one the remainder), S pinned per deployment like a GEMM pin
 * (Detent, §8.1 Kernels: a rebuilt FA3 that keeps split-KV this way, its
 * split stride picked by the tuner).  CoRun instead turns split-KV off for
 * decode, at a cost of 15-41% when prompt lengths vary (CoRun, §V-F Fig. 13).
 *
 * The tree of one output, for sequence b (n keys) and query head h (kv head
 * h / (Hq / Hkv)), D = 128; scores are kept in log2 units (scale * log2(e),
 * rounded to fp32 once) and exponentials are exp2 (v_exp_f32):
 *   split j holds keys jS .. min(jS + S, n) - 1; inside it 16 groups of 16
 *   lanes, group g taking keys g, g+16, ... in ascending order, U at a time
 *   (U = 8, or 4 when Hq / Hkv = 8), and lane r dimensions 8r .. 8r+7;
 *   score: the lane's 8 dimensions as 4 bf16 pairs in order, each pair's two
 *   products added to the running fp32 sum by one v_dot2_f32_bf16, then a
 *   butterfly over the 16 lanes (distances 8, 4, 2, 1), times the scale;
 *   per group and head, a running max m, sum l and weighted sum o: for each
 *   U keys, m' = max(m, their scores), l and o multiplied by exp2(m - m'),
 *   then for each key in order p = exp2(s - m'), l += p and o += p v (one
 *   fused multiply-add per dimension);
 *   the split: M = the largest group max (exact), each group's l and o times
 *   exp2(m_g - M); the four groups of a wave (groups 4w .. 4w+3) added in
 *   order, then the four waves in order, giving (M, l_j, o_j);
 *   combine: M* = max_j M_j, w_j = exp2(M_j - M*), O = sum_j w_j o_j and
 *   L = sum_j w_j l_j in ascending j, out = O / L.
 * All fp32 round-to-nearest-even; multiplies and adds separate except the
 * fused multiply-adds and dot instructions named.  The tree depends on
 * (n, S, D, Hq/Hkv) only: a request's output is a function of its own
 * query, keys and values, whatever the batch holds.
 *
 * Conventions (as bi_gemm.h): device pointers, `stream` a hipStream_t
 * (NULL: the null stream), every argument checked on the host before any
 * HIP call, a failure launches nothing, detail in bi_last_error().
 */
#ifndef BI_ATTN_H
#define BI_ATTN_H

#include "bi_gemm.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct bi_attn *bi_attn_t;

/*
 * A decode-attention handle: Hq query heads, Hkv kv heads (Hq a multiple of
 * Hkv, Hq / Hkv in {1, 2, 4, 8}), head dimension D (128), split size S (a
 * multiple of 64 within 64 .. 16384: the pinned split stride), and the
 * largest batch and sequence length it serves (they size its workspace:
 * max_batch * Hq * ceil(max_seq_len / S) * (D + 2) floats of split partials
 * and a work list of max_batch + 2 ints, allocated here once).  1 <= max_batch, 1 <= max_seq_len <= 2^24,
 * and S * Hkv * D * 2 < 2^32 (one split of a kv head is addressed with 32-bit byte offsets; a split's
 * reads end at its last key, so keys past it read as zero and never outside the caches).
 * BI_ERR_INVALID_ARGUMENT otherwise.
 */
bi_status_t bi_attn_create(int Hq, int Hkv, int D, int split, int max_batch, int max_seq_len,
                           bi_attn_t *out);

/*
 * out[b][h] = attention of q[b][h] over keys/values seq_start[b] ..
 * seq_start[b+1]-1 of the cache, for b < B.  q: bf16 [B, Hq, D]; k, v: bf16
 * [Ntok, Hkv, D] (token-major, sequences' tokens contiguous); seq_start:
 * int32 [B+1] on the device, read only by the kernels, which clamp it to
 * 0 .. Ntok and a sequence's length to max_seq_len (a longer sequence is cut
 * there); out: fp32 [B, Hq, D].  A sequence with no keys gives zeros.
 * scale: the score scale (1/sqrt(D) for standard attention), finite.
 * 0 <= B <= max_batch (B == 0 launches nothing); Ntok >= 0; q, k, v and out
 * 16-byte aligned.  One handle runs one call at a time (shared workspace).
 */
bi_status_t bi_attn_decode(bi_attn_t h, const void *q, const void *k, const void *v,
                           const int32_t *seq_start, int B, int Ntok, float scale, float *out,
                           void *stream);

/* Release a handle (NULL is ignored). */
void bi_attn_destroy(bi_attn_t h);

/*
 * Largest split workspace bi_attn_decode_noalloc serves: 64 MiB, enough for
 * 256 sequences of up to 4096 keys with 32 query heads and split size 512.
 */
#define BI_ATTN_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * bi_attn_decode without a handle and without any allocation, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  The split partials and
 * the work list go to a static device array of BI_ATTN_NOALLOC_SCRATCH_BYTES
 * per GPU instead of a handle's workspace; everything else -- the kernels,
 * the tree, the output bits -- is exactly bi_attn_create(Hq, Hkv, D, split,
 * B, max_seq_len) followed by bi_attn_decode.  The argument rules are those
 * two calls' combined; in addition the partials must fit:
 * B * Hq * ceil(max_seq_len / split) * (D + 2) * 4 + (B + 2) * 4 <=
 * BI_ATTN_NOALLOC_SCRATCH_BYTES, else BI_ERR_INVALID_ARGUMENT (before any HIP
 * call).  The array of a GPU is looked up once (hipGetSymbolAddress) on the
 * first call on that device and is shared by every call on it: calls that
 * overlap on one GPU (on different streams, or from several threads) race
 * and must not be made.  Nothing in it needs to start at zero: each call
 * writes every partial and plan entry it reads.
 */
bi_status_t bi_attn_decode_noalloc(int Hq, int Hkv, int D, int split, int max_seq_len, const void *q,
                                   const void *k, const void *v, const int32_t *seq_start, int B, int Ntok,
                                   float scale, float *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* BI_ATTN_H */
