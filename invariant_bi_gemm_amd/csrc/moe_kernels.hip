// gfx950 kernels of the MoE layer around the grouped GEMM: routing, grouping
// of the rows by expert, row gather, SwiGLU and the weighted combine.
//
// The fused MoE is one of the kernel families whose selection reads the batch
// (Detent, §2 Obs. 1 and Fig. 3a: the tuned configuration row nearest the
// batch's token count).  Every kernel here computes a token's values from
// that token's inputs alone, in an order fixed by the code, so a token's bits
// do not depend on the tokens beside it.  The two expert projections are the
// grouped GEMM of the library, which has the same property.
//
// All are memory-bound elementwise or gather work: coalesced 16-byte
// accesses where rows allow, no MFMA.

#include <math.h>

#include "bf16_round.h"
#include "moe_internal.h"

namespace bimoe {
namespace {

// ---------------------------------------------------------------------------
// Top-k routing: one wave per token, lane l holding logits l, l+64, ....
// Logits (a NaN taken as -inf) become order-preserving 32-bit keys (-0 as
// +0, so equal floats give equal keys).  A radix select over the key bits,
// from the top, finds tau, the k-th largest key, with one ballot per logit
// slot per bit.  The chosen experts are those with a key above tau and,
// among those with key tau, the ones with the lowest ids (an equal logit
// goes to the lower expert id).  Each chosen expert's rank (larger logit
// first, then lower id) is counted against the other chosen ones, and lane
// j collects the expert of rank j.  The weights are the softmax over the k
// chosen logits, exp(l_j - l_0) summed in rank order, divided.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t order_key(float v)
{
    uint32_t u = __float_as_uint(v);
    if ((u << 1) == 0)
        u = 0;  // -0 equals +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Token t's top-k (one wave): lane j < k ends with the expert of rank j in
// *e_out and its weight in *w_out.  Shared by moe_topk and moe_route, so both
// give the same bits.
template <int PL>  // logits per lane: E <= 64 * PL
__device__ __forceinline__ void topk_token(const float* __restrict__ logits, int t, int E, int k, int lane,
                                           int* e_out, float* w_out)
{
    float v[PL];
    uint32_t key[PL];  // 0 for slots past E: below every real key
#pragma unroll
    for (int q = 0; q < PL; ++q) {
        const int e = lane + 64 * q;
        const float x = e < E ? logits[(size_t)t * E + e] : 0.f;
        v[q] = x == x ? x : -INFINITY;
        key[q] = e < E ? order_key(v[q]) : 0u;
    }
    // tau: the largest x with #(key >= x) >= k, built bit by bit
    uint32_t tau = 0;
    for (int b = 31; b >= 0; --b) {
        const uint32_t cand = tau | (1u << b);
        int c = 0;
#pragma unroll
        for (int q = 0; q < PL; ++q)
            c += __popcll(__ballot(key[q] >= cand));
        if (c >= k)
            tau = cand;
    }
    const unsigned long long lt = (1ull << lane) - 1ull;
    int greater = 0;
#pragma unroll
    for (int q = 0; q < PL; ++q)
        greater += __popcll(__ballot(key[q] > tau));
    // among keys equal to tau, the lowest ids: rank by id (q, then lane)
    bool chosen[PL];
    int eq_before = 0;
#pragma unroll
    for (int q = 0; q < PL; ++q) {
        const unsigned long long eq = __ballot(key[q] == tau);
        const int r = eq_before + __popcll(eq & lt);
        chosen[q] = key[q] > tau || (key[q] == tau && r < k - greater);
        eq_before += __popcll(eq);
    }
    // rank of each chosen expert among the chosen: larger key first, then lower id
    int rank[PL];
#pragma unroll
    for (int q = 0; q < PL; ++q)
        rank[q] = 0;
#pragma unroll
    for (int qc = 0; qc < PL; ++qc) {
        unsigned long long m = __ballot(chosen[qc]);
        while (m) {
            const int lc = __builtin_ctzll(m);
            m &= m - 1;
            const uint32_t kc = (uint32_t)__builtin_amdgcn_readlane((int)key[qc], lc);
            const int ec = lc + 64 * qc;
#pragma unroll
            for (int q = 0; q < PL; ++q) {
                const int e = lane + 64 * q;
                rank[q] += (kc > key[q] || (kc == key[q] && ec < e)) ? 1 : 0;
            }
        }
    }
    // lane j takes the expert of rank j
    int my_e = 0;
    float my_v = 0.f;
#pragma unroll
    for (int qc = 0; qc < PL; ++qc) {
        unsigned long long m = __ballot(chosen[qc]);
        while (m) {
            const int lc = __builtin_ctzll(m);
            m &= m - 1;
            const int rc = __builtin_amdgcn_readlane(rank[qc], lc);
            const float vc = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v[qc]), lc));
            if (lane == rc) {
                my_e = lc + 64 * qc;
                my_v = vc;
            }
        }
    }
    const float top = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_v), 0));
    const float z = lane < k ? expf(my_v - top) : 0.f;
    float s = 0.f;
    for (int j = 0; j < k; ++j)
        s = s + __int_as_float(__builtin_amdgcn_readlane(__float_as_int(z), j));
    *e_out = my_e;
    *w_out = z / s;
}

template <int PL>  // logits per lane: E <= 64 * PL
__global__ void __launch_bounds__(256)
    moe_topk(const float* __restrict__ logits, int T, int E, int k, int32_t* __restrict__ ids,
             float* __restrict__ w)
{
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (int)(threadIdx.x >> 6);
    if (t >= T)
        return;  // whole waves only: t is the same for all 64 lanes
    int e;
    float ww;
    topk_token<PL>(logits, t, E, k, lane, &e, &ww);
    if (lane < k) {
        ids[(size_t)t * k + lane] = e;
        w[(size_t)t * k + lane] = ww;
    }
}

// ---------------------------------------------------------------------------
// Grouping by expert.  The flat pair index i = t*k + j is already the stable
// order, so expert e's rows are its pairs in ascending i.  Block (e, c) owns
// the pairs of chunk c (lo <= i < hi): one counting pass over all pairs gives
// the number with an id below e (the expert's first row) and the number
// equal to e before lo (the chunk's first row within the expert); a second
// pass walks the chunk 1024 pairs at a time, four consecutive pairs per
// thread, and ranks the matches with wave ballots and one barrier.  Integer
// counts only: the rows do not depend on the order the hardware runs in.
// Pairs whose id is outside 0..E-1 get row -1 (written by the e = 0 blocks
// of their chunk) and no row.
// ---------------------------------------------------------------------------
constexpr int kPermThreads = 256;
constexpr int kPermWaves = kPermThreads / 64;

__device__ __forceinline__ int wave_sum(int v)
{
#pragma unroll
    for (int d = 32; d > 0; d >>= 1)
        v += __shfl_xor(v, d, 64);
    return v;
}

__global__ void __launch_bounds__(kPermThreads)
    moe_permute(const int32_t* __restrict__ ids, int T, int E, int k, int chunk,
                int32_t* __restrict__ offsets, int32_t* __restrict__ tok, int32_t* __restrict__ row_of)
{
    __shared__ int s_red[3][kPermWaves];
    __shared__ int s_tot[2][kPermWaves];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int e = blockIdx.x;
    const int n = T * k;
    const int lo = min(n, blockIdx.y * chunk), hi = min(n, lo + chunk);

    // pass 1: counts (every pair for "below e" and "equal to e", the pairs
    // before lo for "equal to e before the chunk")
    int below = 0, equal = 0, before = 0;
    auto count = [&](int x, int i) {
        below += (x >= 0 && x < e);
        equal += (x == e);
        before += (x == e && i < lo);
    };
    // four ids per load when ids is 16-byte aligned, then the tail
    const int n4 = (reinterpret_cast<uintptr_t>(ids) & 15u) == 0 ? n / 4 : 0;
#pragma unroll 4
    for (int i4 = tid; i4 < n4; i4 += kPermThreads) {
        const int4 x = reinterpret_cast<const int4*>(ids)[i4];
        count(x.x, 4 * i4);
        count(x.y, 4 * i4 + 1);
        count(x.z, 4 * i4 + 2);
        count(x.w, 4 * i4 + 3);
    }
    for (int i = 4 * n4 + tid; i < n; i += kPermThreads)
        count(ids[i], i);
    below = wave_sum(below);
    equal = wave_sum(equal);
    before = wave_sum(before);
    if (lane == 0) {
        s_red[0][wave] = below;
        s_red[1][wave] = equal;
        s_red[2][wave] = before;
    }
    __syncthreads();
    below = equal = before = 0;
#pragma unroll
    for (int w = 0; w < kPermWaves; ++w) {
        below += s_red[0][w];
        equal += s_red[1][w];
        before += s_red[2][w];
    }
    if (blockIdx.y == 0 && tid == 0) {
        offsets[e + 1] = below + equal;
        if (e == 0)
            offsets[0] = 0;
    }

    // pass 2: place the chunk's pairs of expert e in ascending i
    const unsigned long long lt = (1ull << lane) - 1ull;
    int run = below + before;
    int it = 0;
    for (int base = lo; base < hi; base += 4 * kPermThreads, ++it) {
        const int i0 = base + 4 * tid;
        int v[4];
        int cnt = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            v[q] = (i0 + q < hi) ? ids[i0 + q] : -1;
            cnt += v[q] == e;
            if (e == 0 && i0 + q < hi && (v[q] < 0 || v[q] >= E))
                row_of[i0 + q] = -1;
        }
        // exclusive prefix of cnt (0..4) over the wave, from its three bits
        const unsigned long long b0 = __ballot(cnt & 1), b1 = __ballot(cnt & 2), b2 = __ballot(cnt & 4);
        const int pre = __popcll(b0 & lt) + 2 * __popcll(b1 & lt) + 4 * __popcll(b2 & lt);
        if (lane == 0)
            s_tot[it & 1][wave] = __popcll(b0) + 2 * __popcll(b1) + 4 * __popcll(b2);
        __syncthreads();
        int wbase = 0, total = 0;
#pragma unroll
        for (int w = 0; w < kPermWaves; ++w) {
            const int c = s_tot[it & 1][w];
            wbase += w < wave ? c : 0;
            total += c;
        }
        int r = run + wbase + pre;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (v[q] == e) {
                tok[r] = (i0 + q) / k;
                row_of[i0 + q] = r;
                ++r;
            }
        run += total;
    }
}

// ---------------------------------------------------------------------------
// Routing and grouping of a small batch in one launch (T <= kRouteMaxTokens,
// one wave per token): each wave runs topk_token -- the code of moe_topk, so
// the same ids and weights bit for bit -- and keeps the token's ids in LDS;
// then the grouping of moe_permute over those T*k pairs: expert e's first row
// is the number of pairs with a valid id below e, and a pair's row within its
// expert the number of earlier pairs (in t*k + j order) with the same id.
// Integer counts only, so offsets, rows and row_of are moe_permute's.
// ---------------------------------------------------------------------------
constexpr int kRouteThreads = 64 * kRouteMaxTokens;

template <int PL>
__global__ void __launch_bounds__(kRouteThreads)
    moe_route(const float* __restrict__ logits, int T, int E, int k, int32_t* __restrict__ ids,
              float* __restrict__ w, int32_t* __restrict__ offsets, int32_t* __restrict__ tok,
              int32_t* __restrict__ row_of)
{
    __shared__ int s_id[kRouteMaxTokens * kMaxTopK];
    __shared__ int s_first[kMaxExperts + 1];
    const int tid = threadIdx.x, lane = tid & 63;
    const int t = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = T * k;
    if (t < T) {
        int e;
        float ww;
        topk_token<PL>(logits, t, E, k, lane, &e, &ww);
        if (lane < k) {
            ids[(size_t)t * k + lane] = e;
            w[(size_t)t * k + lane] = ww;
            s_id[t * k + lane] = e;
        }
    }
    __syncthreads();
    for (int e = tid; e <= E; e += kRouteThreads) {
        int c = 0;
        for (int i = 0; i < n; ++i) {
            const int x = s_id[i];
            c += x >= 0 && x < e;
        }
        s_first[e] = c;
        offsets[e] = c;
    }
    __syncthreads();
    for (int i = tid; i < n; i += kRouteThreads) {
        const int x = s_id[i];
        if (x < 0 || x >= E) {
            row_of[i] = -1;
            continue;
        }
        int r = s_first[x];
        for (int j = 0; j < i; ++j)
            r += s_id[j] == x;
        tok[r] = i / k;
        row_of[i] = r;
    }
}

// ---------------------------------------------------------------------------
// Row gather: dst[r] = src[idx[r]] (rows of `row16` 16-byte units); an index
// outside 0..nsrc-1 gives a zero row.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
    gather_rows(const uint4* __restrict__ src, int nsrc, const int32_t* __restrict__ idx, int R,
                int row16, uint4* __restrict__ dst)
{
    const long long total = (long long)R * row16;
    for (long long i = blockIdx.x * 256LL + threadIdx.x; i < total; i += (long long)gridDim.x * 256) {
        const int r = (int)(i / row16);
        const int c = (int)(i % row16);
        const int s = idx[r];
        dst[i] = (s >= 0 && s < nsrc) ? src[(size_t)s * row16 + c] : uint4{0u, 0u, 0u, 0u};
    }
}

// ---------------------------------------------------------------------------
// SwiGLU: a[r][i] = bf16(g / (1 + exp(-g)) * u) (bi::swiglu_bf16), four
// columns per thread (I a multiple of 4; of 16 interleaved).  Plain layout: g = h[r][i],
// u = h[r][I+i].  Interleaved layout (the MoE layer's up projection, whose
// weight rows are packed 16 gate rows then the 16 matching up rows): g =
// h[r][32(i/16) + i%16], u 16 columns after it.
// ---------------------------------------------------------------------------
// A 16-byte load with the non-temporal hint, for rows a kernel reads once
// (the up projection's fp32 product in SwiGLU, the expert outputs in the
// combine): streaming them then does not evict what stays in use.  Measured
// on the layer at T = 4096: the combine 55.0 -> 48.8 us, interleaved on one
// box.
__device__ __forceinline__ float4 ld_once(const float4* p)
{
    typedef float f4v __attribute__((ext_vector_type(4)));
    const f4v v = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(p));
    return float4{v[0], v[1], v[2], v[3]};
}

template <bool kInterleaved>
__global__ void __launch_bounds__(256)
    swiglu(const float* __restrict__ h, int R, int I, uint16_t* __restrict__ a)
{
    const int q4 = I / 4;
    const long long total = (long long)R * q4;
    for (long long i = blockIdx.x * 256LL + threadIdx.x; i < total; i += (long long)gridDim.x * 256) {
        const int r = (int)(i / q4);
        const int c = (int)(i % q4) * 4;
        const int cg = kInterleaved ? 32 * (c / 16) + c % 16 : c;
        const int cu = kInterleaved ? cg + 16 : I + c;
        const float4 g = ld_once(reinterpret_cast<const float4*>(h + (size_t)r * 2 * I + cg));
        const float4 u = ld_once(reinterpret_cast<const float4*>(h + (size_t)r * 2 * I + cu));
        const float gg[4] = {g.x, g.y, g.z, g.w};
        const float uu[4] = {u.x, u.y, u.z, u.w};
        *reinterpret_cast<uint2*>(a + (size_t)r * I + c) = bi::swiglu4(gg, uu);
    }
}

// ---------------------------------------------------------------------------
// Weighted combine: block t computes y[t] = sum_j w[t][j] * o[row_of[t][j]]
// over the token's k slots taken in ascending expert id (a slot's position
// breaks a tie), one fp32 multiply and one fp32 add per slot, in that order.
// Lanes j < k of the first wave load slot j together and rank it by (id,
// slot) against the others; the sorted slots go to LDS.  A row outside
// 0..R-1 contributes nothing.  Each thread owns four columns in each half of
// every 2048-column span.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
    moe_combine(const float* __restrict__ o, int R, const int32_t* __restrict__ ids,
                const float* __restrict__ w, const int32_t* __restrict__ row_of, int k, int H,
                float* __restrict__ y)
{
    __shared__ int s_row[kMaxTopK];
    __shared__ float s_w[kMaxTopK];
    const int t = blockIdx.x;
    if (threadIdx.x < 64) {
        const int j = threadIdx.x;
        int e = 0x7fffffff, r = -1;
        float ww = 0.f;
        if (j < k) {
            e = ids[(size_t)t * k + j];
            r = row_of[(size_t)t * k + j];
            ww = w[(size_t)t * k + j];
        }
        int rank = 0;
        for (int i = 0; i < k; ++i) {
            const int ei = __builtin_amdgcn_readlane(e, i);
            rank += (ei < e || (ei == e && i < j)) ? 1 : 0;
        }
        if (j < k) {
            s_row[rank] = r;
            s_w[rank] = ww;
        }
    }
    __syncthreads();
    // Each thread owns columns c and c + 1024 of every 2048-column span; the
    // eight slots' rows of both are loaded before any of them is added.
    for (int c = threadIdx.x * 4; c < H; c += 2 * 256 * 4) {
        const bool hi = c + 256 * 4 < H;
        float4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
        for (int j0 = 0; j0 < k; j0 += 8) {
            float4 v0[8], v1[8];
            bool ok[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int r = j0 + u < k ? s_row[j0 + u] : -1;
                ok[u] = r >= 0 && r < R;
                const float* row = o + (size_t)(ok[u] ? r : 0) * H + c;
                v0[u] = ok[u] ? ld_once(reinterpret_cast<const float4*>(row)) : float4{0.f, 0.f, 0.f, 0.f};
                v1[u] = ok[u] && hi ? ld_once(reinterpret_cast<const float4*>(row + 256 * 4)) : float4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (ok[u]) {
                    const float ww = s_w[j0 + u];
                    acc0.x = acc0.x + ww * v0[u].x;
                    acc0.y = acc0.y + ww * v0[u].y;
                    acc0.z = acc0.z + ww * v0[u].z;
                    acc0.w = acc0.w + ww * v0[u].w;
                    acc1.x = acc1.x + ww * v1[u].x;
                    acc1.y = acc1.y + ww * v1[u].y;
                    acc1.z = acc1.z + ww * v1[u].z;
                    acc1.w = acc1.w + ww * v1[u].w;
                }
        }
        *reinterpret_cast<float4*>(y + (size_t)t * H + c) = acc0;
        if (hi)
            *reinterpret_cast<float4*>(y + (size_t)t * H + c + 256 * 4) = acc1;
    }
}

int grid_for(long long work, int per_block)
{
    long long g = (work + per_block - 1) / per_block;
    const long long cap = 256LL * 64;
    return (int)(g < 1 ? 1 : (g > cap ? cap : g));
}

}  // namespace

hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                       hipStream_t stream)
{
    const dim3 grid((T + 3) / 4), block(256);
    if (E <= 64)
        hipLaunchKernelGGL(moe_topk<1>, grid, block, 0, stream, logits, T, E, k, ids, w);
    else if (E <= 128)
        hipLaunchKernelGGL(moe_topk<2>, grid, block, 0, stream, logits, T, E, k, ids, w);
    else if (E <= 256)
        hipLaunchKernelGGL(moe_topk<4>, grid, block, 0, stream, logits, T, E, k, ids, w);
    else if (E <= 512)
        hipLaunchKernelGGL(moe_topk<8>, grid, block, 0, stream, logits, T, E, k, ids, w);
    else
        hipLaunchKernelGGL(moe_topk<16>, grid, block, 0, stream, logits, T, E, k, ids, w);
    return hipGetLastError();
}

hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* w, int32_t* offsets,
                        int32_t* tok, int32_t* row_of, hipStream_t stream)
{
    if (T < 1 || T > kRouteMaxTokens)
        return hipErrorInvalidValue;
    const dim3 grid(1), block(kRouteThreads);
    if (E <= 64)
        hipLaunchKernelGGL(moe_route<1>, grid, block, 0, stream, logits, T, E, k, ids, w, offsets, tok, row_of);
    else if (E <= 128)
        hipLaunchKernelGGL(moe_route<2>, grid, block, 0, stream, logits, T, E, k, ids, w, offsets, tok, row_of);
    else if (E <= 256)
        hipLaunchKernelGGL(moe_route<4>, grid, block, 0, stream, logits, T, E, k, ids, w, offsets, tok, row_of);
    else if (E <= 512)
        hipLaunchKernelGGL(moe_route<8>, grid, block, 0, stream, logits, T, E, k, ids, w, offsets, tok, row_of);
    else
        hipLaunchKernelGGL(moe_route<16>, grid, block, 0, stream, logits, T, E, k, ids, w, offsets, tok, row_of);
    return hipGetLastError();
}

hipError_t launch_permute(const int32_t* ids, int T, int E, int k, int32_t* offsets, int32_t* tok,
                          int32_t* row_of, hipStream_t stream)
{
    // chunks of 8192 pairs, at most 8 per expert: every block reads all the
    // ids once (E * chunks * T*k reads, served from L2), and places its chunk
    const long long n = (long long)T * k;
    const int per = 4 * kPermThreads;
    long long chunk = 8192;
    if (n > 8 * chunk)
        chunk = (n + 7) / 8;
    chunk = (chunk + per - 1) / per * per;
    const int chunks = n == 0 ? 1 : (int)((n + chunk - 1) / chunk);
    hipLaunchKernelGGL(moe_permute, dim3(E, chunks), dim3(kPermThreads), 0, stream, ids, T, E, k,
                       (int)chunk, offsets, tok, row_of);
    return hipGetLastError();
}

hipError_t launch_gather(const void* src, int nsrc, const int32_t* idx, int R, int K, void* dst,
                         hipStream_t stream)
{
    const int row16 = K * 2 / 16;
    hipLaunchKernelGGL(gather_rows, dim3(grid_for((long long)R * row16, 256)), dim3(256), 0, stream,
                       static_cast<const uint4*>(src), nsrc, idx, R, row16, static_cast<uint4*>(dst));
    return hipGetLastError();
}

hipError_t launch_swiglu(const float* h, int R, int I, void* a, hipStream_t stream, bool interleaved)
{
    const dim3 grid(grid_for((long long)R * (I / 4), 256));
    if (interleaved)
        hipLaunchKernelGGL(swiglu<true>, grid, dim3(256), 0, stream, h, R, I, static_cast<uint16_t*>(a));
    else
        hipLaunchKernelGGL(swiglu<false>, grid, dim3(256), 0, stream, h, R, I, static_cast<uint16_t*>(a));
    return hipGetLastError();
}

hipError_t launch_combine(const float* o, int R, const int32_t* ids, const float* w,
                          const int32_t* row_of, int T, int k, int H, float* y, hipStream_t stream)
{
    hipLaunchKernelGGL(moe_combine, dim3(T), dim3(256), 0, stream, o, R, ids, w, row_of, k, H, y);
    return hipGetLastError();
}

}  // namespace bimoe
